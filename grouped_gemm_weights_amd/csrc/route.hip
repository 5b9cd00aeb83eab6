// moe_route: top-k expert selection and routing weights, one wave64 per token.
//
// Each lane holds E/64 logits in registers (element i of lane l is expert
// i*64 + l, so the row is read with coalesced 256-byte loads).  The k experts
// are chosen by k rounds of a wave-wide arg-max under the total order
// (logit descending, expert id ascending); comparisons are exact fp32, so the
// selection is deterministic and +0 / -0 tie.  Lane j keeps the j-th choice and
// the weights exp(l_j - l_0) / sum_i exp(l_i - l_0) are formed in fp32.
#include "common.h"

namespace moe {
namespace {

constexpr int kRouteWaves = 4;  // tokens per 256-thread block

__device__ __forceinline__ bool route_better(float a, int ai, float b, int bi) {
  // true when candidate (a, ai) precedes (b, bi); bi == INT_MAX marks "none"
  if (ai == INT_MAX) return false;
  if (bi == INT_MAX) return true;
  return a > b || (a == b && ai < bi);
}

template <int EPL>
__global__ __launch_bounds__(kRouteWaves * kWave) void route_kernel(
    const float* __restrict__ logits, int T, int E, int k, int32_t* __restrict__ topk_idx,
    float* __restrict__ topk_w, int32_t* status) {
  const int lane = threadIdx.x & (kWave - 1);
  const int t = blockIdx.x * kRouteWaves + (threadIdx.x / kWave);
  if (t >= T) return;
  const float* row = logits + static_cast<int64_t>(t) * E;

  float v[EPL];
  uint32_t avail = 0;  // bit i: element i is a real expert not chosen yet
  bool bad = false;
#pragma unroll
  for (int i = 0; i < EPL; ++i) {
    const int e = i * kWave + lane;
    v[i] = 0.f;
    if (e < E) {
      v[i] = row[e];
      avail |= 1u << i;
      bad |= !__builtin_isfinite(v[i]);
    }
  }
  if (__any(bad) && lane == 0) status_or(status, MOE_STATUS_NONFINITE_LOGIT);

  float my_logit = 0.f;
  int my_id = 0;
  for (int j = 0; j < k; ++j) {
    float bv = 0.f;
    int bi = INT_MAX;
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
      // ascending i means ascending id, so strict '>' keeps the smaller id on ties
      if (((avail >> i) & 1u) && (bi == INT_MAX || v[i] > bv)) {
        bv = v[i];
        bi = i * kWave + lane;
      }
    }
#pragma unroll
    for (int off = kWave / 2; off >= 1; off >>= 1) {
      const float ov = __shfl_xor(bv, off);
      const int oi = __shfl_xor(bi, off);
      if (route_better(ov, oi, bv, bi)) {
        bv = ov;
        bi = oi;
      }
    }
    if (bi != INT_MAX && lane == (bi & (kWave - 1))) avail &= ~(1u << (bi / kWave));
    if (lane == j) {
      my_logit = bv;
      my_id = bi;
    }
  }

  const float l0 = __shfl(my_logit, 0);
  float ex = lane < k ? expf(my_logit - l0) : 0.f;
  float sum = ex;
#pragma unroll
  for (int off = kWave / 2; off >= 1; off >>= 1) sum += __shfl_xor(sum, off);
  if (lane < k) {
    topk_idx[static_cast<int64_t>(t) * k + lane] = my_id;
    topk_w[static_cast<int64_t>(t) * k + lane] = ex / sum;
  }
}

template <int EPL>
void launch_route(const float* logits, int T, int E, int k, int32_t* idx, float* w,
                  int32_t* status, hipStream_t s) {
  const int blocks = ceil_div(T, kRouteWaves);
  hipLaunchKernelGGL(route_kernel<EPL>, dim3(blocks), dim3(kRouteWaves * kWave), 0, s, logits,
                     T, E, k, idx, w, status);
}

}  // namespace
}  // namespace moe

extern "C" int moe_route(const float* logits, int T, int E, int k, int32_t* topk_idx,
                         float* topk_w, int32_t* status, moe_stream_t stream) {
  using namespace moe;
  if (T < 0 || E < 1 || k < 1 || k > E)
    return fail(MOE_ERR_ARG, "moe_route: bad sizes T=%d E=%d k=%d", T, E, k);
  if (E > MOE_MAX_E || k > MOE_MAX_K)
    return fail(MOE_ERR_UNSUPPORTED, "moe_route: E=%d or k=%d above the limits", E, k);
  if (T == 0) return MOE_OK;
  if (!logits || !topk_idx || !topk_w) return fail(MOE_ERR_ARG, "moe_route: null pointer");
  hipStream_t s = as_stream(stream);
  if (E <= 64) launch_route<1>(logits, T, E, k, topk_idx, topk_w, status, s);
  else if (E <= 128) launch_route<2>(logits, T, E, k, topk_idx, topk_w, status, s);
  else if (E <= 256) launch_route<4>(logits, T, E, k, topk_idx, topk_w, status, s);
  else if (E <= 512) launch_route<8>(logits, T, E, k, topk_idx, topk_w, status, s);
  else launch_route<16>(logits, T, E, k, topk_idx, topk_w, status, s);
  MOE_LAUNCH_CHECK("moe_route: launch");
  return debug_check(MOE_OK, "moe_route", s, status);
}
