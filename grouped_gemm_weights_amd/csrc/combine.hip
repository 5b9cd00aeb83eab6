// moe_combine: weighted un-permute of the expert outputs, and the residual
// add used between pipeline layers.
//
// One 256-thread block per token: the k routing weights and row indices are
// read once, then each thread sweeps float4 columns of the k expert rows
// (k independent 16-byte loads in flight per step) and accumulates in j order
// with fused multiply-adds.  Every y_perm row is read exactly once, so its loads
// are non-temporal (9 % faster on prefill-sized layers than cached loads).
#include "common.h"

namespace moe {
namespace {

typedef float f32x4_t __attribute__((ext_vector_type(4)));

template <bool VEC>
__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ y_perm,
                                                      const int32_t* __restrict__ row_of,
                                                      const float* __restrict__ topk_w, int T,
                                                      int k, int H, float* __restrict__ y) {
  __shared__ int32_t rows[MOE_MAX_K];
  __shared__ float ws[MOE_MAX_K];
  const int t = blockIdx.x;
  if (threadIdx.x < k) {
    const int32_t r = row_of[static_cast<int64_t>(t) * k + threadIdx.x];
    // an unwritten row index (after an out-of-range expert id) must not fault
    const bool ok = r >= 0 && static_cast<int64_t>(r) < static_cast<int64_t>(T) * k;
    rows[threadIdx.x] = ok ? r : 0;
    ws[threadIdx.x] = ok ? topk_w[static_cast<int64_t>(t) * k + threadIdx.x] : 0.f;
  }
  __syncthreads();
  float* out = y + static_cast<int64_t>(t) * H;
  if (VEC) {
    const int H4 = H / 4;
    for (int c = threadIdx.x; c < H4; c += blockDim.x) {
      float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
      for (int j = 0; j < k; ++j) {
        const f32x4_t v = __builtin_nontemporal_load(
            reinterpret_cast<const f32x4_t*>(y_perm + static_cast<int64_t>(rows[j]) * H) + c);
        const float wj = ws[j];
        acc.x = fmaf(wj, v.x, acc.x);
        acc.y = fmaf(wj, v.y, acc.y);
        acc.z = fmaf(wj, v.z, acc.z);
        acc.w = fmaf(wj, v.w, acc.w);
      }
      reinterpret_cast<float4*>(out)[c] = acc;
    }
  } else {
    for (int c = threadIdx.x; c < H; c += blockDim.x) {
      float acc = 0.f;
      for (int j = 0; j < k; ++j) acc = fmaf(ws[j], y_perm[static_cast<int64_t>(rows[j]) * H + c], acc);
      out[c] = acc;
    }
  }
}

// out may alias x (each element is read before it is written by the same thread)
__global__ __launch_bounds__(256) void residual_kernel(const uint16_t* x, const float* __restrict__ y,
                                                       int64_t n, uint16_t* out) {
  const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n; i += stride)
    out[i] = f32_to_bf16(bf16_to_f32(x[i]) + y[i]);
}

}  // namespace
}  // namespace moe

extern "C" int moe_combine(const float* y_perm, const int32_t* row_of, const float* topk_w, int T,
                           int k, int H, float* y, moe_stream_t stream) {
  using namespace moe;
  if (T < 0 || k < 1 || H < 1) return fail(MOE_ERR_ARG, "moe_combine: bad sizes T=%d k=%d H=%d", T, k, H);
  if (k > MOE_MAX_K) return fail(MOE_ERR_UNSUPPORTED, "moe_combine: k=%d above %d", k, MOE_MAX_K);
  if (T == 0) return MOE_OK;
  if (!y_perm || !row_of || !topk_w || !y) return fail(MOE_ERR_ARG, "moe_combine: null pointer");
  hipStream_t s = as_stream(stream);
  const bool vec = (H % 4 == 0) && ((reinterpret_cast<uintptr_t>(y_perm) | reinterpret_cast<uintptr_t>(y)) % 16 == 0);
  if (vec)
    hipLaunchKernelGGL(combine_kernel<true>, dim3(T), dim3(256), 0, s, y_perm, row_of, topk_w, T, k, H, y);
  else
    hipLaunchKernelGGL(combine_kernel<false>, dim3(T), dim3(256), 0, s, y_perm, row_of, topk_w, T, k, H, y);
  MOE_LAUNCH_CHECK("moe_combine: launch");
  return debug_check(MOE_OK, "moe_combine", s, nullptr);
}

extern "C" int moe_residual_add(const void* x, const float* y, int64_t n, void* out,
                                moe_stream_t stream) {
  using namespace moe;
  if (n < 0) return fail(MOE_ERR_ARG, "moe_residual_add: n < 0");
  if (n == 0) return MOE_OK;
  if (!x || !y || !out) return fail(MOE_ERR_ARG, "moe_residual_add: null pointer");
  const int64_t blocks64 = ceil_div64(n, 256);
  const int blocks = static_cast<int>(blocks64 < 65536 ? blocks64 : 65536);
  hipLaunchKernelGGL(residual_kernel, dim3(blocks), dim3(256), 0, as_stream(stream),
                     static_cast<const uint16_t*>(x), y, n, static_cast<uint16_t*>(out));
  MOE_LAUNCH_CHECK("moe_residual_add: launch");
  return debug_check(MOE_OK, "moe_residual_add", as_stream(stream), nullptr);
}
