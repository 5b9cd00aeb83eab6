// moe_permute: per-expert counts, offsets, the stable expert-major
// permutation and the row gather.
//
// The R = T*k assignments are cut into chunks (at most kMaxChunks of them).
//  1. hist:    one block per chunk builds an LDS histogram of its expert ids.
//  2. scan:    one block turns the chunk histograms into counts[e],
//              offsets[e] (exclusive scan over e) and chunk_base[c][e] =
//              offsets[e] + (rows of expert e in chunks before c), several
//              threads per expert so the chunk walk is not one long chain.
//  3. scatter: one wave per chunk walks its assignments in order, 64 at a
//              time; lanes holding the same expert find each other with one
//              ballot per id bit, so an assignment's rank among equal ids of
//              its batch is a popcount, and a per-expert LDS cursor carries
//              the running position across batches.  No atomics decide an
//              order, so the permutation is the stable counting sort.
//  4. gather:  x_perm[r] = x[src_of[r] / k] with 16-byte vector copies.
#include <mutex>

#include "common.h"

namespace moe {
namespace {

constexpr int kMaxChunks = 256;

struct Chunking {
  int chunk;     // assignments per chunk (multiple of 64)
  int n_chunks;  // <= kMaxChunks
};

Chunking chunking(int64_t R) {
  int64_t c = ceil_div64(R, kMaxChunks);
  c = ceil_div64(c, 64) * 64;
  if (c < 64) c = 64;
  Chunking ch;
  ch.chunk = static_cast<int>(c);
  ch.n_chunks = static_cast<int>(ceil_div64(R, c));
  return ch;
}

size_t permute_ws_bytes(int64_t R, int E) {
  const Chunking ch = chunking(R);
  // chunk_counts and chunk_base, each [n_chunks][E]
  return align_up(2 * static_cast<size_t>(ch.n_chunks) * E * sizeof(int32_t), 256);
}

__global__ __launch_bounds__(256) void hist_kernel(const int32_t* __restrict__ idx, int R, int E,
                                                   int chunk, int32_t* __restrict__ chunk_counts,
                                                   int32_t* status) {
  extern __shared__ int32_t hist[];
  for (int e = threadIdx.x; e < E; e += blockDim.x) hist[e] = 0;
  __syncthreads();
  const int a0 = blockIdx.x * chunk;
  const int a1 = min(R, a0 + chunk);
  bool bad = false;
  for (int a = a0 + threadIdx.x; a < a1; a += blockDim.x) {
    const int e = idx[a];
    if (e >= 0 && e < E) atomicAdd(&hist[e], 1);
    else bad = true;
  }
  if (bad) status_or(status, MOE_STATUS_BAD_EXPERT_ID);
  __syncthreads();
  int32_t* out = chunk_counts + static_cast<int64_t>(blockIdx.x) * E;
  for (int e = threadIdx.x; e < E; e += blockDim.x) out[e] = hist[e];
}

// One block of MOE_MAX_E threads.  Expert e is owned by P = parts_per_expert(E)
// threads (thread e * P + p), part p covering the chunk range
// [p * cp, min((p + 1) * cp, n_chunks)), cp = ceil(n_chunks / P).  Pass 1 sums
// each part's counts (loads batched so their latencies overlap), the parts are
// prefixed per expert and the expert totals scanned in LDS, and pass 2 writes
// chunk_base for each part from its starting value.
constexpr int kScanBatch = 16;

__host__ __device__ constexpr int parts_per_expert(int E) {
  int p = 1;
  while (p * 2 * E <= MOE_MAX_E && p < 64) p *= 2;
  return p;
}

__global__ __launch_bounds__(MOE_MAX_E) void scan_kernel(const int32_t* __restrict__ chunk_counts,
                                                         int n_chunks, int E,
                                                         int32_t* __restrict__ chunk_base,
                                                         int32_t* __restrict__ counts,
                                                         int32_t* __restrict__ offsets) {
  __shared__ int32_t part[MOE_MAX_E];   // part sums, then the part's starting value
  __shared__ int32_t s[MOE_MAX_E];      // expert totals, then their inclusive scan
  const int P = parts_per_expert(E);
  const int t = threadIdx.x;
  const int e = t / P, p = t % P;
  const bool owner = e < E;
  const int cp = (n_chunks + P - 1) / P;
  const int c0 = min(n_chunks, p * cp), c1 = min(n_chunks, c0 + cp);

  int32_t sum = 0;
  if (owner) {
    for (int c = c0; c < c1; c += kScanBatch) {
      int32_t v[kScanBatch];
#pragma unroll
      for (int j = 0; j < kScanBatch; ++j) {
        v[j] = 0;
        if (c + j < c1) v[j] = chunk_counts[static_cast<int64_t>(c + j) * E + e];
      }
#pragma unroll
      for (int j = 0; j < kScanBatch; ++j) sum += v[j];
    }
  }
  part[t] = sum;
  __syncthreads();
  // prefix of the parts of each expert (thread p == 0 of the expert), expert totals
  int32_t total = 0;
  if (owner && p == 0) {
    for (int q = 0; q < P; ++q) {
      const int32_t v = part[t + q];
      part[t + q] = total;
      total += v;
    }
  }
  __syncthreads();
  if (t < MOE_MAX_E) s[t] = 0;
  __syncthreads();
  if (owner && p == 0) {
    s[e] = total;
    counts[e] = total;
  }
  __syncthreads();
  // inclusive Hillis-Steele scan over the experts
  for (int off = 1; off < MOE_MAX_E; off <<= 1) {
    const int32_t add = t >= off ? s[t - off] : 0;
    __syncthreads();
    s[t] += add;
    __syncthreads();
  }
  if (t == 0) offsets[E] = s[E - 1];
  if (owner) {
    const int32_t excl = e > 0 ? s[e - 1] : 0;
    if (p == 0) offsets[e] = excl;
    int32_t run = excl + part[t];
    for (int c = c0; c < c1; c += kScanBatch) {
      int32_t v[kScanBatch];
#pragma unroll
      for (int j = 0; j < kScanBatch; ++j) {
        v[j] = 0;
        if (c + j < c1) v[j] = chunk_counts[static_cast<int64_t>(c + j) * E + e];
      }
#pragma unroll
      for (int j = 0; j < kScanBatch; ++j) {
        if (c + j < c1) chunk_base[static_cast<int64_t>(c + j) * E + e] = run;
        run += v[j];
      }
    }
  }
}

__global__ __launch_bounds__(kWave) void scatter_kernel(const int32_t* __restrict__ idx, int R,
                                                        int E, int chunk,
                                                        const int32_t* __restrict__ chunk_base,
                                                        int32_t* __restrict__ row_of,
                                                        int32_t* __restrict__ src_of) {
  extern __shared__ int32_t cursor[];
  const int lane = threadIdx.x;
  const int32_t* base = chunk_base + static_cast<int64_t>(blockIdx.x) * E;
  for (int e = lane; e < E; e += kWave) cursor[e] = base[e];
  __syncthreads();
  const int nbits = E > 1 ? 32 - __builtin_clz(static_cast<unsigned>(E - 1)) : 0;
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (kWave - lane));
  const int a0 = blockIdx.x * chunk;
  const int a1 = min(R, a0 + chunk);
  for (int ab = a0; ab < a1; ab += kWave) {
    const int a = ab + lane;
    int e = a < a1 ? idx[a] : -1;
    const bool ok = e >= 0 && e < E;
    uint64_t same = __ballot(ok);
    for (int b = 0; b < nbits; ++b) {
      const bool bit = ok && ((e >> b) & 1);
      const uint64_t bb = __ballot(bit);
      same &= bit ? bb : ~bb;
    }
    int pos = 0;
    if (ok) {
      const int rank = __popcll(same & lt_mask);
      pos = cursor[e] + rank;
    }
    // all lanes have read their cursor before the group leaders advance it
    __builtin_amdgcn_wave_barrier();
    if (ok) {
      const int leader = 63 - __clzll(same);
      if (lane == leader) cursor[e] += __popcll(same);
      row_of[a] = pos;
      src_of[pos] = a;
    }
    __builtin_amdgcn_wave_barrier();
  }
}

// One wave per row; 16-byte copies when the row is a whole number of 16-byte words.
__global__ __launch_bounds__(256) void gather_kernel(const char* __restrict__ x,
                                                     const int32_t* __restrict__ src_of, int R,
                                                     int T, int k, int64_t row_bytes,
                                                     char* __restrict__ x_perm) {
  const int lane = threadIdx.x & (kWave - 1);
  const int r = blockIdx.x * 4 + threadIdx.x / kWave;
  if (r >= R) return;
  const int a = src_of[r];
  // rows past offsets[E] are unwritten when an id was out of range: skip them
  if (a < 0 || a >= R) return;
  const int t = a / k;
  if (t >= T) return;
  const char* src = x + static_cast<int64_t>(t) * row_bytes;
  char* dst = x_perm + static_cast<int64_t>(r) * row_bytes;
  if ((row_bytes & 15) == 0) {
    const uint4* s4 = reinterpret_cast<const uint4*>(src);
    uint4* d4 = reinterpret_cast<uint4*>(dst);
    const int64_t n = row_bytes >> 4;
    for (int64_t i = lane; i < n; i += kWave) d4[i] = s4[i];
  } else {
    const uint16_t* s2 = reinterpret_cast<const uint16_t*>(src);
    uint16_t* d2 = reinterpret_cast<uint16_t*>(dst);
    const int64_t n = row_bytes >> 1;
    for (int64_t i = lane; i < n; i += kWave) d2[i] = s2[i];
  }
}

}  // namespace
}  // namespace moe

extern "C" int moe_permute_workspace_size(int T, int E, int k, size_t* bytes) {
  using namespace moe;
  if (!bytes || T < 0 || E < 1 || k < 1) return fail(MOE_ERR_ARG, "moe_permute_workspace_size: bad arguments");
  *bytes = permute_ws_bytes(static_cast<int64_t>(T) * k, E);
  return MOE_OK;
}

namespace moe {

// The allocation-free variant's workspace: chunk_counts and chunk_base, each at most
// kMaxChunks x MOE_MAX_E int32, i.e. the most any (T, E, k) the kernels accept can need
// (2 MiB; every GPU the library runs on holds its own copy until the process ends).  Host
// code must not pass this name to a kernel (on the host it is only a stand-in for the
// symbol): every use goes through the per-device address from hipGetSymbolAddress.
constexpr size_t kPermuteScratchBytes = 2 * size_t{kMaxChunks} * MOE_MAX_E * sizeof(int32_t);
__device__ __align__(256) char permute_scratch[kPermuteScratchBytes];

namespace {

int permute_impl(const char* who, const int32_t* topk_idx, int T, int E, int k, const void* x,
                 int H, moe_dtype dtype, int32_t* counts, int32_t* offsets, int32_t* row_of,
                 int32_t* src_of, void* x_perm, void* ws, size_t ws_bytes, int32_t* status,
                 moe_stream_t stream) {
  if (T < 0 || E < 1 || k < 1 || H < 1 || (dtype != MOE_F32 && dtype != MOE_BF16))
    return fail(MOE_ERR_ARG, "%s: bad sizes T=%d E=%d k=%d H=%d", who, T, E, k, H);
  if (E > MOE_MAX_E) return fail(MOE_ERR_UNSUPPORTED, "%s: E=%d above %d", who, E, MOE_MAX_E);
  const int64_t R64 = static_cast<int64_t>(T) * k;
  if (R64 > INT32_MAX) return fail(MOE_ERR_UNSUPPORTED, "%s: T*k too large", who);
  const int R = static_cast<int>(R64);
  if (!counts || !offsets || (R > 0 && (!topk_idx || !row_of || !src_of)))
    return fail(MOE_ERR_ARG, "%s: null pointer", who);
  if (x_perm && R > 0 && !x) return fail(MOE_ERR_ARG, "%s: x_perm given without x", who);
  const size_t need = permute_ws_bytes(R, E);
  if (need > 0 && (!ws || ws_bytes < need))
    return fail(MOE_ERR_WORKSPACE, "%s: workspace %zu < %zu bytes", who, ws_bytes, need);

  hipStream_t s = as_stream(stream);
  const Chunking ch = R > 0 ? chunking(R) : Chunking{64, 0};
  int32_t* chunk_counts = static_cast<int32_t*>(ws);
  int32_t* chunk_base = chunk_counts + static_cast<int64_t>(ch.n_chunks) * E;
  const size_t lds = static_cast<size_t>(E) * sizeof(int32_t);

  if (ch.n_chunks > 0) {
    hipLaunchKernelGGL(hist_kernel, dim3(ch.n_chunks), dim3(256), lds, s, topk_idx, R, E,
                       ch.chunk, chunk_counts, status);
    MOE_LAUNCH_CHECK("moe_permute: hist launch");
  }
  hipLaunchKernelGGL(scan_kernel, dim3(1), dim3(MOE_MAX_E), 0, s, chunk_counts, ch.n_chunks, E,
                     chunk_base, counts, offsets);
  MOE_LAUNCH_CHECK("moe_permute: scan launch");
  if (ch.n_chunks > 0) {
    hipLaunchKernelGGL(scatter_kernel, dim3(ch.n_chunks), dim3(kWave), lds, s, topk_idx, R, E,
                       ch.chunk, chunk_base, row_of, src_of);
    MOE_LAUNCH_CHECK("moe_permute: scatter launch");
  }
  if (x_perm && R > 0) {
    const int64_t row_bytes = static_cast<int64_t>(H) * elem_size(dtype);
    hipLaunchKernelGGL(gather_kernel, dim3(ceil_div(R, 4)), dim3(256), 0, s,
                       static_cast<const char*>(x), src_of, R, T, k, row_bytes,
                       static_cast<char*>(x_perm));
    MOE_LAUNCH_CHECK("moe_permute: gather launch");
  }
  return MOE_OK;
}

constexpr int kMaxDevices = 64;
std::mutex scratch_mu;
void* scratch_ptr[kMaxDevices] = {};

// Device address of permute_scratch on the current device, looked up once per device.
int scratch_on_current_device(void** out) {
  int dev = -1;
  MOE_HIP_CHECK(hipGetDevice(&dev));
  if (dev < 0 || dev >= kMaxDevices)
    return fail(MOE_ERR_UNSUPPORTED, "moe_permute_noalloc: device %d above %d", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(scratch_mu);
  if (!scratch_ptr[dev]) {
    void* p = nullptr;
    MOE_HIP_CHECK(hipGetSymbolAddress(&p, HIP_SYMBOL(permute_scratch)));
    if (!p) return fail(MOE_ERR_HIP, "moe_permute_noalloc: no device address for the scratch array");
    scratch_ptr[dev] = p;
  }
  *out = scratch_ptr[dev];
  return MOE_OK;
}

}  // namespace
}  // namespace moe

extern "C" int moe_permute(const int32_t* topk_idx, int T, int E, int k, const void* x, int H,
                           moe_dtype dtype, int32_t* counts, int32_t* offsets, int32_t* row_of,
                           int32_t* src_of, void* x_perm, void* ws, size_t ws_bytes,
                           int32_t* status, moe_stream_t stream) {
  const int rc = moe::permute_impl("moe_permute", topk_idx, T, E, k, x, H, dtype, counts, offsets,
                                   row_of, src_of, x_perm, ws, ws_bytes, status, stream);
  return moe::debug_check(rc, "moe_permute", moe::as_stream(stream), status);
}

extern "C" int moe_permute_noalloc(const int32_t* topk_idx, int T, int E, int k, const void* x,
                                   int H, moe_dtype dtype, int32_t* counts, int32_t* offsets,
                                   int32_t* row_of, int32_t* src_of, void* x_perm, int32_t* status,
                                   moe_stream_t stream) {
  using namespace moe;
  if (T < 0 || E < 1 || k < 1)
    return fail(MOE_ERR_ARG, "moe_permute_noalloc: bad sizes T=%d E=%d k=%d", T, E, k);
  if (E > MOE_MAX_E) return fail(MOE_ERR_UNSUPPORTED, "moe_permute_noalloc: E=%d above %d", E, MOE_MAX_E);
  const int64_t R = static_cast<int64_t>(T) * k;
  if (R > INT32_MAX) return fail(MOE_ERR_UNSUPPORTED, "moe_permute_noalloc: T*k too large");
  const size_t need = permute_ws_bytes(R, E);
  if (need > kPermuteScratchBytes)
    return fail(MOE_ERR_WORKSPACE, "moe_permute_noalloc: needs %zu scratch bytes, above the "
                "%zu the library holds", need, kPermuteScratchBytes);
  void* scratch = nullptr;
  const int rc = scratch_on_current_device(&scratch);
  if (rc) return rc;
  const int rc2 = permute_impl("moe_permute_noalloc", topk_idx, T, E, k, x, H, dtype, counts,
                               offsets, row_of, src_of, x_perm, scratch, kPermuteScratchBytes,
                               status, stream);
  return debug_check(rc2, "moe_permute_noalloc", as_stream(stream), status);
}
