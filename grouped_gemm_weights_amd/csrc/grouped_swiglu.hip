// moe_grouped_swiglu: the grouped GEMM over the experts of the merged buffer,
// with each expert's SwiGLU FFN, and moe_dense_gemm (the pipeline's dense
// stand-in block), which runs the same tile loop on one weight matrix.
//
// bf16 path (gfx950 MFMA, v_mfma_f32_16x16x32_bf16, fp32 accumulate):
//   1. plan:  one block turns offsets[] into a list of BM-row tiles
//             (expert, first row, rows, slot), expert-major, and checks that
//             every expert with rows has a slot in the merged buffer.
//   2. gemm1: per (tile, 64-column block): g = X Wg^T and u = X Wu^T share the
//             A tile; the epilogue writes h = bf16(silu(g) * u).
//   3. gemm2: per (tile, column block): y_perm = h Wd^T in fp32.
// Both GEMMs stage A and B tiles through LDS, double-buffered, with the next
// K step's global loads in flight while the current one feeds the MFMAs.
// Weights are stored output-major ([N][K], K contiguous), so every operand
// row is a contiguous 16-byte vector per lane, as the MFMA wants it.
//
// Two tile shapes are compiled: a decode shape (16-row tiles; the expert
// groups hold a few rows and the kernel streams weights) and a prefill shape
// (128-row tiles, MFMA-bound).  The host picks by the average rows per expert.
//
// f32 path (tiny exact-check workloads): plain fp32 FMA kernels, one thread
// per output element, fp32 throughout.
#include "common.h"

namespace moe {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

struct Tile {
  int32_t expert;
  int32_t row0;
  int32_t rows;
  int32_t slot;
};

constexpr int kMinBM = 16;  // smallest tile height: bounds the tile list

int64_t max_tiles(int64_t R, int E) { return ceil_div64(R, kMinBM) + std::min<int64_t>(E, R); }

struct SwigluWs {
  size_t h_bytes, tiles_off, count_off, total;
};

SwigluWs swiglu_ws(int64_t R, int E, int I, moe_dtype dt) {
  SwigluWs w;
  w.h_bytes = align_up(static_cast<size_t>(R) * I * elem_size(dt), 256);
  w.tiles_off = w.h_bytes;
  w.count_off = w.tiles_off + align_up(static_cast<size_t>(max_tiles(R, E)) * sizeof(Tile), 256);
  w.total = w.count_off + 256;
  return w;
}

// ---------------------------------------------------------------------------
// tile plan
// ---------------------------------------------------------------------------

__global__ __launch_bounds__(MOE_MAX_E) void plan_kernel(const int32_t* __restrict__ offsets, int E,
                                                         int e_begin, int e_end,
                                                         int BM, const int32_t* __restrict__ slot_of,
                                                         Tile* __restrict__ tiles,
                                                         int32_t* __restrict__ n_tiles,
                                                         int32_t* status) {
  __shared__ int32_t s[MOE_MAX_E];
  const int e = threadIdx.x;
  int nt = 0, lo = 0, cnt = 0, slot = -1;
  if (e < E && e >= e_begin && e < e_end) {
    lo = offsets[e];
    cnt = offsets[e + 1] - lo;
    if (cnt > 0) {
      slot = slot_of[e];
      if (slot < 0) status_or(status, MOE_STATUS_EXPERT_ABSENT);
      else nt = (cnt + BM - 1) / BM;
    }
  }
  s[e] = nt;
  __syncthreads();
  for (int off = 1; off < MOE_MAX_E; off <<= 1) {
    const int32_t add = e >= off ? s[e - off] : 0;
    __syncthreads();
    s[e] += add;
    __syncthreads();
  }
  const int start = s[e] - nt;
  for (int i = 0; i < nt; ++i) {
    Tile t;
    t.expert = e;
    t.row0 = lo + i * BM;
    t.rows = min(BM, cnt - i * BM);
    t.slot = slot;
    tiles[start + i] = t;
  }
  if (e == MOE_MAX_E - 1) *n_tiles = s[e];
}

// ---------------------------------------------------------------------------
// bf16 MFMA tile GEMM
// ---------------------------------------------------------------------------

__device__ __forceinline__ float silu_f32(float g) { return g / (1.0f + expf(-g)); }

// out[tile rows][n0 .. n0+BN) for one (tile, column block).
//   A      bf16 rows, row stride lda; rows of this tile start at tile.row0
//   B0/B1  bf16 [N][K] weight matrices at wbase + slot*expert_bytes + b?_off
//   DUAL   gemm1: B0 = Wg, B1 = Wu, out = bf16(silu(A B0^T) * (A B1^T))
//   !DUAL  out = A B0^T, as f32 (OUT_BF16 = false) or bf16
template <int BM, int BN, int BK, int WM, int WN, bool DUAL, bool OUT_BF16>
__global__ __launch_bounds__(WM* WN* kWave) void gemm_bf16_kernel(
    const uint16_t* __restrict__ A, int lda, const int32_t* __restrict__ a_index, int a_div,
    const char* __restrict__ wbase, int64_t expert_bytes,
    int64_t b0_off, int64_t b1_off, int N, int K, const Tile* __restrict__ tiles,
    const int32_t* __restrict__ n_tiles, int dense_M, void* __restrict__ out, int ldo) {
  constexpr int NT = WM * WN * kWave;
  constexpr int NB = DUAL ? 2 : 1;
  constexpr int LDS_LD = BK + 8;             // row stride in elements (16-byte pad)
  constexpr int KC = BK / 8;                 // 16-byte chunks per row per K step
  constexpr int CA = BM * KC / NT;           // A chunks per thread per K step
  constexpr int CB = NB * BN * KC / NT;      // B chunks per thread per K step
  constexpr int TM = BM / WM / 16;
  constexpr int TN = BN / WN / 16;
  static_assert(CA * NT == BM * KC, "A tile must split evenly over the threads");
  static_assert(CB * NT == NB * BN * KC, "B tile must split evenly over the threads");
  static_assert(TM >= 1 && TN >= 1 && BK % 32 == 0, "bad tile shape");

  Tile tile;
  if (tiles) {
    if (static_cast<int>(blockIdx.x) >= *n_tiles) return;
    tile = tiles[blockIdx.x];
  } else {
    tile.expert = 0;
    tile.row0 = blockIdx.x * BM;
    tile.rows = min(BM, dense_M - tile.row0);
    tile.slot = 0;
  }
  const int n0 = blockIdx.y * BN;

  extern __shared__ __align__(16) uint16_t smem[];
  uint16_t* As = smem;                         // [2][BM][LDS_LD]
  uint16_t* Bs = smem + 2 * BM * LDS_LD;       // [2][NB*BN][LDS_LD]

  const char* wexp = wbase + static_cast<int64_t>(tile.slot) * expert_bytes;
  const uint16_t* B0 = reinterpret_cast<const uint16_t*>(wexp + b0_off);
  const uint16_t* B1 = reinterpret_cast<const uint16_t*>(wexp + b1_off);

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const int wm0 = (wave / WN) * (BM / WM);
  const int wn0 = (wave % WN) * (BN / WN);

  // A rows this thread loads: row r of the tile is A row tile.row0 + r, or, gathered,
  // A row a_index[tile.row0 + r] / a_div (rows past the tile read row 0, never stored)
  const uint16_t* a_row[CA];
#pragma unroll
  for (int i = 0; i < CA; ++i) {
    const int r = (tid + i * NT) / KC;
    int src = tile.row0 + (r < tile.rows ? r : 0);
    if (a_index) src = a_index[src] / a_div;
    a_row[i] = A + static_cast<int64_t>(src) * lda;
  }

  uint4 ra[CA], rb[CB];

#define MOE_LOAD_REGS(k0)                                                                     \
  do {                                                                                        \
    _Pragma("unroll") for (int i = 0; i < CA; ++i) {                                          \
      const int c = tid + i * NT;                                                             \
      const int r = c / KC, k = (k0) + (c % KC) * 8;                                          \
      ra[i] = make_uint4(0, 0, 0, 0);                                                         \
      if (r < tile.rows && k < K)                                                             \
        ra[i] = *reinterpret_cast<const uint4*>(a_row[i] + k);                               \
    }                                                                                         \
    _Pragma("unroll") for (int i = 0; i < CB; ++i) {                                          \
      const int c = tid + i * NT;                                                             \
      const int r = c / KC, k = (k0) + (c % KC) * 8;                                          \
      const int n = n0 + (DUAL ? r % BN : r);                                                 \
      const uint16_t* Bm = (DUAL && r >= BN) ? B1 : B0;                                       \
      rb[i] = make_uint4(0, 0, 0, 0);                                                         \
      if (n < N && k < K)                                                                     \
        rb[i] = *reinterpret_cast<const uint4*>(Bm + static_cast<int64_t>(n) * K + k);        \
    }                                                                                         \
  } while (0)

#define MOE_STORE_LDS(buf)                                                                    \
  do {                                                                                        \
    uint16_t* as_ = As + (buf) * BM * LDS_LD;                                                 \
    uint16_t* bs_ = Bs + (buf) * NB * BN * LDS_LD;                                            \
    _Pragma("unroll") for (int i = 0; i < CA; ++i) {                                          \
      const int c = tid + i * NT;                                                             \
      *reinterpret_cast<uint4*>(as_ + (c / KC) * LDS_LD + (c % KC) * 8) = ra[i];              \
    }                                                                                         \
    _Pragma("unroll") for (int i = 0; i < CB; ++i) {                                          \
      const int c = tid + i * NT;                                                             \
      *reinterpret_cast<uint4*>(bs_ + (c / KC) * LDS_LD + (c % KC) * 8) = rb[i];              \
    }                                                                                         \
  } while (0)

  floatx4 acc0[TM][TN], acc1[DUAL ? TM : 1][DUAL ? TN : 1];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc0[i][j] = floatx4{0.f, 0.f, 0.f, 0.f};
  if (DUAL) {
#pragma unroll
    for (int i = 0; i < (DUAL ? TM : 1); ++i)
#pragma unroll
      for (int j = 0; j < (DUAL ? TN : 1); ++j) acc1[i][j] = floatx4{0.f, 0.f, 0.f, 0.f};
  }

  const int nk = (K + BK - 1) / BK;
  MOE_LOAD_REGS(0);
  MOE_STORE_LDS(0);
  __syncthreads();

  const int lrow = lane & 15;        // operand row (A) / column (B) of this lane
  const int lk = (lane >> 4) * 8;    // first of this lane's 8 K values
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nk) MOE_LOAD_REGS((kt + 1) * BK);
    const uint16_t* as = As + cur * BM * LDS_LD;
    const uint16_t* bs = Bs + cur * NB * BN * LDS_LD;
#pragma unroll
    for (int kk = 0; kk < BK; kk += 32) {
      bf16x8_t a[TM], b0[TN], b1[DUAL ? TN : 1];
#pragma unroll
      for (int i = 0; i < TM; ++i)
        a[i] = *reinterpret_cast<const bf16x8_t*>(as + (wm0 + i * 16 + lrow) * LDS_LD + kk + lk);
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        b0[j] = *reinterpret_cast<const bf16x8_t*>(bs + (wn0 + j * 16 + lrow) * LDS_LD + kk + lk);
        if (DUAL)
          b1[DUAL ? j : 0] = *reinterpret_cast<const bf16x8_t*>(
              bs + (BN + wn0 + j * 16 + lrow) * LDS_LD + kk + lk);
      }
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) {
          acc0[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[i], b0[j], acc0[i][j], 0, 0, 0);
          if (DUAL)
            acc1[DUAL ? i : 0][DUAL ? j : 0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                a[i], b1[DUAL ? j : 0], acc1[DUAL ? i : 0][DUAL ? j : 0], 0, 0, 0);
        }
    }
    if (kt + 1 < nk) MOE_STORE_LDS(cur ^ 1);
    __syncthreads();
  }

  // epilogue: lane holds D[(lane/16)*4 + q][lane%16] of each 16x16 block
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int r = wm0 + i * 16 + (lane >> 4) * 4 + q;
        const int n = n0 + wn0 + j * 16 + (lane & 15);
        if (r >= tile.rows || n >= N) continue;
        const int64_t o = static_cast<int64_t>(tile.row0 + r) * ldo + n;
        if (DUAL) {
          const float g = acc0[i][j][q];
          const float u = acc1[DUAL ? i : 0][DUAL ? j : 0][q];
          static_cast<uint16_t*>(out)[o] = f32_to_bf16(silu_f32(g) * u);
        } else if (OUT_BF16) {
          static_cast<uint16_t*>(out)[o] = f32_to_bf16(acc0[i][j][q]);
        } else {
          static_cast<float*>(out)[o] = acc0[i][j][q];
        }
      }
}

#undef MOE_LOAD_REGS
#undef MOE_STORE_LDS

template <int BM, int BN, int BK, int WM, int WN, bool DUAL, bool OUT_BF16>
struct GemmShape {
  static constexpr int kThreads = WM * WN * kWave;
  static constexpr size_t kLds =
      2 * static_cast<size_t>(BM + (DUAL ? 2 : 1) * BN) * (BK + 8) * sizeof(uint16_t);

  static int launch(const uint16_t* A, int lda, const int32_t* a_index, int a_div,
                    const char* wbase, int64_t expert_bytes,
                    int64_t b0_off, int64_t b1_off, int N, int K, const Tile* tiles,
                    const int32_t* n_tiles, int64_t grid_tiles, int dense_M, void* out, int ldo,
                    hipStream_t s) {
    auto kern = gemm_bf16_kernel<BM, BN, BK, WM, WN, DUAL, OUT_BF16>;
    static bool configured = false;
    if (!configured) {
      MOE_HIP_CHECK(hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                        hipFuncAttributeMaxDynamicSharedMemorySize,
                                        static_cast<int>(kLds)));
      configured = true;
    }
    if (grid_tiles <= 0) return MOE_OK;
    dim3 grid(static_cast<unsigned>(grid_tiles), static_cast<unsigned>(ceil_div(N, BN)));
    hipLaunchKernelGGL(kern, grid, dim3(kThreads), kLds, s, A, lda, a_index, a_div, wbase,
                       expert_bytes, b0_off, b1_off, N, K, tiles, n_tiles, dense_M, out, ldo);
    MOE_LAUNCH_CHECK("gemm_bf16_kernel launch");
    return MOE_OK;
  }
};


// ---------------------------------------------------------------------------
// Prefill tile GEMM: 256 x 256 block tile, 8 waves (two per SIMD), 32x32x16
// MFMA, BK = 64, LDS double buffer (144 KB of the CU's 160 KB).
//
// DUAL (gate/up): the B tile holds 128 Wg rows and the same 128 Wu rows, so
// a block produces 256 rows x 128 columns of h; each wave owns 128 rows x 32
// columns of both g and u and applies silu(g) * u in registers.  !DUAL: the B
// tile is 256 rows of one matrix; each wave owns 128 rows x 64 columns.
//
// Work order: the (m-tile, n-tile) items are cut into 8 contiguous chunks,
// one per XCD (workgroup i runs on XCD i % 8), and inside a chunk groups of
// kMGroup consecutive m-tiles sweep the n-tiles together, so the blocks that
// run at the same time on one XCD share A tiles and weight panels in its L2.
// ---------------------------------------------------------------------------

typedef float floatx16 __attribute__((ext_vector_type(16)));

constexpr int kXcds = 8;
constexpr int kMGroup = 4;

template <bool DUAL, bool OUT_BF16>
__global__ __launch_bounds__(512) void gemm_big_kernel(
    const uint16_t* __restrict__ A, int lda, const int32_t* __restrict__ a_index, int a_div,
    const char* __restrict__ wbase, int64_t expert_bytes,
    int64_t b0_off, int64_t b1_off, int N, int K, const Tile* __restrict__ tiles,
    const int32_t* __restrict__ n_tiles, int dense_M, void* __restrict__ out, int ldo) {
  constexpr int BM = 256, BN = 256, BK = 64, NT = 512;
  constexpr int LDS_LD = BK + 8;
  constexpr int KC = BK / 8;
  constexpr int CA = BM * KC / NT;   // 4
  constexpr int CB = BN * KC / NT;   // 4
  constexpr int OUTN = DUAL ? BN / 2 : BN;

  const int n_m = tiles ? *n_tiles : (dense_M + BM - 1) / BM;
  const int n_n = (N + OUTN - 1) / OUTN;
  const int total = n_m * n_n;
  const int chunk = (total + kXcds - 1) / kXcds;
  const int local = blockIdx.x / kXcds;
  if (local >= chunk) return;
  const int w = (blockIdx.x % kXcds) * chunk + local;
  if (w >= total) return;
  const int g = w / (n_n * kMGroup);
  const int gsize = min(kMGroup, n_m - g * kMGroup);
  const int rem = w - g * (n_n * kMGroup);
  const int nt = rem / gsize;
  const int mt = g * kMGroup + rem % gsize;

  Tile tile;
  if (tiles) {
    tile = tiles[mt];
  } else {
    tile.expert = 0;
    tile.row0 = mt * BM;
    tile.rows = min(BM, dense_M - tile.row0);
    tile.slot = 0;
  }
  const int n0 = nt * OUTN;

  extern __shared__ __align__(16) uint16_t smem[];
  uint16_t* As = smem;                       // [2][BM][LDS_LD]
  uint16_t* Bs = smem + 2 * BM * LDS_LD;     // [2][BN][LDS_LD]

  const char* wexp = wbase + static_cast<int64_t>(tile.slot) * expert_bytes;
  const uint16_t* B0 = reinterpret_cast<const uint16_t*>(wexp + b0_off);
  const uint16_t* B1 = reinterpret_cast<const uint16_t*>(wexp + b1_off);

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const int wm0 = (wave >> 2) * 128;          // 2 waves down M
  const int wq = wave & 3;                     // 4 waves across N

  // per-thread load slots (fixed over the K loop)
  const uint16_t* a_src[CA];
  bool a_ok[CA];
  int a_lds[CA];
#pragma unroll
  for (int i = 0; i < CA; ++i) {
    const int c = tid + i * NT;
    const int r = c / KC, kc = c % KC;
    a_ok[i] = r < tile.rows;
    // tile row r is A row tile.row0 + r, or, gathered, A row a_index[tile.row0 + r] / a_div
    int src = tile.row0 + (a_ok[i] ? r : 0);
    if (a_index) src = a_index[src] / a_div;
    a_src[i] = A + static_cast<int64_t>(src) * lda + kc * 8;
    a_lds[i] = r * LDS_LD + kc * 8;
  }
  const uint16_t* b_src[CB];
  bool b_ok[CB];
  int b_lds[CB];
#pragma unroll
  for (int i = 0; i < CB; ++i) {
    const int c = tid + i * NT;
    const int r = c / KC, kc = c % KC;
    const int n = n0 + (DUAL ? (r & (BN / 2 - 1)) : r);
    const uint16_t* Bm = (DUAL && r >= BN / 2) ? B1 : B0;
    b_ok[i] = n < N;
    b_src[i] = Bm + static_cast<int64_t>(b_ok[i] ? n : 0) * K + kc * 8;
    b_lds[i] = r * LDS_LD + kc * 8;
  }

  uint4 ra[CA], rb[CB];
#define BIG_LOAD(k0)                                                              \
  do {                                                                            \
    _Pragma("unroll") for (int i = 0; i < CA; ++i) {                              \
      ra[i] = make_uint4(0, 0, 0, 0);                                             \
      if (a_ok[i] && (k0) + (((tid + i * NT) % KC) * 8) < K)                      \
        ra[i] = *reinterpret_cast<const uint4*>(a_src[i] + (k0));                 \
    }                                                                             \
    _Pragma("unroll") for (int i = 0; i < CB; ++i) {                              \
      rb[i] = make_uint4(0, 0, 0, 0);                                             \
      if (b_ok[i] && (k0) + (((tid + i * NT) % KC) * 8) < K)                      \
        rb[i] = *reinterpret_cast<const uint4*>(b_src[i] + (k0));                 \
    }                                                                             \
  } while (0)
#define BIG_STORE(buf)                                                            \
  do {                                                                            \
    _Pragma("unroll") for (int i = 0; i < CA; ++i)                                \
      *reinterpret_cast<uint4*>(As + (buf) * BM * LDS_LD + a_lds[i]) = ra[i];     \
    _Pragma("unroll") for (int i = 0; i < CB; ++i)                                \
      *reinterpret_cast<uint4*>(Bs + (buf) * BN * LDS_LD + b_lds[i]) = rb[i];     \
  } while (0)

  floatx16 acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.f;

  // operand rows of this lane inside the LDS tiles
  const int lrow = lane & 31;
  const int lk = (lane >> 5) * 8;
  int brow[2];
  if (DUAL) {
    brow[0] = wq * 32 + lrow;
    brow[1] = BN / 2 + wq * 32 + lrow;
  } else {
    brow[0] = wq * 64 + lrow;
    brow[1] = wq * 64 + 32 + lrow;
  }

  const int nk = (K + BK - 1) / BK;
  BIG_LOAD(0);
  BIG_STORE(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nk) BIG_LOAD((kt + 1) * BK);
    const uint16_t* as = As + cur * BM * LDS_LD;
    const uint16_t* bs = Bs + cur * BN * LDS_LD;
#pragma unroll
    for (int ks = 0; ks < BK; ks += 16) {
      bf16x8_t a[4], b[2];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        a[i] = *reinterpret_cast<const bf16x8_t*>(as + (wm0 + i * 32 + lrow) * LDS_LD + ks + lk);
#pragma unroll
      for (int j = 0; j < 2; ++j)
        b[j] = *reinterpret_cast<const bf16x8_t*>(bs + brow[j] * LDS_LD + ks + lk);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
    }
    if (kt + 1 < nk) BIG_STORE(cur ^ 1);
    __syncthreads();
  }
#undef BIG_LOAD
#undef BIG_STORE

  // epilogue: element q of a 32x32 block sits at row (q/4)*8 + (lane/32)*4 + q%4, column lane%32
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      const int r = wm0 + i * 32 + (q >> 2) * 8 + (lane >> 5) * 4 + (q & 3);
      if (r >= tile.rows) continue;
      const int64_t orow = static_cast<int64_t>(tile.row0 + r) * ldo;
      if (DUAL) {
        const int n = n0 + wq * 32 + lrow;
        if (n < N)
          static_cast<uint16_t*>(out)[orow + n] = f32_to_bf16(silu_f32(acc[i][0][q]) * acc[i][1][q]);
      } else {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int n = n0 + wq * 64 + j * 32 + lrow;
          if (n >= N) continue;
          if (OUT_BF16) static_cast<uint16_t*>(out)[orow + n] = f32_to_bf16(acc[i][j][q]);
          else static_cast<float*>(out)[orow + n] = acc[i][j][q];
        }
      }
    }
}

template <bool DUAL, bool OUT_BF16>
struct GemmBig {
  static constexpr int BM = 256;
  static constexpr size_t kLds = 2 * static_cast<size_t>(256 + 256) * (64 + 8) * sizeof(uint16_t);

  // grid_m: upper bound on the number of m-tiles
  static int launch(const uint16_t* A, int lda, const int32_t* a_index, int a_div,
                    const char* wbase, int64_t expert_bytes,
                    int64_t b0_off, int64_t b1_off, int N, int K, const Tile* tiles,
                    const int32_t* n_tiles, int64_t grid_m, int dense_M, void* out, int ldo,
                    hipStream_t s) {
    auto kern = gemm_big_kernel<DUAL, OUT_BF16>;
    static bool configured = false;
    if (!configured) {
      MOE_HIP_CHECK(hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                        hipFuncAttributeMaxDynamicSharedMemorySize,
                                        static_cast<int>(kLds)));
      configured = true;
    }
    if (grid_m <= 0) return MOE_OK;
    const int outn = DUAL ? 128 : 256;
    const int64_t items = grid_m * ceil_div(N, outn);
    const int64_t blocks = ceil_div64(items, kXcds) * kXcds;
    hipLaunchKernelGGL(kern, dim3(static_cast<unsigned>(blocks)), dim3(512), kLds, s, A, lda, a_index,
                       a_div, wbase, expert_bytes, b0_off, b1_off, N, K, tiles, n_tiles, dense_M,
                       out, ldo);
    MOE_LAUNCH_CHECK("gemm_big_kernel launch");
    return MOE_OK;
  }
};

// decode shapes: 16-row tiles, weights streamed in 128-deep K steps
using Gemm1Decode = GemmShape<16, 64, 128, 1, 4, true, false>;
using Gemm2Decode = GemmShape<16, 64, 128, 1, 4, false, false>;
// prefill shapes: 128-row tiles
using Gemm1Prefill = GemmBig<true, false>;
using Gemm2Prefill = GemmBig<false, false>;
using DenseBf16 = GemmBig<false, true>;

// ---------------------------------------------------------------------------
// f32 path
// ---------------------------------------------------------------------------

__device__ __forceinline__ int expert_of_row(const int32_t* offsets, int E, int r) {
  int lo = 0, hi = E;  // find e with offsets[e] <= r < offsets[e+1]
  while (hi - lo > 1) {
    const int mid = (lo + hi) / 2;
    if (offsets[mid] <= r) lo = mid;
    else hi = mid;
  }
  return lo;
}

__global__ __launch_bounds__(256) void gemm1_f32_kernel(const float* __restrict__ x_perm,
                                                        const int32_t* __restrict__ a_index, int a_div,
                                                        const int32_t* __restrict__ offsets, int E,
                                                        int e_begin, int e_end,
                                                        const int32_t* __restrict__ slot_of,
                                                        const char* __restrict__ wbase,
                                                        int64_t eb, int H, int I,
                                                        float* __restrict__ h, int32_t* status) {
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  const int R = offsets[E];
  if (idx >= static_cast<int64_t>(R) * I) return;
  const int r = static_cast<int>(idx / I), n = static_cast<int>(idx % I);
  const int e = expert_of_row(offsets, E, r);
  if (e < e_begin || e >= e_end) return;
  const int slot = slot_of[e];
  if (slot < 0) {
    status_or(status, MOE_STATUS_EXPERT_ABSENT);
    return;
  }
  const float* W = reinterpret_cast<const float*>(wbase + static_cast<int64_t>(slot) * eb);
  const float* wg = W + static_cast<int64_t>(n) * H;
  const float* wu = W + static_cast<int64_t>(H) * I + static_cast<int64_t>(n) * H;
  const float* x = x_perm + static_cast<int64_t>(a_index ? a_index[r] / a_div : r) * H;
  float g = 0.f, u = 0.f;
  for (int c = 0; c < H; ++c) {
    g = fmaf(x[c], wg[c], g);
    u = fmaf(x[c], wu[c], u);
  }
  h[idx] = silu_f32(g) * u;
}

__global__ __launch_bounds__(256) void gemm2_f32_kernel(const float* __restrict__ h,
                                                        const int32_t* __restrict__ offsets, int E,
                                                        int e_begin, int e_end,
                                                        const int32_t* __restrict__ slot_of,
                                                        const char* __restrict__ wbase,
                                                        int64_t eb, int H, int I,
                                                        float* __restrict__ y_perm) {
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  const int R = offsets[E];
  if (idx >= static_cast<int64_t>(R) * H) return;
  const int r = static_cast<int>(idx / H), o = static_cast<int>(idx % H);
  const int e = expert_of_row(offsets, E, r);
  if (e < e_begin || e >= e_end) return;
  const int slot = slot_of[e];
  if (slot < 0) return;
  const float* wd = reinterpret_cast<const float*>(wbase + static_cast<int64_t>(slot) * eb) +
                    2 * static_cast<int64_t>(H) * I + static_cast<int64_t>(o) * I;
  const float* hr = h + static_cast<int64_t>(r) * I;
  float acc = 0.f;
  for (int n = 0; n < I; ++n) acc = fmaf(hr[n], wd[n], acc);
  y_perm[idx] = acc;
}

}  // namespace
}  // namespace moe

extern "C" int moe_grouped_swiglu_workspace_size(int R, int E, int H, int I, moe_dtype dtype,
                                                 size_t* bytes) {
  using namespace moe;
  if (!bytes || R < 0 || E < 1 || H < 1 || I < 1 || (dtype != MOE_F32 && dtype != MOE_BF16))
    return fail(MOE_ERR_ARG, "moe_grouped_swiglu_workspace_size: bad arguments");
  *bytes = swiglu_ws(R, E, I, dtype).total;
  return MOE_OK;
}

namespace moe {
namespace {

// The grouped SwiGLU over experts [e_begin, e_end).  A row r of the gate/up GEMM is row r of
// x_perm, or, when a_index is given, row a_index[r] / a_div of x (the gather done on load).
int grouped_swiglu_impl(const void* x_perm, const int32_t* a_index, int a_div,
                        const int32_t* offsets, int R, int E, int H, int I, moe_dtype dtype,
                        const moe_wbuf* w, int e_begin, int e_end, void* ws, size_t ws_bytes,
                        float* y_perm, int32_t* status, moe_stream_t stream) {
  if (e_begin < 0 || e_end > E || e_begin > e_end)
    return fail(MOE_ERR_ARG, "moe_grouped_swiglu: expert range [%d, %d) outside [0, %d)", e_begin,
                e_end, E);
  if (R < 0 || E < 1 || H < 1 || I < 1 || (dtype != MOE_F32 && dtype != MOE_BF16))
    return fail(MOE_ERR_ARG, "moe_grouped_swiglu: bad sizes R=%d E=%d H=%d I=%d", R, E, H, I);
  if (E > MOE_MAX_E) return fail(MOE_ERR_UNSUPPORTED, "moe_grouped_swiglu: E=%d above %d", E, MOE_MAX_E);
  if (!w || !w->base || !w->slot_of || !offsets)
    return fail(MOE_ERR_ARG, "moe_grouped_swiglu: null pointer");
  const int64_t eb = 3 * static_cast<int64_t>(H) * I * elem_size(dtype);
  if (w->expert_bytes != eb || w->n_experts != E)
    return fail(MOE_ERR_ARG, "moe_grouped_swiglu: merged buffer holds %lld-byte blocks for E=%d, "
                "expected %lld for E=%d", static_cast<long long>(w->expert_bytes), w->n_experts,
                static_cast<long long>(eb), E);
  if (dtype == MOE_BF16 && (H % 8 != 0 || I % 8 != 0))
    return fail(MOE_ERR_UNSUPPORTED, "moe_grouped_swiglu: H=%d and I=%d must be multiples of 8", H, I);
  const SwigluWs L = swiglu_ws(R, E, I, dtype);
  if (!ws || ws_bytes < L.total)
    return fail(MOE_ERR_WORKSPACE, "moe_grouped_swiglu: workspace %zu < %zu bytes", ws_bytes, L.total);
  if (R == 0) return MOE_OK;
  if (!x_perm || !y_perm) return fail(MOE_ERR_ARG, "moe_grouped_swiglu: null pointer");

  hipStream_t s = as_stream(stream);
  char* wsb = static_cast<char*>(ws);
  void* h = wsb;
  const char* wbase = static_cast<const char*>(w->base);

  if (dtype == MOE_F32) {
    const int64_t n1 = static_cast<int64_t>(R) * I, n2 = static_cast<int64_t>(R) * H;
    hipLaunchKernelGGL(gemm1_f32_kernel, dim3(static_cast<unsigned>(ceil_div64(n1, 256))), dim3(256),
                       0, s, static_cast<const float*>(x_perm), a_index, a_div, offsets, E,
                       e_begin, e_end,
                       w->slot_of, wbase, eb, H, I, static_cast<float*>(h), status);
    MOE_LAUNCH_CHECK("moe_grouped_swiglu: gemm1 f32");
    hipLaunchKernelGGL(gemm2_f32_kernel, dim3(static_cast<unsigned>(ceil_div64(n2, 256))), dim3(256),
                       0, s, static_cast<const float*>(h), offsets, E, e_begin, e_end, w->slot_of,
                       wbase, eb, H, I, y_perm);
    MOE_LAUNCH_CHECK("moe_grouped_swiglu: gemm2 f32");
    return MOE_OK;
  }

  Tile* tiles = reinterpret_cast<Tile*>(wsb + L.tiles_off);
  int32_t* n_tiles = reinterpret_cast<int32_t*>(wsb + L.count_off);
  const bool decode = static_cast<int64_t>(R) <= 4 * static_cast<int64_t>(E);
  const int BM = decode ? 16 : GemmBig<true, false>::BM;
  const int64_t grid_tiles = ceil_div64(R, BM) + std::min(E, R);
  hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(MOE_MAX_E), 0, s, offsets, E, e_begin, e_end, BM,
                     w->slot_of, tiles, n_tiles, status);
  MOE_LAUNCH_CHECK("moe_grouped_swiglu: plan");

  const int64_t HI2 = static_cast<int64_t>(H) * I * 2;  // bytes of one H x I bf16 matrix
  const uint16_t* xp = static_cast<const uint16_t*>(x_perm);
  const uint16_t* hp = static_cast<const uint16_t*>(h);
  int rc;
  if (decode) {
    rc = Gemm1Decode::launch(xp, H, a_index, a_div, wbase, eb, 0, HI2, I, H, tiles, n_tiles,
                             grid_tiles, 0, h, I, s);
    if (rc) return rc;
    rc = Gemm2Decode::launch(hp, I, nullptr, 1, wbase, eb, 2 * HI2, 0, H, I, tiles, n_tiles,
                             grid_tiles, 0, y_perm, H, s);
  } else {
    rc = Gemm1Prefill::launch(xp, H, a_index, a_div, wbase, eb, 0, HI2, I, H, tiles, n_tiles,
                              grid_tiles, 0, h, I, s);
    if (rc) return rc;
    rc = Gemm2Prefill::launch(hp, I, nullptr, 1, wbase, eb, 2 * HI2, 0, H, I, tiles, n_tiles,
                              grid_tiles, 0, y_perm, H, s);
  }
  return rc;
}

}  // namespace
}  // namespace moe

extern "C" int moe_grouped_swiglu_range(const void* x_perm, const int32_t* offsets, int R, int E,
                                        int H, int I, moe_dtype dtype, const moe_wbuf* w,
                                        int e_begin, int e_end, void* ws, size_t ws_bytes,
                                        float* y_perm, int32_t* status, moe_stream_t stream) {
  return moe::grouped_swiglu_impl(x_perm, nullptr, 1, offsets, R, E, H, I, dtype, w, e_begin, e_end,
                                  ws, ws_bytes, y_perm, status, stream);
}

extern "C" int moe_grouped_swiglu_gathered(const void* x, const int32_t* src_of, int k,
                                           const int32_t* offsets, int R, int E, int H, int I,
                                           moe_dtype dtype, const moe_wbuf* w, int e_begin,
                                           int e_end, void* ws, size_t ws_bytes, float* y_perm,
                                           int32_t* status, moe_stream_t stream) {
  using namespace moe;
  if (k < 1) return fail(MOE_ERR_ARG, "moe_grouped_swiglu_gathered: k=%d", k);
  if (R > 0 && !src_of) return fail(MOE_ERR_ARG, "moe_grouped_swiglu_gathered: null src_of");
  return grouped_swiglu_impl(x, src_of, k, offsets, R, E, H, I, dtype, w, e_begin, e_end, ws,
                             ws_bytes, y_perm, status, stream);
}


extern "C" int moe_grouped_swiglu(const void* x_perm, const int32_t* offsets, int R, int E, int H,
                                  int I, moe_dtype dtype, const moe_wbuf* w, void* ws,
                                  size_t ws_bytes, float* y_perm, int32_t* status,
                                  moe_stream_t stream) {
  return moe_grouped_swiglu_range(x_perm, offsets, R, E, H, I, dtype, w, 0, E, ws, ws_bytes, y_perm,
                                  status, stream);
}

extern "C" int moe_dense_gemm(const void* x, const void* w, int M, int N, int K, void* out,
                              moe_stream_t stream) {
  using namespace moe;
  if (M < 0 || N < 1 || K < 1) return fail(MOE_ERR_ARG, "moe_dense_gemm: bad sizes M=%d N=%d K=%d", M, N, K);
  if (N % 8 != 0 || K % 8 != 0)
    return fail(MOE_ERR_UNSUPPORTED, "moe_dense_gemm: N=%d and K=%d must be multiples of 8", N, K);
  if (M == 0) return MOE_OK;
  if (!x || !w || !out) return fail(MOE_ERR_ARG, "moe_dense_gemm: null pointer");
  return DenseBf16::launch(static_cast<const uint16_t*>(x), K, nullptr, 1, static_cast<const char*>(w), 0, 0, 0,
                           N, K, nullptr, nullptr, ceil_div(M, DenseBf16::BM), M, out, N,
                           as_stream(stream));
}
