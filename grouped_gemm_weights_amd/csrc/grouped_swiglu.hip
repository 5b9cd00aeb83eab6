// moe_grouped_swiglu: the grouped GEMM over the experts of the merged buffer
// (DWDP explainer, contiguous-buffer panel: local and fetched experts feed one
// grouped GEMM), with each expert's SwiGLU FFN, and moe_dense_gemm (the
// pipeline's dense stand-in block), which runs the prefill tile loop on one
// weight matrix.
//
// bf16 path (gfx950 MFMA, fp32 accumulate):
//   1. plan:  one block turns offsets[] into a list of BM-row tiles
//             (expert, first row, rows, slot), expert-major; prefill tiles go
//             into two lists (full tiles, and short last tiles), and every
//             expert with rows must have a slot in the merged buffer.
//   2. gemm1: per (tile, column block): g = X Wg^T and u = X Wu^T share the
//             A rows; the epilogue writes h = bf16(silu(g) * u).
//   3. gemm2: per (tile, column block): y_perm = h Wd^T in fp32.
// Weights are stored output-major ([N][K], K contiguous), so every operand
// row is a contiguous 16-byte vector per lane, as the MFMA wants it.
//
// Two tile kernels, picked by the average rows per expert:
//   decode  (<= 4 rows per expert on average): 16-row tiles, gemm_stream_kernel
//           streams each weight row once from HBM straight into 16x16x32 MFMA
//           operand registers (no LDS): the call is bound by weight bytes.
//   prefill: 256-row tiles, gemm_wide_kernel: one wave per SIMD with 128 x 128
//           accumulator quarters, 32x32x16 MFMA, LDS double buffer, a hand-
//           pipelined K loop; MFMA-bound.
//
// f32 path (tiny exact-check workloads): plain fp32 FMA kernels, one thread
// per output element, fp32 throughout.
#include <type_traits>

#include "common.h"

namespace moe {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

struct Tile {
  int32_t expert;
  int32_t row0;
  int32_t rows;
  int32_t slot;
};

// The combine folded into the down GEMM's epilogue: output row r of expert e belongs to
// assignment a = src_of[r] (token a / k, slot a % k); its row is scaled by w[a] and added
// into y[a / k] with a float atomic.  y = nullptr: plain stores into y_perm instead.
struct Scatter {
  const int32_t* src_of;
  const float* w;
  int k;
  float* y;
};

constexpr int kMinBM = 16;        // smallest tile height: bounds the tile list
constexpr int kWidePlanBM = 256;  // prefill tile height: tiles split into heavy and light lists

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

// Tiles of BM rows per expert.  Decode tiles (BM < 256) go out expert-major.
// Prefill tiles are split into two expert-major lists: heavy tiles (more than
// 3/4 of BM rows, MFMA-bound) at [0, n_heavy) and light tiles (an expert's
// short last tile, bound by streaming that expert's weights) at
// [n_heavy, n_heavy + n_light), so the GEMM can interleave the two kinds.
// n_tiles[0] = all tiles, n_tiles[1] = heavy, n_tiles[2] = light.
__global__ __launch_bounds__(MOE_MAX_E) void plan_kernel(const int32_t* __restrict__ offsets, int E,
                                                         int e_begin, int e_end,
                                                         int BM, const int32_t* __restrict__ slot_of,
                                                         int n_slots,
                                                         Tile* __restrict__ tiles,
                                                         int32_t* __restrict__ n_tiles,
                                                         int32_t* status) {
  __shared__ int64_t s[MOE_MAX_E];   // heavy count in the low 32 bits, light count in the high
  const int e = threadIdx.x;
  int nh = 0, nl = 0, lo = 0, cnt = 0, slot = -1;
  if (e < E && e >= e_begin && e < e_end) {
    lo = offsets[e];
    cnt = offsets[e + 1] - lo;
    if (cnt > 0) {
      slot = slot_of[e];
      // a slot outside the merged buffer is treated as absent, never read
      if (slot < 0 || slot >= n_slots) {
        slot = -1;
        status_or(status, MOE_STATUS_EXPERT_ABSENT);
      } else if (BM < kWidePlanBM) {
        nh = (cnt + BM - 1) / BM;
      } else {
        const int rem = cnt % BM;
        nh = cnt / BM + (4 * rem > 3 * BM ? 1 : 0);
        nl = (rem > 0 && 4 * rem <= 3 * BM) ? 1 : 0;
      }
    }
  }
  s[e] = static_cast<int64_t>(nh) | (static_cast<int64_t>(nl) << 32);
  __syncthreads();
  for (int off = 1; off < MOE_MAX_E; off <<= 1) {
    const int64_t add = e >= off ? s[e - off] : 0;
    __syncthreads();
    s[e] += add;
    __syncthreads();
  }
  const int n_heavy = static_cast<int>(s[MOE_MAX_E - 1] & 0xffffffff);
  const int n_light = static_cast<int>(s[MOE_MAX_E - 1] >> 32);
  const int h0 = static_cast<int>(s[e] & 0xffffffff) - nh;
  const int l0 = static_cast<int>(s[e] >> 32) - nl;
  for (int i = 0; i < nh + nl; ++i) {
    Tile t;
    t.expert = e;
    t.row0 = lo + i * BM;
    t.rows = min(BM, cnt - i * BM);
    t.slot = slot;
    tiles[i < nh ? h0 + i : n_heavy + l0] = t;
  }
  if (e == 0) {
    n_tiles[0] = n_heavy + n_light;
    n_tiles[1] = n_heavy;
    n_tiles[2] = n_light;
  }
}

// ---------------------------------------------------------------------------
// bf16 MFMA tile GEMM
// ---------------------------------------------------------------------------

// silu(g) = g * sigmoid(g) = g / (1 + e^-g), with e^-g = 2^(-g log2 e) and the quotient
// from the hardware exp2 and reciprocal (about 1 ulp each, so a few fp32 ulp in all).
// Limits hold: g -> -inf gives e^-g = inf, 1 / inf = 0 and a (signed) zero; g -> +inf
// gives g.  This runs once per output of the gate/up GEMM while its MFMA pipes wait, so
// the libm exp and the IEEE division (dozens of instructions each) are avoided.
__device__ __forceinline__ float silu_f32(float g) {
  const float e = __builtin_amdgcn_exp2f(g * -1.4426950408889634f);
  return g * __builtin_amdgcn_rcpf(1.0f + e);
}

// ---------------------------------------------------------------------------
// Prefill work order: groups of kMGroup consecutive m-tiles sweep all n-tiles
// together on one XCD (workgroup i runs on XCD i % 8), so the blocks that run
// at the same time there share A tiles and weight panels in its L2; groups go
// round-robin over the XCDs (a split into 8 contiguous ranges left one XCD 17 %
// over the mean under Zipf routing).  Heavy groups (full tiles, MFMA-bound) are
// spread evenly among light ones (an expert's short last tile, bound by
// streaming the expert's weights from HBM), so at any time some CUs stream
// weights while others compute, instead of a hot expert's tiles running
// together and leaving HBM idle.
//
// A hot expert (skewed routing) fills several consecutive heavy groups.  Where
// 4 (else 2) consecutive groups, aligned to 4 (2) in the heavy list, hold tiles
// of one expert only, they are regrouped: each takes all 4 kMGroup (2 kMGroup)
// m-tiles of the run but only a quarter (half) of the n-tiles, so an XCD holds
// 8 A tiles and 4 weight panels of the gate/up GEMM at a time instead of 2 and
// 16, and each panel crosses the fabric once per 8 m-tiles rather than per 2
// (8K tokens under Zipf(1.1) routing: 164 of 235 heavy tiles, the call ~1.5 %
// faster; uniform routing gives experts 2 full tiles and nothing to regroup).
// ---------------------------------------------------------------------------

typedef float floatx16 __attribute__((ext_vector_type(16)));

constexpr int kXcds = 8;
constexpr int kMGroup = 2;

// ---------------------------------------------------------------------------
// Prefill tile GEMM, one wave per SIMD: 256 x 256 block tile, 4 waves, 32x32x16
// MFMA, BK = 64, LDS double buffer (144 KB).
//
// Full tiles (more than 192 rows): each wave owns a 128 x 128 quarter (4 x 4
// MFMA blocks, all 256 accumulators per lane).  Against an 8-wave split into
// 128 x 64 quarters this reads a third less LDS per MFMA (each operand fetched
// from LDS feeds four MFMAs), and LDS bandwidth is what bounds this loop.
// Partial tiles (at most MI * 32 rows, MI = 1, 2, 4 or 6): the waves split the
// columns instead and each owns all MI * 32 rows x 64 columns, so the MFMA work
// of the tile shrinks with its row count rather than idling whole SIMDs (a tile of
// at most 32 rows, most of an expert's short last tiles under skewed routing, issues
// half the MFMAs and A stage writes of a 64-row one: 1-2 % off the grouped call).  An
// expert's last tile is usually partial (8K-token Zipf routing: 38 % of the
// tile rows would be padding), as is every tile of a 4096-token layer.
//
// Cache hints: a partial tile is its expert's only reader of the weight panels it
// streams (the expert's full tiles, if any, run in heavy groups elsewhere), so its
// weight loads are non-temporal and do not evict the panels a heavy group on the same
// XCD shares between its m-tiles; the epilogue's stores (h, y_perm) are non-temporal
// too, as they are far larger than L2 and read back only by the next kernel.  Full
// tiles' weight loads and every activation load stay cached.
//
// The loop is software-pipelined by hand: the operand fragments of K step
// s + 1 are read from LDS while the MFMAs of step s issue, and every stage's
// global loads are issued two K iterations before their LDS write (a two-slot
// register ring), one chunk per MFMA slot, so HBM latency stays hidden with a
// single wave per SIMD even when a partial tile's iterations are short.
//
// DUAL (gate/up): the B tile holds 128 Wg rows and the same 128 Wu rows.  Full
// tiles: wave (wm, wn) owns h rows 128 wm .. +128 and columns 64 wn .. +64,
// i.e. B-tile rows 64 wn .. +64 (gate) and 128 + 64 wn .. +64 (up).  Partial
// tiles: wave w owns h columns 32 w .. +32 (gate rows 32 w, up rows 128 + 32 w).
// !DUAL: full tiles, wave (wm, wn) owns output columns 128 wn .. +128; partial
// tiles, wave w owns columns 64 w .. +64.
// ---------------------------------------------------------------------------

constexpr int kWideBM = 256, kWideBN = 256, kWideBK = 64, kWideLd = kWideBK + 8;

// MI = 0: full tile; MI > 0: partial tile of at most MI * 32 rows.  COMB (down GEMM only):
// the epilogue scatters w-scaled rows into y (Scatter) instead of storing them.
template <bool DUAL, bool OUT_BF16, bool KFULL, int MI, bool COMB>
__device__ __forceinline__ void wide_tile(const Tile& tile, int n0, const uint16_t* __restrict__ A,
                                          int lda, const int32_t* __restrict__ a_index, int a_div,
                                          const uint16_t* __restrict__ B0,
                                          const uint16_t* __restrict__ B1, int N, int K,
                                          void* __restrict__ out, int ldo, uint16_t* smem,
                                          const Scatter& sc) {
  static_assert(!COMB || (!DUAL && !OUT_BF16), "the combine runs in the f32 down GEMM");
  constexpr int BN = kWideBN, BK = kWideBK, NT = 256;
  constexpr int LDS_LD = kWideLd;
  constexpr int KC = BK / 8;            // 16-byte chunks per row per stage
  constexpr int RSTEP = NT / KC;        // 32: row distance between a thread's chunks
  constexpr int CHB = BN / RSTEP;       // 8 B chunks per thread per stage
  constexpr int CHA = MI ? MI : 8;      // A chunks per thread per stage (rows the tile can have)
  constexpr int MW = MI ? MI : 4;       // 32-row MFMA blocks per wave
  constexpr int NJ = MI ? 2 : 4;        // 32-column MFMA blocks per wave
  constexpr int NMF = MW * NJ;          // MFMAs per 16-deep K step
  constexpr int NRD = MW + NJ;          // operand fragments per K step
  constexpr int NLD = CHA + CHB;        // staged chunks per stage
  constexpr int NS = NMF > NLD ? NMF : NLD;
  constexpr int STAGE = kWideBM * LDS_LD;  // elements of one A (or B) stage buffer

  uint16_t* As = smem;                  // [2][BM][LDS_LD]
  uint16_t* Bs = smem + 2 * STAGE;      // [2][BN][LDS_LD]

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const int wm0 = MI ? 0 : (wave >> 1) * 128;
  const int wn = wave & 1;

  // Load slots: chunk i of this thread is tile row tid / KC + RSTEP * i, K chunk tid % KC.
  // Rows past the tile and columns past N read a valid row instead (row 0 of the tile,
  // weight row 0): their products only reach outputs that are never stored.
  const int kc = tid % KC;
  const int lr0 = tid / KC;
  // A chunks: 32-bit byte offsets from a wave-uniform base (the tile's first row, or the
  // start of x when rows are gathered; the host keeps gathered offsets below 2^32)
  const char* a_base = reinterpret_cast<const char*>(
      a_index ? A : A + static_cast<int64_t>(tile.row0) * lda);
  uint32_t a_off[CHA];
  uint32_t b_off[CHB];                  // element offsets into B0 (B1 for DUAL chunks >= CHB / 2)
  // tile row r is A row tile.row0 + r, or, gathered, A row a_index[tile.row0 + r] / a_div
  int src[CHA];
#pragma unroll
  for (int i = 0; i < CHA; ++i) {
    const int r = lr0 + RSTEP * i;
    src[i] = tile.row0 + (r < tile.rows ? r : 0);
  }
  if (a_index) {
#pragma unroll
    for (int i = 0; i < CHA; ++i) src[i] = a_index[src[i]];
#pragma unroll
    for (int i = 0; i < CHA; ++i) src[i] /= a_div;
  }
#pragma unroll
  for (int i = 0; i < CHA; ++i)
    a_off[i] = static_cast<uint32_t>(a_index ? src[i] : src[i] - tile.row0) *
                   static_cast<uint32_t>(lda) * 2u + kc * 16u;
#pragma unroll
  for (int i = 0; i < CHB; ++i) {
    const int r = lr0 + RSTEP * i;
    const int n = n0 + (DUAL ? (r & (BN / 2 - 1)) : r);
    b_off[i] = static_cast<uint32_t>(n < N ? n : 0) * static_cast<uint32_t>(K) + kc * 8;
  }
  const int st_off = lr0 * LDS_LD + kc * 8;

  // operand rows of this lane inside the LDS tiles (32x32x16: row lane % 32, K (lane / 32) * 8)
  const int lrow = lane & 31;
  const int lk = (lane >> 5) * 8;
  const int a_rd = (wm0 + lrow) * LDS_LD + lk;
  int b_rd[NJ];
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    int br;
    if (MI) br = DUAL ? (j == 0 ? wave * 32 : BN / 2 + wave * 32) : wave * 64 + j * 32;
    else br = DUAL ? (j < 2 ? wn * 64 + j * 32 : BN / 2 + wn * 64 + (j - 2) * 32) : wn * 128 + j * 32;
    b_rd[j] = (br + lrow) * LDS_LD + lk;
  }

  floatx16 acc[MW][NJ];
#pragma unroll
  for (int i = 0; i < MW; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
      for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.f;

  // two stages in flight from global memory for every tile mode (a partial tile's short K
  // iterations would not cover the latency of one; with one, 65-192-row tiles measured
  // the same or slightly slower)
  constexpr int RING = 2;
  u32x4_t ra[RING][CHA], rb[RING][CHB];
  bf16x8_t pa[MW], pb[NJ], qa[MW], qb[NJ]; // operands of two consecutive K steps

  // one global chunk load into ring slot rs (chunk t: A chunks first, then B); past K
  // the chunk is zero.  A and B chunks are separate statements so that the B chunks'
  // non-temporal hint survives (one load of either kind behind a select on t would be
  // merged into a plain load before the loop is unrolled)
#define W_GLD(t, k0, rs)                                                               \
  do {                                                                                 \
    if ((t) < CHA) {                                                                   \
      const u32x4_t* src_ = reinterpret_cast<const u32x4_t*>(                          \
          a_base + (a_off[(t) % CHA] + 2u * (k0)));                                    \
      u32x4_t v_ = u32x4_t{0, 0, 0, 0};                                                \
      if (KFULL || (k0) + kc * 8 < K) v_ = *src_;                                      \
      ra[rs][(t) % CHA] = v_;                                                          \
    } else {                                                                           \
      const u32x4_t* src_ = reinterpret_cast<const u32x4_t*>(                          \
          ((DUAL && ((t) - CHA) % CHB >= CHB / 2) ? B1 : B0) +                         \
          (b_off[((t) - CHA) % CHB] + (k0)));                                          \
      u32x4_t v_ = u32x4_t{0, 0, 0, 0};                                                \
      if (KFULL || (k0) + kc * 8 < K)                                                  \
        v_ = MI ? __builtin_nontemporal_load(src_) : *src_;                            \
      rb[rs][((t) - CHA) % CHB] = v_;                                                  \
    }                                                                                  \
  } while (0)
#define W_DSW(t, buf, rs)                                                              \
  do {                                                                                 \
    if ((t) < CHA)                                                                     \
      *reinterpret_cast<u32x4_t*>(As + (buf) * STAGE + st_off + ((t) % CHA) * RSTEP * LDS_LD) = \
          ra[rs][(t) % CHA];                                                           \
    else                                                                               \
      *reinterpret_cast<u32x4_t*>(Bs + (buf) * STAGE + st_off +                        \
                                (((t) - CHA) % CHB) * RSTEP * LDS_LD) = rb[rs][((t) - CHA) % CHB]; \
  } while (0)
  // one operand fragment read (slot t: A row blocks first, then B column blocks) of K step s
#define W_DSR(RA, RB, t, buf, s)                                                       \
  do {                                                                                 \
    if ((t) < MW)                                                                      \
      RA[(t) % MW] = *reinterpret_cast<const bf16x8_t*>(As + (buf) * STAGE + a_rd +    \
                                                        ((t) % MW) * 32 * LDS_LD + (s) * 16); \
    else                                                                               \
      RB[((t) - MW) % NJ] = *reinterpret_cast<const bf16x8_t*>(                        \
          Bs + (buf) * STAGE + b_rd[((t) - MW) % NJ] + (s) * 16);                      \
  } while (0)
#define W_MFMA(RA, RB, t)                                                              \
  acc[(t) / NJ][(t) % NJ] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(                   \
      RA[(t) / NJ], RB[(t) % NJ], acc[(t) / NJ][(t) % NJ], 0, 0, 0)
  // One K step: the MFMAs on (RA, RB); between them, in issue order, the operand reads of
  // the following step into (NA, NB), and, for the staged chunks io_lo .. io_hi - 1 of ring
  // slot rs, the LDS write of each chunk followed by the global load that refills it.  The
  // reads go into the step's first MFMA slots and the chunks spread evenly over the slots
  // after them (over all slots when those are too few), so that the LDS does not take
  // writes and reads in the same stretch of MFMAs (2 % faster than writes spread over all
  // slots, 3-4 % faster than all writes in one step).
#define W_SLOT(i, n) (NS - NRD >= (n) ? NRD + (i) * (NS - NRD) / (n) : (i) * NS / (n))
#define W_STEP(RA, RB, NA, NB, rd_buf, rd_s, DO_RD, io_lo, io_hi, wbuf, gk0, rs)         \
  do {                                                                                 \
    _Pragma("unroll") for (int t = 0; t < NS; ++t) {                                   \
      if (t < NMF) W_MFMA(RA, RB, t);                                                  \
      if ((DO_RD) && t < NRD) W_DSR(NA, NB, t, rd_buf, rd_s);                          \
      _Pragma("unroll") for (int c = (io_lo); c < (io_hi); ++c) {                      \
        if (W_SLOT(c - (io_lo), (io_hi) - (io_lo)) == t) {                            \
          W_DSW(c, wbuf, rs);                                                          \
          W_GLD(c, gk0, rs);                                                           \
        }                                                                              \
      }                                                                                \
      __builtin_amdgcn_sched_barrier(0);                                               \
    }                                                                                  \
  } while (0)
  // K iteration kt computes stage kt from LDS buffer kt & 1.  Stage s >= 1 waits in ring
  // slot s % RING from its global load, issued RING iterations ahead, until iteration
  // s - 1 writes it to LDS buffer s & 1 and reuses the slot for stage s + RING (past the
  // last stage the load repeats the last stage and is never used).  Buffer kt & 1 ^ 1 is
  // free from the barrier that ended iteration kt - 1, so the stage's LDS writes (64 KB per
  // full tile) are spread over the three steps before this iteration's barrier: in one step
  // they would ask the LDS for about 1.5 times what it moves during that step's MFMAs, on
  // top of the operand reads.  Step 3's MFMAs run after the barrier that publishes stage
  // kt + 1, overlapping the first operand reads.  With a K tail (!KFULL) the writes stay in
  // the last step before the barrier: spread, the tail checks' live ranges spill registers.
  constexpr int IO1 = KFULL ? NLD / 3 : 0, IO2 = KFULL ? (2 * NLD) / 3 : 0;
#define W_ITER(rs)                                                                     \
  do {                                                                                 \
    const int cur = kt & 1;                                                            \
    const int gk_ = min(kt + 1 + RING, nk - 1) * BK;                                   \
    W_STEP(pa, pb, qa, qb, cur, 1, true, 0, IO1, cur ^ 1, gk_, rs);                    \
    W_STEP(qa, qb, pa, pb, cur, 2, true, IO1, IO2, cur ^ 1, gk_, rs);                  \
    W_STEP(pa, pb, qa, qb, cur, 3, true, IO2, NLD, cur ^ 1, gk_, rs);                  \
    __syncthreads();                                                                   \
    W_STEP(qa, qb, pa, pb, cur ^ 1, 0, true, 0, 0, 0, 0, 0);                           \
  } while (0)

  const int nk = (K + BK - 1) / BK;
#pragma unroll
  for (int t = 0; t < NLD; ++t) W_GLD(t, 0, 0);
#pragma unroll
  for (int t = 0; t < NLD; ++t) W_DSW(t, 0, 0);
#pragma unroll
  for (int t = 0; t < NLD; ++t) W_GLD(t, min(1, nk - 1) * BK, 1);
#pragma unroll
  for (int t = 0; t < NLD; ++t) W_GLD(t, min(2, nk - 1) * BK, 0);
  __syncthreads();
#pragma unroll
  for (int t = 0; t < NRD; ++t) W_DSR(pa, pb, t, 0, 0);

  int kt = 0;
  while (kt + 2 < nk) {
    W_ITER(1);
    ++kt;
    W_ITER(0);
    ++kt;
  }
  if (kt + 1 < nk) {
    W_ITER(1);
    ++kt;
  }
  // last stage: no LDS writes or loads left
  {
    const int cur = kt & 1;
    W_STEP(pa, pb, qa, qb, cur, 1, true, 0, 0, 0, 0, 0);
    W_STEP(qa, qb, pa, pb, cur, 2, true, 0, 0, 0, 0, 0);
    W_STEP(pa, pb, qa, qb, cur, 3, true, 0, 0, 0, 0, 0);
    W_STEP(qa, qb, pa, pb, 0, 0, false, 0, 0, 0, 0, 0);
  }
#undef W_ITER
#undef W_GLD
#undef W_DSW
#undef W_DSR
#undef W_MFMA
#undef W_STEP
#undef W_SLOT

  // epilogue: element q of a 32x32 block sits at row (q/4)*8 + (lane/32)*4 + q%4, column
  // lane%32.  Offsets run from this lane's first output; a wave whose rows and columns all
  // lie inside the tile and N (every full tile of an R1 layer) stores without checks.
  constexpr int NO = DUAL ? NJ / 2 : NJ;  // 32-column output blocks per wave
  const int r0 = wm0 + (lane >> 5) * 4;
  const int cw = n0 + (MI ? (DUAL ? wave * 32 : wave * 64) : (DUAL ? wn * 64 : wn * 128));
  const int64_t o0 = static_cast<int64_t>(tile.row0 + r0) * ldo + cw + lrow;
  using OutT = typename std::conditional<DUAL || OUT_BF16, uint16_t, float>::type;
  OutT* const obase = static_cast<OutT*>(out) + o0;
#define W_EPI(CHECK)                                                                   \
  do {                                                                                 \
    _Pragma("unroll") for (int i = 0; i < MW; ++i)                                     \
    _Pragma("unroll") for (int q = 0; q < 16; ++q) {                                   \
      const int dr = i * 32 + (q >> 2) * 8 + (q & 3);                                  \
      if ((CHECK) && r0 + dr >= tile.rows) continue;                                   \
      OutT* const orow = obase + static_cast<int64_t>(dr) * ldo;                      \
      _Pragma("unroll") for (int j = 0; j < NO; ++j) {                                 \
        if ((CHECK) && cw + j * 32 + lrow >= N) continue;                              \
        const float v = DUAL ? silu_f32(acc[i][j][q]) * acc[i][NO + j][q] : acc[i][j][q]; \
        if constexpr (DUAL || OUT_BF16) __builtin_nontemporal_store(f32_to_bf16(v), orow + j * 32); \
        else __builtin_nontemporal_store(v, orow + j * 32);                            \
      }                                                                                \
    }                                                                                  \
  } while (0)
  if constexpr (COMB) {
    // y[a / k] += w[a] * row, one float atomic per element (the k rows of a token sit in k
    // different experts' tiles, so no tile owns a token's sum)
    _Pragma("unroll") for (int i = 0; i < MW; ++i)
    _Pragma("unroll") for (int q = 0; q < 16; ++q) {
      const int dr = i * 32 + (q >> 2) * 8 + (q & 3);
      if (r0 + dr >= tile.rows) continue;
      const int a = sc.src_of[tile.row0 + r0 + dr];
      const float wa = sc.w[a];
      float* const yrow = sc.y + static_cast<int64_t>(a / sc.k) * ldo + cw + lrow;
      _Pragma("unroll") for (int j = 0; j < NO; ++j) {
        if (cw + j * 32 + lrow >= N) continue;
        unsafeAtomicAdd(yrow + j * 32, wa * acc[i][j][q]);
      }
    }
    return;
  }
  if (wm0 + MW * 32 <= tile.rows && cw + NO * 32 <= N)
    W_EPI(false);
  else
    W_EPI(true);
#undef W_EPI
}

template <bool DUAL, bool OUT_BF16, bool KFULL, bool COMB>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1))) void gemm_wide_kernel(
    const uint16_t* __restrict__ A, int lda, const int32_t* __restrict__ a_index, int a_div,
    const char* __restrict__ wbase, int64_t expert_bytes,
    int64_t b0_off, int64_t b1_off, int N, int K, const Tile* __restrict__ tiles,
    const int32_t* __restrict__ n_tiles, int dense_M, void* __restrict__ out, int ldo,
    Scatter sc) {
  constexpr int BM = kWideBM;
  constexpr int OUTN = DUAL ? kWideBN / 2 : kWideBN;

  // heavy (MFMA-bound) and light (weight-streaming) tiles, each list cut into groups of
  // kMGroup; group position gp holds a heavy group when the count of heavy groups up to
  // it, floor((gp + 1) F / G), steps up, so the F heavy groups spread evenly over all G
  const int n_heavy = tiles ? n_tiles[1] : (dense_M + BM - 1) / BM;
  const int n_light = tiles ? n_tiles[2] : 0;
  const int n_n = (N + OUTN - 1) / OUTN;
  const int F = (n_heavy + kMGroup - 1) / kMGroup, P = (n_light + kMGroup - 1) / kMGroup;
  const int G = F + P;
  const int per_group = n_n * kMGroup;
  const int xcd = blockIdx.x % kXcds, local = blockIdx.x / kXcds;
  const int gp = (local / per_group) * kXcds + xcd;
  if (gp >= G) return;
  const int64_t c0 = static_cast<int64_t>(gp) * F / G, c1 = static_cast<int64_t>(gp + 1) * F / G;
  const bool heavy = c1 > c0;
  const int gi = heavy ? static_cast<int>(c0) : gp - static_cast<int>(c1);
  const int first = heavy ? gi * kMGroup : n_heavy + gi * kMGroup;
  const int gsize = min(kMGroup, (heavy ? n_heavy : n_light) - gi * kMGroup);
  const int rem = local % per_group;
  if (rem >= gsize * n_n) return;
  int nt = rem / gsize;
  int mt = first + rem % gsize;
  // a run of 4 (else 2) aligned heavy groups of one expert: the same blocks per group,
  // span * kMGroup m-tiles by n_n / span n-tiles each (every group of the run takes the
  // same branch, so the run's tiles are still covered exactly once)
  if (tiles && heavy) {
    for (int span = 4; span >= 2; span >>= 1) {
      if (n_n % span) continue;
      const int pb = (gi & ~(span - 1)) * kMGroup;
      if (pb + span * kMGroup <= n_heavy &&
          tiles[pb].expert == tiles[pb + span * kMGroup - 1].expert) {
        nt = (gi & (span - 1)) * (n_n / span) + rem / (span * kMGroup);
        mt = pb + rem % (span * kMGroup);
        break;
      }
    }
  }

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
  const char* wexp = wbase + static_cast<int64_t>(tile.slot) * expert_bytes;
  const uint16_t* B0 = reinterpret_cast<const uint16_t*>(wexp + b0_off);
  const uint16_t* B1 = reinterpret_cast<const uint16_t*>(wexp + b1_off);
  if (tile.rows > 192)
    wide_tile<DUAL, OUT_BF16, KFULL, 0, COMB>(tile, n0, A, lda, a_index, a_div, B0, B1, N, K, out, ldo, smem, sc);
  else if (tile.rows > 128)
    wide_tile<DUAL, OUT_BF16, KFULL, 6, COMB>(tile, n0, A, lda, a_index, a_div, B0, B1, N, K, out, ldo, smem, sc);
  else if (tile.rows > 64)
    wide_tile<DUAL, OUT_BF16, KFULL, 4, COMB>(tile, n0, A, lda, a_index, a_div, B0, B1, N, K, out, ldo, smem, sc);
  else if (tile.rows > 32)
    wide_tile<DUAL, OUT_BF16, KFULL, 2, COMB>(tile, n0, A, lda, a_index, a_div, B0, B1, N, K, out, ldo, smem, sc);
  else
    wide_tile<DUAL, OUT_BF16, KFULL, 1, COMB>(tile, n0, A, lda, a_index, a_div, B0, B1, N, K, out, ldo, smem, sc);
}

template <bool DUAL, bool OUT_BF16, bool COMB = false>
struct GemmWide {
  static constexpr int BM = kWideBM;
  static constexpr size_t kLds =
      2 * static_cast<size_t>(kWideBM + kWideBN) * kWideLd * sizeof(uint16_t);

  // grid_m: upper bound on the number of m-tiles
  static int launch(const uint16_t* A, int lda, const int32_t* a_index, int a_div,
                    const char* wbase, int64_t expert_bytes,
                    int64_t b0_off, int64_t b1_off, int N, int K, const Tile* tiles,
                    const int32_t* n_tiles, int64_t grid_m, int dense_M, void* out, int ldo,
                    hipStream_t s, Scatter sc = Scatter{nullptr, nullptr, 1, nullptr}) {
    auto kern = K % 64 == 0 ? gemm_wide_kernel<DUAL, OUT_BF16, true, COMB>
                            : gemm_wide_kernel<DUAL, OUT_BF16, false, COMB>;
    // the dynamic-LDS limit above 64 KB is set on every launch: it is a cheap host call
    // and, unlike a once-per-process flag, holds for every device and thread
    MOE_HIP_CHECK(hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                      hipFuncAttributeMaxDynamicSharedMemorySize,
                                      static_cast<int>(kLds)));
    if (grid_m <= 0) return MOE_OK;
    const int outn = DUAL ? 128 : 256;
    // heavy and light groups: at most one more group than one list of grid_m tiles
    const int64_t groups = ceil_div64(grid_m, kMGroup) + 1;
    const int64_t blocks = ceil_div64(groups, kXcds) * kXcds * kMGroup * ceil_div(N, outn);
    hipLaunchKernelGGL(kern, dim3(static_cast<unsigned>(blocks)), dim3(256), kLds, s, A, lda, a_index,
                       a_div, wbase, expert_bytes, b0_off, b1_off, N, K, tiles, n_tiles, dense_M,
                       out, ldo, sc);
    MOE_LAUNCH_CHECK("gemm_wide_kernel launch");
    return MOE_OK;
  }
};

// ---------------------------------------------------------------------------
// Decode tile GEMM: a tile holds at most 16 rows, so each weight element feeds
// exactly one MFMA and the kernel is a weight stream.  No LDS and no barriers:
// every wave streams its own weight rows straight into registers in the MFMA
// operand layout (lane l: row l % 16, the 8 K values 8 (l / 16) .. +8 of each
// 32-deep MFMA step), so one load instruction reads 64 contiguous bytes of
// each of 16 rows.  K is consumed in 128-deep superblocks of four MFMA steps,
// two superblocks in flight per wave (ping-pong register sets).
//   DUAL: a wave owns 16 output columns (1 gate + 1 up 16-column MFMA block);
//   !DUAL: 32 output columns (2 blocks).  Four waves per block.  At 140-144 registers
//   three waves fit per SIMD (with 4 blocks per wave, two), which streams 2-3 % faster;
//   8 blocks, or 64- or 256-deep stages, measured the same or slower.
// Grid: x = column block, y = tile, so an expert's column blocks are dispatched one
// after another (round-robin over the XCDs) and the chip streams a few experts' weight
// matrices at a time in long contiguous runs (2-3 % faster than tiles fastest).
// ---------------------------------------------------------------------------

//   NB  16-column MFMA blocks per wave (DUAL: NB / 2 gate + NB / 2 up blocks)
//   KS  32-deep MFMA steps per register stage
template <bool DUAL, bool KFULL, int NB, int KS, bool COMB>
__global__ __launch_bounds__(256) void gemm_stream_kernel(
    const uint16_t* __restrict__ A, int lda, const int32_t* __restrict__ a_index, int a_div,
    const char* __restrict__ wbase, int64_t expert_bytes, int64_t b0_off, int64_t b1_off, int N,
    int K, const Tile* __restrict__ tiles, const int32_t* __restrict__ n_tiles,
    void* __restrict__ out, int ldo, Scatter sc) {
  static_assert(!COMB || !DUAL, "the combine runs in the down GEMM");
  constexpr int WCOLS = DUAL ? NB * 8 : NB * 16;
  constexpr int BCOLS = 4 * WCOLS;
  constexpr int SK = 32 * KS;  // K depth of one register stage
  static_assert(!DUAL || NB % 2 == 0, "gate and up blocks come in pairs");
  if (static_cast<int>(blockIdx.y) >= *n_tiles) return;
  const Tile tile = tiles[blockIdx.y];
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int c0 = blockIdx.x * BCOLS + wave * WCOLS;
  if (c0 >= N) return;
  const int lr = lane & 15, lg = lane >> 4;

  // A row of this lane (rows past the tile read the tile's first row; never stored)
  int src = tile.row0 + (lr < tile.rows ? lr : 0);
  if (a_index) src = a_index[src] / a_div;
  const uint16_t* arow = A + static_cast<int64_t>(src) * lda + lg * 8;
  const char* wexp = wbase + static_cast<int64_t>(tile.slot) * expert_bytes;
  const uint16_t* B0 = reinterpret_cast<const uint16_t*>(wexp + b0_off);
  const uint16_t* B1 = reinterpret_cast<const uint16_t*>(wexp + b1_off);
  const uint16_t* brow[NB];
#pragma unroll
  for (int j = 0; j < NB; ++j) {
    const int jj = DUAL ? j % (NB / 2) : j;
    const int n = c0 + jj * 16 + lr;
    const uint16_t* Bm = (DUAL && j >= NB / 2) ? B1 : B0;
    brow[j] = Bm + static_cast<int64_t>(n < N ? n : 0) * K + lg * 8;
  }

  floatx4 acc[NB];
#pragma unroll
  for (int j = 0; j < NB; ++j) acc[j] = floatx4{0.f, 0.f, 0.f, 0.f};

  uint4 a0[KS], b0[NB][KS], a1[KS], b1[NB][KS];
#define STREAM_LOAD(AR, BR, k0)                                                                   \
  do {                                                                                            \
    _Pragma("unroll") for (int c = 0; c < KS; ++c) {                                              \
      const bool in = KFULL || (k0) + c * 32 + lg * 8 < K;                                        \
      AR[c] = make_uint4(0, 0, 0, 0);                                                             \
      if (in) AR[c] = *reinterpret_cast<const uint4*>(arow + (k0) + c * 32);                      \
      _Pragma("unroll") for (int j = 0; j < NB; ++j) {                                            \
        BR[j][c] = make_uint4(0, 0, 0, 0);                                                        \
        if (in) BR[j][c] = *reinterpret_cast<const uint4*>(brow[j] + (k0) + c * 32);              \
      }                                                                                           \
    }                                                                                             \
  } while (0)
#define STREAM_MFMA(AR, BR)                                                                       \
  do {                                                                                            \
    _Pragma("unroll") for (int c = 0; c < KS; ++c) {                                              \
      const bf16x8_t a = __builtin_bit_cast(bf16x8_t, AR[c]);                                     \
      _Pragma("unroll") for (int j = 0; j < NB; ++j)                                              \
        acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(                                         \
            a, __builtin_bit_cast(bf16x8_t, BR[j][c]), acc[j], 0, 0, 0);                          \
    }                                                                                             \
  } while (0)

  const int nsb = (K + SK - 1) / SK;
  STREAM_LOAD(a0, b0, 0);
  for (int sb = 0; sb < nsb; sb += 2) {
    if (sb + 1 < nsb) STREAM_LOAD(a1, b1, (sb + 1) * SK);
    STREAM_MFMA(a0, b0);
    if (sb + 1 >= nsb) break;
    if (sb + 2 < nsb) STREAM_LOAD(a0, b0, (sb + 2) * SK);
    STREAM_MFMA(a1, b1);
  }
#undef STREAM_LOAD
#undef STREAM_MFMA

  // lane holds C[(lane / 16) * 4 + q][lane % 16] of each 16x16 block
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int r = lg * 4 + q;
    if (r >= tile.rows) continue;
    const int64_t orow = static_cast<int64_t>(tile.row0 + r) * ldo;
    if (DUAL) {
#pragma unroll
      for (int jj = 0; jj < NB / 2; ++jj) {
        const int n = c0 + jj * 16 + lr;
        if (n < N)
          static_cast<uint16_t*>(out)[orow + n] =
              f32_to_bf16(silu_f32(acc[jj][q]) * acc[NB / 2 + jj][q]);
      }
    } else if (COMB) {
      // y[a / k] += w[a] * row (the combine folded into the epilogue)
      const int a = sc.src_of[tile.row0 + r];
      const float wa = sc.w[a];
      float* const yrow = sc.y + static_cast<int64_t>(a / sc.k) * ldo;
#pragma unroll
      for (int j = 0; j < NB; ++j) {
        const int n = c0 + j * 16 + lr;
        if (n < N) unsafeAtomicAdd(yrow + n, wa * acc[j][q]);
      }
    } else {
#pragma unroll
      for (int j = 0; j < NB; ++j) {
        const int n = c0 + j * 16 + lr;
        if (n < N) static_cast<float*>(out)[orow + n] = acc[j][q];
      }
    }
  }
}

template <bool DUAL, int NB, int KS, bool COMB = false>
struct GemmStream {
  static constexpr int BM = 16;
  static constexpr int BCOLS = 4 * (DUAL ? NB * 8 : NB * 16);
  static int launch(const uint16_t* A, int lda, const int32_t* a_index, int a_div,
                    const char* wbase, int64_t expert_bytes, int64_t b0_off, int64_t b1_off, int N,
                    int K, const Tile* tiles, const int32_t* n_tiles, int64_t grid_tiles, void* out,
                    int ldo, hipStream_t s, Scatter sc = Scatter{nullptr, nullptr, 1, nullptr}) {
    if (grid_tiles <= 0) return MOE_OK;
    dim3 grid(static_cast<unsigned>(ceil_div(N, BCOLS)), static_cast<unsigned>(grid_tiles));
    if (K % (32 * KS) == 0)
      hipLaunchKernelGGL((gemm_stream_kernel<DUAL, true, NB, KS, COMB>), grid, dim3(256), 0, s, A,
                         lda, a_index, a_div, wbase, expert_bytes, b0_off, b1_off, N, K, tiles,
                         n_tiles, out, ldo, sc);
    else
      hipLaunchKernelGGL((gemm_stream_kernel<DUAL, false, NB, KS, COMB>), grid, dim3(256), 0, s, A,
                         lda, a_index, a_div, wbase, expert_bytes, b0_off, b1_off, N, K, tiles,
                         n_tiles, out, ldo, sc);
    MOE_LAUNCH_CHECK("gemm_stream_kernel launch");
    return MOE_OK;
  }
};

// decode shapes: gate/up with 2 + 2 blocks per wave, down with 4, 128-deep stages
using Gemm1Stream = GemmStream<true, 2, 4>;
using Gemm2Stream = GemmStream<false, 2, 4>;
using Gemm2StreamComb = GemmStream<false, 2, 4, true>;

// prefill shapes: 256-row tiles
using Gemm1Prefill = GemmWide<true, false>;
using Gemm2Prefill = GemmWide<false, false>;
using Gemm2PrefillComb = GemmWide<false, false, true>;
using DenseBf16 = GemmWide<false, true>;

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
                                                        int n_slots,
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
  if (slot < 0 || slot >= n_slots) {
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
                                                        int n_slots,
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
  if (slot < 0 || slot >= n_slots) return;
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
__global__ __launch_bounds__(256) void zero_f32_kernel(float* __restrict__ p, int64_t n) {
  const int64_t step = static_cast<int64_t>(gridDim.x) * blockDim.x;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n; i += step)
    p[i] = 0.f;
}

// sc (optional): the combine folded into the down GEMM (y_perm is then not written).
int grouped_swiglu_impl(const void* x_perm, const int32_t* a_index, int a_div,
                        const int32_t* offsets, int R, int E, int H, int I, moe_dtype dtype,
                        const moe_wbuf* w, int e_begin, int e_end, void* ws, size_t ws_bytes,
                        float* y_perm, int32_t* status, moe_stream_t stream,
                        const Scatter* sc = nullptr) {
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
  if (static_cast<int64_t>(H) * I >= (int64_t{1} << 31))
    return fail(MOE_ERR_UNSUPPORTED, "moe_grouped_swiglu: H*I=%lld is 2^31 or more",
                static_cast<long long>(H) * I);
  if (dtype == MOE_BF16 && (H % 8 != 0 || I % 8 != 0))
    return fail(MOE_ERR_UNSUPPORTED, "moe_grouped_swiglu: H=%d and I=%d must be multiples of 8", H, I);
  const SwigluWs L = swiglu_ws(R, E, I, dtype);
  if (!ws || ws_bytes < L.total)
    return fail(MOE_ERR_WORKSPACE, "moe_grouped_swiglu: workspace %zu < %zu bytes", ws_bytes, L.total);
  if (R == 0) return MOE_OK;
  if (!x_perm || (!y_perm && !sc)) return fail(MOE_ERR_ARG, "moe_grouped_swiglu: null pointer");

  hipStream_t s = as_stream(stream);
  char* wsb = static_cast<char*>(ws);
  void* h = wsb;
  const char* wbase = static_cast<const char*>(w->base);

  if (dtype == MOE_F32) {
    const int64_t n1 = static_cast<int64_t>(R) * I, n2 = static_cast<int64_t>(R) * H;
    hipLaunchKernelGGL(gemm1_f32_kernel, dim3(static_cast<unsigned>(ceil_div64(n1, 256))), dim3(256),
                       0, s, static_cast<const float*>(x_perm), a_index, a_div, offsets, E,
                       e_begin, e_end,
                       w->slot_of, w->n_slots, wbase, eb, H, I, static_cast<float*>(h), status);
    MOE_LAUNCH_CHECK("moe_grouped_swiglu: gemm1 f32");
    hipLaunchKernelGGL(gemm2_f32_kernel, dim3(static_cast<unsigned>(ceil_div64(n2, 256))), dim3(256),
                       0, s, static_cast<const float*>(h), offsets, E, e_begin, e_end, w->slot_of,
                       w->n_slots, wbase, eb, H, I, y_perm);
    MOE_LAUNCH_CHECK("moe_grouped_swiglu: gemm2 f32");
    return MOE_OK;
  }

  Tile* tiles = reinterpret_cast<Tile*>(wsb + L.tiles_off);
  int32_t* n_tiles = reinterpret_cast<int32_t*>(wsb + L.count_off);
  const bool decode = static_cast<int64_t>(R) <= 4 * static_cast<int64_t>(E);
  if (!decode && a_index &&
      (static_cast<int64_t>(R) / a_div + 1) * H * 2 >= (int64_t{1} << 32))
    return fail(MOE_ERR_UNSUPPORTED, "moe_grouped_swiglu_gathered: x of %lld rows x %d is 4 GiB "
                "or more", static_cast<long long>(R) / a_div + 1, H);
  const int BM = decode ? 16 : Gemm1Prefill::BM;
  const int64_t grid_tiles = ceil_div64(R, BM) + std::min(E, R);
  if (sc) {
    // y is accumulated into: clear it on the stream first (a kernel, so the call can be
    // captured into a graph)
    const int64_t n = static_cast<int64_t>(R / sc->k) * H;
    hipLaunchKernelGGL(zero_f32_kernel,
                       dim3(static_cast<unsigned>(std::min<int64_t>(ceil_div64(n, 256), 65536))),
                       dim3(256), 0, s, sc->y, n);
    MOE_LAUNCH_CHECK("moe_grouped_swiglu_combine: clear y");
  }
  hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(MOE_MAX_E), 0, s, offsets, E, e_begin, e_end, BM,
                     w->slot_of, w->n_slots, tiles, n_tiles, status);
  MOE_LAUNCH_CHECK("moe_grouped_swiglu: plan");

  const int64_t HI2 = static_cast<int64_t>(H) * I * 2;  // bytes of one H x I bf16 matrix
  const uint16_t* xp = static_cast<const uint16_t*>(x_perm);
  const uint16_t* hp = static_cast<const uint16_t*>(h);
  int rc;
  if (decode) {
    rc = Gemm1Stream::launch(xp, H, a_index, a_div, wbase, eb, 0, HI2, I, H, tiles, n_tiles,
                                  grid_tiles, h, I, s);
    if (rc) return rc;
    if (sc)
      rc = Gemm2StreamComb::launch(hp, I, nullptr, 1, wbase, eb, 2 * HI2, 0, H, I, tiles, n_tiles,
                                   grid_tiles, nullptr, H, s, *sc);
    else
      rc = Gemm2Stream::launch(hp, I, nullptr, 1, wbase, eb, 2 * HI2, 0, H, I, tiles, n_tiles,
                               grid_tiles, y_perm, H, s);
  } else {
    rc = Gemm1Prefill::launch(xp, H, a_index, a_div, wbase, eb, 0, HI2, I, H, tiles, n_tiles,
                              grid_tiles, 0, h, I, s);
    if (rc) return rc;
    if (sc)
      rc = Gemm2PrefillComb::launch(hp, I, nullptr, 1, wbase, eb, 2 * HI2, 0, H, I, tiles, n_tiles,
                                    grid_tiles, 0, nullptr, H, s, *sc);
    else
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
  const int rc = moe::grouped_swiglu_impl(x_perm, nullptr, 1, offsets, R, E, H, I, dtype, w,
                                          e_begin, e_end, ws, ws_bytes, y_perm, status, stream);
  return moe::debug_check(rc, "moe_grouped_swiglu_range", moe::as_stream(stream), status);
}

extern "C" int moe_grouped_swiglu_gathered(const void* x, const int32_t* src_of, int k,
                                           const int32_t* offsets, int R, int E, int H, int I,
                                           moe_dtype dtype, const moe_wbuf* w, int e_begin,
                                           int e_end, void* ws, size_t ws_bytes, float* y_perm,
                                           int32_t* status, moe_stream_t stream) {
  using namespace moe;
  if (k < 1) return fail(MOE_ERR_ARG, "moe_grouped_swiglu_gathered: k=%d", k);
  if (R > 0 && !src_of) return fail(MOE_ERR_ARG, "moe_grouped_swiglu_gathered: null src_of");
  const int rc = grouped_swiglu_impl(x, src_of, k, offsets, R, E, H, I, dtype, w, e_begin, e_end,
                                     ws, ws_bytes, y_perm, status, stream);
  return debug_check(rc, "moe_grouped_swiglu_gathered", as_stream(stream), status);
}


extern "C" int moe_grouped_swiglu_combine(const void* x, const int32_t* src_of,
                                          const float* topk_w, int T, int k,
                                          const int32_t* offsets, int E, int H, int I,
                                          moe_dtype dtype, const moe_wbuf* w, void* ws,
                                          size_t ws_bytes, float* y, int32_t* status,
                                          moe_stream_t stream) {
  using namespace moe;
  if (T < 0 || k < 1) return fail(MOE_ERR_ARG, "moe_grouped_swiglu_combine: T=%d k=%d", T, k);
  if (dtype != MOE_BF16)
    return fail(MOE_ERR_UNSUPPORTED, "moe_grouped_swiglu_combine: bf16 weights only");
  const int64_t R64 = static_cast<int64_t>(T) * k;
  if (R64 > INT32_MAX) return fail(MOE_ERR_UNSUPPORTED, "moe_grouped_swiglu_combine: T*k too large");
  const int R = static_cast<int>(R64);
  if (T > 0 && (!y || !src_of || !topk_w))
    return fail(MOE_ERR_ARG, "moe_grouped_swiglu_combine: null pointer");
  const Scatter sc{src_of, topk_w, k, y};
  const int rc = grouped_swiglu_impl(x, src_of, k, offsets, R, E, H, I, dtype, w, 0, E, ws,
                                     ws_bytes, nullptr, status, stream, &sc);
  return debug_check(rc, "moe_grouped_swiglu_combine", as_stream(stream), status);
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
  if (static_cast<int64_t>(N) * K >= (int64_t{1} << 31))
    return fail(MOE_ERR_UNSUPPORTED, "moe_dense_gemm: N*K=%lld is 2^31 or more",
                static_cast<long long>(N) * K);
  if (M == 0) return MOE_OK;
  if (!x || !w || !out) return fail(MOE_ERR_ARG, "moe_dense_gemm: null pointer");
  const int rc = DenseBf16::launch(static_cast<const uint16_t*>(x), K, nullptr, 1,
                                   static_cast<const char*>(w), 0, 0, 0, N, K, nullptr, nullptr,
                                   ceil_div(M, DenseBf16::BM), M, out, N, as_stream(stream));
  return debug_check(rc, "moe_dense_gemm", as_stream(stream), nullptr);
}
