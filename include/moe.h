/*
 * moe.h -- C ABI of the DWDP-style MoE layer forward on one MI355X (gfx950).
 *
 * The layer follows the pattern of "DWDP: Distributed Weight Data Parallelism
 * for High-Performance LLM Inference on NVL72" (arXiv 2604.01621v1, abstract)
 * and its explainer (viz: "Distributed Weight Data Parallelism cuts LLM
 * inference stalls"): every GPU stays data-parallel and holds a share of the
 * MoE experts; the missing ("remote") experts are pulled on a copy engine into
 * an alternate buffer while compute runs ("stay data-parallel" and
 * prefetch-schedule panels), and local plus remote weights reach the grouped
 * GEMM as one contiguous buffer (contiguous-buffer panel).  On one GPU the
 * peers' share is a separate device pool (or pinned host memory).
 *
 * The pages do not define the MoE layer's arithmetic; the library computes the
 * plain top-k softmax-gated mixture of SwiGLU experts: route -> permute ->
 * grouped SwiGLU -> combine, with the weight merge and prefetch in between.
 *
 * Conventions shared by every call
 * --------------------------------
 * - Pointers named *_host are host memory; every other pointer is device
 *   memory (or pinned host memory where stated).  The caller owns all memory,
 *   streams and events; the library allocates nothing (the moe_vmm_* set-up
 *   calls excepted, whose purpose is to allocate) and keeps no state except
 *   the thread-local text returned by moe_last_error().
 * - Every call only enqueues work on the stream it is given and returns; none
 *   synchronises the device.  A return value < 0 means nothing was enqueued
 *   (MOE_ERR_ARG, MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE) or a HIP call failed
 *   part-way (MOE_ERR_HIP); moe_last_error() then holds a description.
 * - Data errors found on the device set bits of a caller-provided int32
 *   status word (MOE_STATUS_*), which the caller reads after a sync.  The
 *   kernels only OR bits into it; the caller clears it.
 * - Sizes are int (T, E, k, H, I, R = T*k all < 2^31); byte counts are
 *   int64_t / size_t.
 *
 * Layouts
 * -------
 * - logits  f32[T][E], row-major.
 * - x       [T][H] row-major, f32 (MOE_F32) or bf16 (MOE_BF16).
 * - topk_idx i32[T][k], topk_w f32[T][k]: slot j of token t is assignment
 *   a = t*k + j.
 * - Expert block (one expert, row-major, dtype elements, output-major):
 *     [ Wg : I rows x H cols ][ Wu : I rows x H cols ][ Wd : H rows x I cols ]
 *   so that g = x Wg^T, u = x Wu^T, y = h Wd^T.  expert_bytes = 3*H*I*elem.
 * - Permuted rows: the rows of expert e are [offsets[e], offsets[e+1]), in
 *   ascending assignment index (a stable counting sort by expert id).
 */
#ifndef MOE_H_
#define MOE_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef void* moe_stream_t; /* a hipStream_t; NULL is the null stream */
typedef void* moe_event_t;  /* a hipEvent_t */

typedef enum { MOE_F32 = 0, MOE_BF16 = 1 } moe_dtype;

enum {
  MOE_OK = 0,
  MOE_ERR_ARG = -1,         /* invalid argument; nothing enqueued */
  MOE_ERR_UNSUPPORTED = -2, /* valid, but outside what the kernels support; nothing enqueued */
  MOE_ERR_WORKSPACE = -3,   /* workspace missing or too small; nothing enqueued */
  MOE_ERR_HIP = -4,         /* a HIP runtime call failed; see moe_last_error() */
  MOE_ERR_STATUS = -5       /* debug mode only: the call's kernels set a status bit */
};

/*
 * Debug mode: with MOE_DEBUG_SYNC set in the environment (to anything but "" or "0"),
 * every call that enqueues work synchronises its stream before returning.  A kernel that
 * failed then returns MOE_ERR_HIP, and a set bit of the call's status word (when it takes
 * one) MOE_ERR_STATUS, each with a description in moe_last_error(); the failing call is
 * the one that returns.  Off by default: the calls then only enqueue.
 */

/* bits of the device status word */
#define MOE_STATUS_NONFINITE_LOGIT 1 /* a router logit was NaN or +-inf */
#define MOE_STATUS_EXPERT_ABSENT 2   /* a routed expert has no slot in the merged buffer */
#define MOE_STATUS_BAD_EXPERT_ID 4   /* a top-k id outside [0, E) reached the permutation */

/* copy-engine selection for moe_merge_weights / moe_prefetch_layer */
#define MOE_COPY_SDMA 0 /* device-to-device copies on the SDMA engines, no compute units */
#define MOE_COPY_ANY 1  /* let the runtime choose (it may use a copy kernel on the CUs) */
/* The library's own streaming copy kernel for device-to-device runs, on at most n
 * workgroups of 1024 threads (n = 0: as many as the copy can use).  A small n holds the
 * pull to at most n compute units at a time, leaving the rest to a grouped GEMM running
 * beside it (one workgroup per CU).  Each workgroup moves only ~20-25 GB/s, though, so on
 * MI355X the unbounded copy (n = 0) is the faster choice even beside a GEMM.  Host-memory
 * sources still use the runtime copy. */
#define MOE_COPY_KERNEL 2
#define MOE_COPY_KERNEL_ON(n) (MOE_COPY_KERNEL | ((n) << 8))

/* Limits of the kernels (MOE_ERR_UNSUPPORTED beyond them). */
#define MOE_MAX_E 1024
#define MOE_MAX_K 64

/*
 * A pool of consecutive experts [first_expert, first_expert + n_experts):
 * n_experts contiguous expert blocks of expert_bytes each, in device memory
 * or in pinned host memory.  The local pool is this rank's resident share;
 * the remote pool stands in for the peers' shares (DWDP abstract: MoE weights
 * are offloaded across peer GPUs and missing experts fetched on demand).
 * An empty pool (n_experts == 0: every expert local, or none) may have base NULL.
 */
typedef struct moe_pool {
  const void* base;
  int64_t expert_bytes;
  int32_t first_expert;
  int32_t n_experts;
} moe_pool;

/*
 * One half of the double buffer: n_slots expert blocks in ONE contiguous
 * device allocation (DWDP explainer, contiguous-buffer panel) plus the device
 * slot map slot_of[E] (slot of expert e, or -1) that the grouped GEMM reads.
 * The caller allocates base (n_slots * expert_bytes bytes) and slot_of
 * (E int32); the merge call writes slot_of on its stream.
 */
typedef struct moe_wbuf {
  void* base;
  int64_t expert_bytes;
  int32_t n_slots;
  int32_t n_experts; /* E: length of slot_of */
  int32_t* slot_of;  /* device int32[E] */
} moe_wbuf;

/*
 * moe_route -- top-k routing with weights renormalised over the chosen k.
 *
 * For each token t: topk_idx[t][0..k-1] are the k experts with the largest
 * logits, in order of (logit descending, expert id ascending), so +0 and -0
 * tie and ties go to the smaller id; topk_w[t][j] = exp(l_j - l_0) /
 * sum_{i<k} exp(l_i - l_0), which equals the softmax over all E experts
 * renormalised over the chosen k.  Routing exists on the pages only as the
 * "weight-level imbalance" its skew causes (DWDP explainer); the rule is the
 * plain top-k softmax gate.
 *   logits   device f32[T][E]          (read)
 *   topk_idx device i32[T][k]          (written)
 *   topk_w   device f32[T][k]          (written)
 *   status   device i32, may be NULL   (MOE_STATUS_NONFINITE_LOGIT is ORed in
 *            when a token has a non-finite logit; that token's outputs are
 *            then unspecified)
 * Errors: MOE_ERR_ARG for null outputs, T < 0, k < 1 or k > E;
 * MOE_ERR_UNSUPPORTED for E > MOE_MAX_E or k > MOE_MAX_K.  T = 0 is a no-op.
 */
int moe_route(const float* logits, int T, int E, int k, int32_t* topk_idx, float* topk_w,
              int32_t* status, moe_stream_t stream);

/* Workspace bytes moe_permute needs for (T, E, k). */
int moe_permute_workspace_size(int T, int E, int k, size_t* bytes);

/*
 * moe_permute -- counts, offsets, the stable expert-major permutation and the
 * row gather that put the tokens in expert-contiguous order for the grouped
 * GEMM (the grouped GEMM of the DWDP explainer's contiguous-buffer panel
 * consumes rows grouped by expert).
 *   topk_idx device i32[T*k]     (read; a = t*k + j)
 *   x        device [T][H] dtype (read)
 *   counts   device i32[E]       counts[e] = #assignments routed to e
 *   offsets  device i32[E+1]     exclusive prefix sum; offsets[E] = T*k
 *   row_of   device i32[T*k]     row of assignment a
 *   src_of   device i32[T*k]     assignment held by row r (src_of[row_of[a]] = a)
 *   x_perm   device [T*k][H] dtype, x_perm[r] = x[src_of[r] / k]; may be NULL
 *            to skip the gather
 *   ws       device workspace of moe_permute_workspace_size() bytes
 *   status   device i32, may be NULL (MOE_STATUS_BAD_EXPERT_ID for an id
 *            outside [0, E); such assignments are dropped and the outputs
 *            are then unspecified)
 * Errors: MOE_ERR_ARG for null required pointers or bad sizes;
 * MOE_ERR_WORKSPACE when ws_bytes is too small; MOE_ERR_UNSUPPORTED for
 * E > MOE_MAX_E.
 */
int moe_permute(const int32_t* topk_idx, int T, int E, int k, const void* x, int H,
                moe_dtype dtype, int32_t* counts, int32_t* offsets, int32_t* row_of,
                int32_t* src_of, void* x_perm, void* ws, size_t ws_bytes, int32_t* status,
                moe_stream_t stream);

/*
 * moe_permute_noalloc -- moe_permute with no workspace argument and no allocation, for
 * callers that cannot allocate device memory: code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc.  Its kernels use a file-scope device array of
 * 2 MiB (the most moe_permute's workspace can need for any T, k and E <= MOE_MAX_E) that
 * each GPU holds until the process ends; its address is looked up once per device.
 * Every call on a GPU shares that array: calls that overlap on one GPU (on different
 * streams, or from several threads) race and must be ordered by the caller.  Nothing in it
 * needs clearing: each call writes all of it that it reads.
 * Arguments and outputs: as moe_permute, without ws / ws_bytes.
 * Errors: as moe_permute; MOE_ERR_WORKSPACE if a size needed more than the array (not
 * reachable within the other limits); MOE_ERR_HIP if the array's address cannot be found.
 */
int moe_permute_noalloc(const int32_t* topk_idx, int T, int E, int k, const void* x, int H,
                        moe_dtype dtype, int32_t* counts, int32_t* offsets, int32_t* row_of,
                        int32_t* src_of, void* x_perm, int32_t* status, moe_stream_t stream);

/*
 * moe_merge_weights -- make the merged buffer: write the slot map for the
 * expert set ids_host (strictly ascending; slot = position in ids_host) and
 * copy every expert of that set that the local pool holds into its slot
 * (DWDP explainer, contiguous-buffer panel: local and remote expert weights
 * reach the grouped GEMM as one contiguous buffer; the copy is the
 * "buffer-merge overhead" of the iteration-latency panel).
 *   local     pool of this rank's resident experts (device or pinned host)
 *   ids_host  host i32[n_ids], read during the call only
 *   dst       merged buffer half; dst->slot_of is written on the stream
 *   wait_free if not NULL, the stream first waits for it (the last reader of
 *             this half is done)
 *   ready     if not NULL, recorded on the stream after the copies
 *   copy_mode MOE_COPY_SDMA, MOE_COPY_ANY or MOE_COPY_KERNEL_ON(n), n in [0, 65535]
 * Copies of consecutive ids in consecutive slots are coalesced, and a run
 * whose source bytes are its destination bytes is skipped: when the merged
 * range is stitched with the local-expert block at its head (moe_vmm_map
 * below) and that range is passed as the local pool, the merge copies nothing
 * and only writes the slot map.
 * Errors: MOE_ERR_ARG for unsorted or out-of-range ids, n_ids > n_slots,
 * mismatched expert_bytes or null pointers.
 */
int moe_merge_weights(const moe_pool* local, const int32_t* ids_host, int n_ids, moe_wbuf* dst,
                      moe_stream_t stream, moe_event_t wait_free, moe_event_t ready,
                      int copy_mode);

/*
 * moe_prefetch_layer -- pull the experts of ids_host that the remote pool
 * holds into their slots of dst (slot = position in ids_host, the same set
 * the merge of this half is given), asynchronously on copy_stream: the
 * one-GPU stand-in of the peer pull on the copy engine that fills the
 * alternate buffer while compute runs (DWDP explainer, "stay data-parallel"
 * and prefetch-schedule panels).  It does not write dst->slot_of.
 *   wait_free / ready / copy_mode as for moe_merge_weights.
 * Errors: as for moe_merge_weights.  For tests of a caller's error handling,
 * the environment variable MOE_INJECT_FAULT=prefetch makes the call return
 * MOE_ERR_HIP at once, with nothing enqueued (the ready event is not recorded).
 */
int moe_prefetch_layer(const moe_pool* remote, const int32_t* ids_host, int n_ids, moe_wbuf* dst,
                       moe_stream_t copy_stream, moe_event_t wait_free, moe_event_t ready,
                       int copy_mode);

/*
 * moe_prefetch_routed -- the routed pull with the expert set decided on the
 * device, so nothing is read back to the host between the routing and the
 * pull: on copy_stream, every expert e of the remote pool with counts[e] > 0
 * is copied into slot e of dst, and dst->slot_of[e] is set to e, or to -1 for
 * an expert with no tokens (whose slot keeps what it held).  The same pull
 * as moe_prefetch_layer (DWDP explainer, "stay data-parallel" and
 * prefetch-schedule panels) for the set that moe_permute's counts name.  The
 * slots of the experts outside the remote pool are the caller's: a
 * moe_merge_weights of ids 0 .. n_local - 1 before this call copies (or, for a
 * stitched half, maps) the local experts to slots 0 .. n_local - 1 and writes
 * -1 for every other expert.
 *   remote       pool of experts [first, first + n) in device memory; a pool
 *                in host memory is MOE_ERR_UNSUPPORTED (its pull stays on
 *                moe_prefetch_layer, whose copies the copy engine runs)
 *   counts       device i32[dst->n_experts], tokens per expert (moe_permute)
 *   dst          merged buffer half with n_slots >= first + n: slot = expert id
 *   counts_ready if not NULL, the stream first waits for it (the permute that
 *                writes counts is done)
 *   wait_free / ready as for moe_merge_weights
 *   max_blocks   bound on the copy's workgroups (0: the library's default)
 * Expert blocks and both bases must be 16-byte aligned (MOE_ERR_UNSUPPORTED
 * otherwise).  MOE_INJECT_FAULT=prefetch makes the call fail as for
 * moe_prefetch_layer.
 */
int moe_prefetch_routed(const moe_pool* remote, const int32_t* counts, moe_wbuf* dst,
                        moe_stream_t copy_stream, moe_event_t counts_ready,
                        moe_event_t wait_free, moe_event_t ready, int max_blocks);

/* Workspace bytes moe_grouped_swiglu needs for R = T*k rows. */
int moe_grouped_swiglu_workspace_size(int R, int E, int H, int I, moe_dtype dtype, size_t* bytes);

/*
 * moe_grouped_swiglu -- the grouped GEMM over the experts of the merged
 * buffer (DWDP explainer, contiguous-buffer panel), with the SwiGLU FFN of
 * each expert (Shazeer 2020, "GLU Variants Improve Transformer"):
 *   for the rows r of each expert e:  g = x_perm[r] Wg_e^T,  u = x_perm[r] Wu_e^T,
 *   h = silu(g) * u  (stored as bf16 for MOE_BF16, f32 for MOE_F32),
 *   y_perm[r] = h Wd_e^T  (always f32).
 * Accumulation is f32 (bf16 MFMA for MOE_BF16, f32 FMA for MOE_F32).
 *   x_perm  device [R][H] dtype
 *   offsets device i32[E+1] (from moe_permute)
 *   w       merged buffer; expert e is read at w->base + w->slot_of[e]*expert_bytes
 *   ws      device workspace of moe_grouped_swiglu_workspace_size() bytes
 *   y_perm  device f32[R][H]
 *   status  device i32, may be NULL (MOE_STATUS_EXPERT_ABSENT when an expert
 *           with rows has slot -1, or a slot outside [0, w->n_slots), which is
 *           never read; that expert's rows are then left unwritten)
 * Errors: MOE_ERR_ARG for null pointers or sizes that disagree with w;
 * MOE_ERR_UNSUPPORTED for E > MOE_MAX_E, H*I >= 2^31, or (MOE_BF16) H or I
 * not a multiple of 8; MOE_ERR_WORKSPACE when ws_bytes is too small.
 */
int moe_grouped_swiglu(const void* x_perm, const int32_t* offsets, int R, int E, int H, int I,
                       moe_dtype dtype, const moe_wbuf* w, void* ws, size_t ws_bytes,
                       float* y_perm, int32_t* status, moe_stream_t stream);

/*
 * moe_grouped_swiglu_range -- moe_grouped_swiglu restricted to the experts
 * [e_begin, e_end): only their rows of h and y_perm are written, the rows of
 * other experts are left untouched, and only their slots are read.  Lets the
 * compute stream start on the experts whose weights have arrived while the
 * copy stream is still pulling the rest (per-chunk readiness: one ready event
 * per chunk of the prefetch, each chunk's GEMM waiting only for its own
 * chunk).  Calls on one stream may share the workspace.
 * Errors: as moe_grouped_swiglu, plus MOE_ERR_ARG for a range outside [0, E].
 */
int moe_grouped_swiglu_range(const void* x_perm, const int32_t* offsets, int R, int E, int H, int I,
                             moe_dtype dtype, const moe_wbuf* w, int e_begin, int e_end, void* ws,
                             size_t ws_bytes, float* y_perm, int32_t* status, moe_stream_t stream);

/*
 * moe_grouped_swiglu_gathered -- moe_grouped_swiglu_range with the row gather
 * of moe_permute folded into the GEMM's operand loads: row r of the gate/up
 * GEMM is read from x[src_of[r] / k] instead of x_perm[r], so moe_permute may
 * be called with x_perm = NULL and the [T*k][H] copy is never written.
 *   x      device [T][H] dtype; src_of device i32[T*k] (from moe_permute); k >= 1
 *   other arguments as moe_grouped_swiglu_range.
 * Errors: as moe_grouped_swiglu_range, plus MOE_ERR_ARG for k < 1 or a null src_of,
 * and MOE_ERR_UNSUPPORTED when R > 4*E (prefill tiles) and x spans 4 GiB or more
 * ((R/k + 1) * H * 2 bytes): those tiles address x with 32-bit byte offsets.
 */
int moe_grouped_swiglu_gathered(const void* x, const int32_t* src_of, int k, const int32_t* offsets,
                                int R, int E, int H, int I, moe_dtype dtype, const moe_wbuf* w,
                                int e_begin, int e_end, void* ws, size_t ws_bytes, float* y_perm,
                                int32_t* status, moe_stream_t stream);

/*
 * moe_grouped_swiglu_combine -- the grouped SwiGLU GEMM with the row gather folded into its
 * operand loads (as moe_grouped_swiglu_gathered) and the combine folded into the down
 * GEMM's epilogue: each output row of assignment a = src_of[r] is scaled by topk_w[a] and
 * added into y[a / k] with a float atomic, so neither x_perm nor y_perm is written (the
 * groupedGEMM of the DWDP explainer's contiguous-buffer panel, producing the layer output).
 * y is cleared on the stream first.  The k terms of a token are added in whatever order
 * the tiles finish, so y agrees with moe_combine's fixed-order sum to rounding, not bit for
 * bit, and can differ in its last bits from run to run.  All experts of the buffer.
 *   x device [T][H] bf16; src_of device i32[T*k]; topk_w device f32[T][k]; y device f32[T][H]
 *   offsets, w, ws (moe_grouped_swiglu_workspace_size(T*k, ...)), status: as moe_grouped_swiglu.
 * Errors: as moe_grouped_swiglu_gathered; MOE_ERR_UNSUPPORTED for MOE_F32.
 */
int moe_grouped_swiglu_combine(const void* x, const int32_t* src_of, const float* topk_w, int T,
                               int k, const int32_t* offsets, int E, int H, int I, moe_dtype dtype,
                               const moe_wbuf* w, void* ws, size_t ws_bytes, float* y,
                               int32_t* status, moe_stream_t stream);

/*
 * moe_combine -- the weighted un-permute:
 *   y[t] = sum_{j=0..k-1} topk_w[t][j] * y_perm[row_of[t*k + j]], summed in j order, f32.
 * The pages give no combine rule of their own (like routing, the mixture only appears
 * through the DWDP explainer's imbalance panels); this is the output of the plain top-k
 * mixture of experts: each chosen expert's output weighted by its moe_route weight.  The
 * fixed j order makes the sum reproducible run to run.
 *   y_perm device f32[T*k][H]; row_of device i32[T*k]; topk_w device f32[T][k];
 *   y device f32[T][H] (must not alias y_perm).
 * Errors: MOE_ERR_ARG for null pointers or bad sizes.
 */
int moe_combine(const float* y_perm, const int32_t* row_of, const float* topk_w, int T, int k,
                int H, float* y, moe_stream_t stream);

/*
 * Multi-layer pipeline helpers (the block between two MoE layers).  The
 * explainer's prefetch-schedule panel hides the fetch of layer l+1's remote
 * experts behind layer l's MoE block and layer l+1's attention block; a
 * dense bf16 GEMM stands in for the attention block.
 *
 * moe_dense_gemm: out[M][N] = bf16(x[M][K] W[N][K]^T), bf16 in, f32 accumulate.
 *   K and N must be multiples of 8 and N*K below 2^31 (MOE_ERR_UNSUPPORTED otherwise).
 * moe_residual_add: out[i] = bf16(x[i] + y[i]) for i < n; x, out bf16, y f32;
 *   out may alias x.
 */
int moe_dense_gemm(const void* x, const void* w, int M, int N, int K, void* out,
                   moe_stream_t stream);
int moe_residual_add(const void* x, const float* y, int64_t n, void* out, moe_stream_t stream);

/*
 * Split-weight management by page stitching (set-up calls: these allocate and
 * map; never call them on the hot path).  The merged-buffer half of the
 * contiguous-buffer panel is built as one virtual range over physical blocks
 * placed back to back -- the local-expert block of the layer it serves, then
 * the half's own block for fetched experts -- so the local experts need no
 * copy (the "buffer-merge overhead" of the iteration-latency panel).
 *   moe_vmm_granularity: the allocation granularity on `device` (block sizes
 *                        must be multiples of it; an R1 expert block is 42 x 2 MiB)
 *   moe_vmm_create:      a physical block of `bytes` on `device` (no mapping)
 *   moe_vmm_map:         reserve one virtual range, map the n blocks back to
 *                        back, grant `device` read/write; *va is its base
 *   moe_vmm_unmap:       undo moe_vmm_map (same blocks sizes, in order)
 *   moe_vmm_release:     free a physical block once no range maps it
 * With such a range the expert set given to merge and prefetch must begin
 * with every expert of the stitched local block (their slots then coincide
 * with the block); a set that skips one would shift later experts into the
 * block and overwrite it.
 * Errors: MOE_ERR_ARG for empty or non-granular sizes, MOE_ERR_HIP from the runtime.
 */
typedef void* moe_phys_t; /* a hipMemGenericAllocationHandle_t */
int moe_vmm_granularity(int device, size_t* bytes);
int moe_vmm_create(int device, size_t bytes, moe_phys_t* phys);
int moe_vmm_map(int device, const moe_phys_t* phys, const size_t* bytes, int n, void** va);
int moe_vmm_unmap(void* va, const size_t* bytes, int n);
int moe_vmm_release(moe_phys_t phys);

/* Events and stream waits, so a caller without HIP headers can order the
 * copy stream against the compute stream.  timing != 0 makes a timing event. */
int moe_event_create(moe_event_t* ev, int timing);
int moe_event_destroy(moe_event_t ev);
int moe_event_record(moe_event_t ev, moe_stream_t stream);
int moe_event_elapsed_ms(moe_event_t start, moe_event_t stop, float* ms);
int moe_stream_wait_event(moe_stream_t stream, moe_event_t ev);

/* Thread-local text describing the last failed call on this thread ("" if none). */
const char* moe_last_error(void);
/* Library version string. */
const char* moe_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MOE_H_ */
