// Merged weight buffer management: the slot map, the merge of the local
// experts and the copy-engine prefetch of the remote ones.  Also the small
// event / error helpers of the C ABI.
//
// A merged buffer half holds n_slots expert blocks in one contiguous
// allocation; the expert set of a layer (ascending ids) fills slots 0..n-1 in
// order.  moe_merge_weights writes the device slot map with a kernel whose
// arguments carry the map (so it is ordered on the stream like the copies and
// needs no host staging buffer that could be overwritten while in flight),
// then copies the local pool's experts into their slots; moe_prefetch_layer
// copies the remote pool's experts.  Runs of consecutive ids that sit in
// consecutive slots and consecutive pool positions go out as one copy.  With
// MOE_COPY_SDMA a device-to-device copy is issued as
// hipMemcpyDeviceToDeviceNoCU, which the runtime executes on an SDMA engine
// and never on the compute units (DWDP explainer, "stay data-parallel" panel:
// the pull runs on the copy engine, off the compute units).  With
// MOE_COPY_KERNEL_ON(n) it is the library's streaming copy kernel on at most n
// workgroups: on one GPU, where the stand-in pull is an HBM-to-HBM copy, this
// keeps it on a bounded set of compute units instead of spreading a runtime
// copy kernel over the whole chip under a concurrent grouped GEMM.
#include <cstdlib>
#include <cstring>
#include <vector>

#include "common.h"

namespace moe {

std::string& last_error() {
  static thread_local std::string s;
  return s;
}

int debug_check(int rc, const char* who, hipStream_t s, const int32_t* status) {
  if (rc != MOE_OK) return rc;
  const char* v = std::getenv("MOE_DEBUG_SYNC");
  if (!v || !*v || std::strcmp(v, "0") == 0) return rc;
  hipError_t e = hipStreamSynchronize(s);
  if (e == hipSuccess) e = hipGetLastError();
  if (e != hipSuccess)
    return fail(MOE_ERR_HIP, "%s (debug sync): %s", who, hipGetErrorString(e));
  if (status) {
    int32_t bits = 0;
    e = hipMemcpy(&bits, status, sizeof(bits), hipMemcpyDeviceToHost);
    if (e != hipSuccess)
      return fail(MOE_ERR_HIP, "%s (debug sync, status read): %s", who, hipGetErrorString(e));
    if (bits)
      return fail(MOE_ERR_STATUS, "%s (debug sync): device status 0x%x:%s%s%s", who, bits,
                  (bits & MOE_STATUS_NONFINITE_LOGIT) ? " non-finite logit" : "",
                  (bits & MOE_STATUS_EXPERT_ABSENT) ? " expert absent from the merged buffer" : "",
                  (bits & MOE_STATUS_BAD_EXPERT_ID) ? " expert id out of range" : "");
  }
  return MOE_OK;
}

namespace {

constexpr int kSlotIdsPerLaunch = 256;

struct SlotChunk {
  int32_t ids[kSlotIdsPerLaunch];
  int32_t n;
  int32_t first_slot;
};

__global__ void slot_fill_kernel(int32_t* slot_of, int E) {
  const int e = blockIdx.x * blockDim.x + threadIdx.x;
  if (e < E) slot_of[e] = -1;
}

__global__ void slot_set_kernel(int32_t* slot_of, SlotChunk c) {
  const int i = threadIdx.x;
  if (i < c.n) slot_of[c.ids[i]] = c.first_slot + i;
}

// A caller's handling of a failed pull can be tested on a healthy device: with
// MOE_INJECT_FAULT=<site> in the environment, the call at that site fails the way a failed
// HIP call does, before it enqueues anything.
bool injected_fault(const char* site) {
  const char* v = std::getenv("MOE_INJECT_FAULT");
  return v && std::strcmp(v, site) == 0;
}

int check_ids(const char* who, const int32_t* ids, int n, const moe_wbuf* dst) {
  if (!dst || !dst->base || dst->expert_bytes <= 0 || dst->n_experts < 1 || dst->n_slots < 0)
    return fail(MOE_ERR_ARG, "%s: bad merged buffer", who);
  if (n < 0 || n > dst->n_slots)
    return fail(MOE_ERR_ARG, "%s: %d ids for %d slots", who, n, dst->n_slots);
  if (n > 0 && !ids) return fail(MOE_ERR_ARG, "%s: null ids", who);
  for (int i = 0; i < n; ++i) {
    if (ids[i] < 0 || ids[i] >= dst->n_experts)
      return fail(MOE_ERR_ARG, "%s: id %d outside [0, %d)", who, ids[i], dst->n_experts);
    if (i > 0 && ids[i] <= ids[i - 1])
      return fail(MOE_ERR_ARG, "%s: ids not strictly ascending at %d", who, i);
  }
  return MOE_OK;
}

int check_pool(const char* who, const moe_pool* p, const moe_wbuf* dst) {
  // an empty pool (n_experts == 0) may have a null base
  if (!p || (!p->base && p->n_experts != 0) || p->n_experts < 0 || p->first_expert < 0)
    return fail(MOE_ERR_ARG, "%s: bad pool", who);
  if (p->expert_bytes != dst->expert_bytes)
    return fail(MOE_ERR_ARG, "%s: pool expert_bytes %lld != buffer %lld", who,
                static_cast<long long>(p->expert_bytes), static_cast<long long>(dst->expert_bytes));
  return MOE_OK;
}

// How a pool's runs are copied: a runtime copy of `kind`, or (kernel_blocks >= 0) the
// library's copy kernel on at most kernel_blocks workgroups (0: no limit).
struct CopyPlan {
  hipMemcpyKind kind;
  int kernel_blocks;
};

constexpr int kCopyThreads = 1024;
constexpr int kCopyUnroll = 8;
constexpr int64_t kCopyMaxBlocks = int64_t{1} << 20;

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

int copy_plan(const char* who, const void* src, int copy_mode, CopyPlan* plan) {
  const int base = copy_mode & 0xff, blocks = copy_mode >> 8;
  if (copy_mode < 0 || (base != MOE_COPY_SDMA && base != MOE_COPY_ANY && base != MOE_COPY_KERNEL) ||
      (base != MOE_COPY_KERNEL && blocks != 0))
    return fail(MOE_ERR_ARG, "%s: bad copy_mode %d", who, copy_mode);
  plan->kernel_blocks = -1;
  plan->kind = hipMemcpyDefault;
  if (base == MOE_COPY_ANY || !src) return MOE_OK;   // !src: an empty pool, nothing to copy
  hipPointerAttribute_t attr;
  hipError_t e = hipPointerGetAttributes(&attr, src);
  if (e != hipSuccess) return hip_fail(e, "hipPointerGetAttributes(pool)");
  const bool host = attr.type == hipMemoryTypeHost;
  if (base == MOE_COPY_SDMA) {
    plan->kind = host ? hipMemcpyHostToDevice : hipMemcpyDeviceToDeviceNoCU;
  } else if (host) {
    plan->kind = hipMemcpyHostToDevice;
  } else {
    plan->kernel_blocks = blocks;
  }
  return MOE_OK;
}

// dst[i] = src[i] for i < n16 (16-byte units); each thread keeps kCopyUnroll loads in flight.
// Loads and stores are non-temporal: the pulled weights are read once, and streaming them
// through L2 would evict what a grouped GEMM running beside the pull is reusing.
__global__ __launch_bounds__(kCopyThreads) void copy_kernel(const u32x4* __restrict__ src,
                                                            u32x4* __restrict__ dst, int64_t n16) {
  const int64_t step = static_cast<int64_t>(gridDim.x) * kCopyThreads * kCopyUnroll;
  for (int64_t i0 = static_cast<int64_t>(blockIdx.x) * kCopyThreads * kCopyUnroll + threadIdx.x;
       i0 < n16; i0 += step) {
    u32x4 v[kCopyUnroll];
#pragma unroll
    for (int u = 0; u < kCopyUnroll; ++u) {
      const int64_t i = i0 + static_cast<int64_t>(u) * kCopyThreads;
      v[u] = u32x4{0, 0, 0, 0};
      if (i < n16) v[u] = __builtin_nontemporal_load(src + i);
    }
#pragma unroll
    for (int u = 0; u < kCopyUnroll; ++u) {
      const int64_t i = i0 + static_cast<int64_t>(u) * kCopyThreads;
      if (i < n16) __builtin_nontemporal_store(v[u], dst + i);
    }
  }
}

// The routed pull with the expert set read on the device.  A chunk is the kCopyThreads *
// kRoutedUnroll 16-byte units a workgroup moves at once; work unit c is kRoutedChunks
// consecutive chunks (group c % gpe) of pool expert c / gpe.  Workgroups take units
// c = blockIdx.x, blockIdx.x + gridDim.x, ... and skip those of experts that received no
// tokens; reading that count is one dependent load before a unit's copies start, so a unit
// holds two chunks to spread it (one chunk or four per unit made the pull 2-3 % slower).
// The slot map entries of the pool's experts (the slot, or -1 for an expert with no
// tokens, whose slot is left as it was) are written by the first threads of the grid.
constexpr int kRoutedChunks = 2;
// 16-byte loads in flight per thread and chunk: 4 here (64 KB chunks), where 8 made the
// routed pull 2 % slower; the whole-pool copy kernel above keeps 8, where 4 made it 7 %
// slower
constexpr int kRoutedUnroll = 4;

__global__ __launch_bounds__(kCopyThreads) void copy_routed_kernel(
    const u32x4* __restrict__ src, u32x4* __restrict__ dst, int64_t eb16, int64_t gpe, int first,
    int n, const int32_t* __restrict__ counts, int32_t* __restrict__ slot_of) {
  constexpr int64_t kChunk = static_cast<int64_t>(kCopyThreads) * kRoutedUnroll;
  const int64_t nthreads = static_cast<int64_t>(gridDim.x) * kCopyThreads;
  for (int64_t q = static_cast<int64_t>(blockIdx.x) * kCopyThreads + threadIdx.x; q < n;
       q += nthreads) {
    const int e = first + static_cast<int>(q);
    slot_of[e] = counts[e] > 0 ? e : -1;
  }
  const int64_t units = static_cast<int64_t>(n) * gpe;
  for (int64_t c = blockIdx.x; c < units; c += gridDim.x) {
    const int p = static_cast<int>(c / gpe);
    if (counts[first + p] <= 0) continue;
    const u32x4* __restrict__ from = src + static_cast<int64_t>(p) * eb16;
    u32x4* __restrict__ to = dst + static_cast<int64_t>(first + p) * eb16;
    const int64_t c0 = (c % gpe) * kRoutedChunks * kChunk;   // first unit of the group
    for (int g = 0; g < kRoutedChunks; ++g) {
      const int64_t chunk0 = c0 + g * kChunk;
      const int64_t base = chunk0 + threadIdx.x;
      u32x4 v[kRoutedUnroll];
      if (chunk0 + kChunk <= eb16) {
        // a whole chunk (a workgroup-uniform test): straight-line loads, then stores, so the
        // next chunk's loads issue without waiting for these stores
#pragma unroll
        for (int u = 0; u < kRoutedUnroll; ++u)
          v[u] = __builtin_nontemporal_load(from + base + static_cast<int64_t>(u) * kCopyThreads);
#pragma unroll
        for (int u = 0; u < kRoutedUnroll; ++u)
          __builtin_nontemporal_store(v[u], to + base + static_cast<int64_t>(u) * kCopyThreads);
      } else if (chunk0 < eb16) {
#pragma unroll
        for (int u = 0; u < kRoutedUnroll; ++u) {
          const int64_t i = base + static_cast<int64_t>(u) * kCopyThreads;
          v[u] = u32x4{0, 0, 0, 0};
          if (i < eb16) v[u] = __builtin_nontemporal_load(from + i);
        }
#pragma unroll
        for (int u = 0; u < kRoutedUnroll; ++u) {
          const int64_t i = base + static_cast<int64_t>(u) * kCopyThreads;
          if (i < eb16) __builtin_nontemporal_store(v[u], to + i);
        }
      }
    }
  }
}

int copy_run(void* to, const void* from, size_t bytes, const CopyPlan& plan, hipStream_t s) {
  const bool aligned = (reinterpret_cast<uintptr_t>(to) % 16 == 0) &&
                       (reinterpret_cast<uintptr_t>(from) % 16 == 0) && (bytes % 16 == 0);
  if (plan.kernel_blocks < 0 || !aligned) {
    MOE_HIP_CHECK(hipMemcpyAsync(to, from, bytes, plan.kernel_blocks < 0 ? plan.kind : hipMemcpyDefault, s));
    return MOE_OK;
  }
  const int64_t n16 = static_cast<int64_t>(bytes / 16);
  int64_t blocks = ceil_div64(n16, static_cast<int64_t>(kCopyThreads) * kCopyUnroll);
  blocks = std::min<int64_t>(blocks, plan.kernel_blocks > 0 ? plan.kernel_blocks : kCopyMaxBlocks);
  hipLaunchKernelGGL(copy_kernel, dim3(static_cast<unsigned>(blocks)), dim3(kCopyThreads), 0, s,
                     static_cast<const u32x4*>(from), static_cast<u32x4*>(to), n16);
  MOE_LAUNCH_CHECK("copy kernel launch");
  return MOE_OK;
}

// Copy the experts of ids that the pool holds into their slots.
int copy_pool_experts(const moe_pool* p, const int32_t* ids, int n, moe_wbuf* dst,
                      hipStream_t s, const CopyPlan& plan) {
  const int64_t eb = dst->expert_bytes;
  const int64_t lo = p->first_expert, hi = lo + p->n_experts;
  auto in_pool = [&](int32_t e) { return e >= lo && e < hi; };
  int i = 0;
  while (i < n) {
    if (!in_pool(ids[i])) {
      ++i;
      continue;
    }
    int j = i + 1;
    while (j < n && in_pool(ids[j]) && ids[j] == ids[j - 1] + 1) ++j;
    const char* src = static_cast<const char*>(p->base) + (ids[i] - lo) * eb;
    char* to = static_cast<char*>(dst->base) + static_cast<int64_t>(i) * eb;
    // a run already in place (the local block stitched at the head of the range) needs no copy
    if (src != to) {
      const int rc = copy_run(to, src, static_cast<size_t>(j - i) * eb, plan, s);
      if (rc) return rc;
    }
    i = j;
  }
  return MOE_OK;
}

}  // namespace
}  // namespace moe

extern "C" int moe_merge_weights(const moe_pool* local, const int32_t* ids_host, int n_ids,
                                 moe_wbuf* dst, moe_stream_t stream, moe_event_t wait_free,
                                 moe_event_t ready, int copy_mode) {
  using namespace moe;
  int rc = check_ids("moe_merge_weights", ids_host, n_ids, dst);
  if (rc) return rc;
  if (!dst->slot_of) return fail(MOE_ERR_ARG, "moe_merge_weights: null slot map");
  rc = check_pool("moe_merge_weights", local, dst);
  if (rc) return rc;
  CopyPlan plan;
  rc = copy_plan("moe_merge_weights", local->base, copy_mode, &plan);
  if (rc) return rc;
  hipStream_t s = as_stream(stream);
  if (wait_free) MOE_HIP_CHECK(hipStreamWaitEvent(s, as_event(wait_free), 0));
  const int E = dst->n_experts;
  hipLaunchKernelGGL(slot_fill_kernel, dim3(ceil_div(E, 256)), dim3(256), 0, s, dst->slot_of, E);
  MOE_LAUNCH_CHECK("moe_merge_weights: slot fill");
  for (int i0 = 0; i0 < n_ids; i0 += kSlotIdsPerLaunch) {
    SlotChunk c;
    c.n = std::min(kSlotIdsPerLaunch, n_ids - i0);
    c.first_slot = i0;
    for (int i = 0; i < c.n; ++i) c.ids[i] = ids_host[i0 + i];
    hipLaunchKernelGGL(slot_set_kernel, dim3(1), dim3(kSlotIdsPerLaunch), 0, s, dst->slot_of, c);
    MOE_LAUNCH_CHECK("moe_merge_weights: slot set");
  }
  rc = copy_pool_experts(local, ids_host, n_ids, dst, s, plan);
  if (rc) return rc;
  if (ready) MOE_HIP_CHECK(hipEventRecord(as_event(ready), s));
  return debug_check(MOE_OK, "moe_merge_weights", s, nullptr);
}

extern "C" int moe_prefetch_layer(const moe_pool* remote, const int32_t* ids_host, int n_ids,
                                  moe_wbuf* dst, moe_stream_t copy_stream, moe_event_t wait_free,
                                  moe_event_t ready, int copy_mode) {
  using namespace moe;
  if (injected_fault("prefetch"))
    return fail(MOE_ERR_HIP, "moe_prefetch_layer: fault injected (MOE_INJECT_FAULT=prefetch)");
  int rc = check_ids("moe_prefetch_layer", ids_host, n_ids, dst);
  if (rc) return rc;
  rc = check_pool("moe_prefetch_layer", remote, dst);
  if (rc) return rc;
  CopyPlan plan;
  rc = copy_plan("moe_prefetch_layer", remote->base, copy_mode, &plan);
  if (rc) return rc;
  hipStream_t s = as_stream(copy_stream);
  if (wait_free) MOE_HIP_CHECK(hipStreamWaitEvent(s, as_event(wait_free), 0));
  rc = copy_pool_experts(remote, ids_host, n_ids, dst, s, plan);
  if (rc) return rc;
  if (ready) MOE_HIP_CHECK(hipEventRecord(as_event(ready), s));
  return debug_check(MOE_OK, "moe_prefetch_layer", s, nullptr);
}

extern "C" int moe_event_create(moe_event_t* ev, int timing) {
  using namespace moe;
  if (!ev) return fail(MOE_ERR_ARG, "moe_event_create: null");
  hipEvent_t e;
  MOE_HIP_CHECK(hipEventCreateWithFlags(&e, timing ? hipEventDefault : hipEventDisableTiming));
  *ev = reinterpret_cast<moe_event_t>(e);
  return MOE_OK;
}

extern "C" int moe_event_destroy(moe_event_t ev) {
  using namespace moe;
  if (!ev) return MOE_OK;
  MOE_HIP_CHECK(hipEventDestroy(as_event(ev)));
  return MOE_OK;
}

extern "C" int moe_event_record(moe_event_t ev, moe_stream_t stream) {
  using namespace moe;
  if (!ev) return fail(MOE_ERR_ARG, "moe_event_record: null");
  MOE_HIP_CHECK(hipEventRecord(as_event(ev), as_stream(stream)));
  return MOE_OK;
}

extern "C" int moe_event_elapsed_ms(moe_event_t start, moe_event_t stop, float* ms) {
  using namespace moe;
  if (!start || !stop || !ms) return fail(MOE_ERR_ARG, "moe_event_elapsed_ms: null");
  MOE_HIP_CHECK(hipEventElapsedTime(ms, as_event(start), as_event(stop)));
  return MOE_OK;
}

extern "C" int moe_stream_wait_event(moe_stream_t stream, moe_event_t ev) {
  using namespace moe;
  if (!ev) return fail(MOE_ERR_ARG, "moe_stream_wait_event: null");
  MOE_HIP_CHECK(hipStreamWaitEvent(as_stream(stream), as_event(ev), 0));
  return MOE_OK;
}

extern "C" const char* moe_last_error(void) { return moe::last_error().c_str(); }

extern "C" const char* moe_version(void) { return "moe-gfx950 0.1"; }

extern "C" int moe_prefetch_routed(const moe_pool* remote, const int32_t* counts, moe_wbuf* dst,
                                   moe_stream_t copy_stream, moe_event_t counts_ready,
                                   moe_event_t wait_free, moe_event_t ready, int max_blocks) {
  using namespace moe;
  if (injected_fault("prefetch"))
    return fail(MOE_ERR_HIP, "moe_prefetch_routed: fault injected (MOE_INJECT_FAULT=prefetch)");
  int rc = check_ids("moe_prefetch_routed", nullptr, 0, dst);
  if (rc) return rc;
  rc = check_pool("moe_prefetch_routed", remote, dst);
  if (rc) return rc;
  if (!counts || !dst->slot_of) return fail(MOE_ERR_ARG, "moe_prefetch_routed: null pointer");
  if (max_blocks < 0) return fail(MOE_ERR_ARG, "moe_prefetch_routed: max_blocks %d", max_blocks);
  const int64_t first = remote->first_expert, n = remote->n_experts;
  if (first + n > dst->n_experts || first + n > dst->n_slots)
    return fail(MOE_ERR_ARG, "moe_prefetch_routed: experts [%lld, %lld) need slots up to their "
                "ids (buffer: %d experts, %d slots)", static_cast<long long>(first),
                static_cast<long long>(first + n), dst->n_experts, dst->n_slots);
  const int64_t eb = dst->expert_bytes;
  if (eb % 16 != 0 || reinterpret_cast<uintptr_t>(remote->base) % 16 != 0 ||
      reinterpret_cast<uintptr_t>(dst->base) % 16 != 0)
    return fail(MOE_ERR_UNSUPPORTED, "moe_prefetch_routed: expert blocks of %lld bytes or bases "
                "not 16-byte aligned", static_cast<long long>(eb));
  if (n > 0) {
    hipPointerAttribute_t attr;
    MOE_HIP_CHECK(hipPointerGetAttributes(&attr, remote->base));
    if (attr.type == hipMemoryTypeHost)
      return fail(MOE_ERR_UNSUPPORTED, "moe_prefetch_routed: the pool is in host memory (pull it "
                  "with moe_prefetch_layer after reading the counts back)");
  }
  hipStream_t s = as_stream(copy_stream);
  if (counts_ready) MOE_HIP_CHECK(hipStreamWaitEvent(s, as_event(counts_ready), 0));
  if (wait_free) MOE_HIP_CHECK(hipStreamWaitEvent(s, as_event(wait_free), 0));
  if (n > 0) {
    const int64_t eb16 = eb / 16;
    const int64_t gpe = ceil_div64(eb16, static_cast<int64_t>(kCopyThreads) * kRoutedUnroll *
                                             kRoutedChunks);
    const int64_t units = n * gpe;
    // one workgroup per unit unless bounded (the slot map needs ceil(n / kCopyThreads) at most,
    // which a bound of one workgroup still covers through the loop)
    int64_t blocks = max_blocks > 0 ? std::min<int64_t>(max_blocks, units) : units;
    blocks = std::min<int64_t>(blocks, kCopyMaxBlocks);
    hipLaunchKernelGGL(copy_routed_kernel, dim3(static_cast<unsigned>(blocks)), dim3(kCopyThreads),
                       0, s, static_cast<const u32x4*>(remote->base),
                       static_cast<u32x4*>(dst->base), eb16, gpe, static_cast<int>(first),
                       static_cast<int>(n), counts, dst->slot_of);
    MOE_LAUNCH_CHECK("moe_prefetch_routed: copy");
  }
  if (ready) MOE_HIP_CHECK(hipEventRecord(as_event(ready), s));
  return debug_check(MOE_OK, "moe_prefetch_routed", s, nullptr);
}
