// Split-weight management with virtual-memory page stitching (set-up calls).
//
// A merged buffer half must reach the grouped GEMM as one contiguous range
// (DWDP explainer, contiguous-buffer panel); copying the local experts into
// every half is the "buffer-merge overhead" its iteration-latency panel
// blames.  Here a half is instead one virtual range stitched from physical
// blocks: the local-expert block of the layer it serves, then the half's own
// block for the fetched experts.  The local experts' bytes then already sit
// at their slots, so moe_merge_weights, given that range as the local pool,
// finds source == destination and copies nothing; only the slot map is
// written.  Expert blocks of the R1 shape are 42 x 2 MiB, so the blocks meet
// the allocation granularity exactly.
#include <vector>

#include "common.h"

namespace moe {
namespace {

hipMemAllocationProp device_prop(int device) {
  hipMemAllocationProp prop = {};
  prop.type = hipMemAllocationTypePinned;
  prop.location.type = hipMemLocationTypeDevice;
  prop.location.id = device;
  return prop;
}

}  // namespace
}  // namespace moe

extern "C" int moe_vmm_granularity(int device, size_t* bytes) {
  using namespace moe;
  if (!bytes) return fail(MOE_ERR_ARG, "moe_vmm_granularity: null");
  hipMemAllocationProp prop = device_prop(device);
  MOE_HIP_CHECK(hipMemGetAllocationGranularity(bytes, &prop, hipMemAllocationGranularityMinimum));
  return MOE_OK;
}

extern "C" int moe_vmm_create(int device, size_t bytes, moe_phys_t* phys) {
  using namespace moe;
  if (!phys || bytes == 0) return fail(MOE_ERR_ARG, "moe_vmm_create: bad arguments");
  size_t g = 0;
  int rc = moe_vmm_granularity(device, &g);
  if (rc) return rc;
  if (bytes % g != 0)
    return fail(MOE_ERR_ARG, "moe_vmm_create: %zu bytes is not a multiple of the granularity %zu",
                bytes, g);
  hipMemAllocationProp prop = device_prop(device);
  hipMemGenericAllocationHandle_t h;
  MOE_HIP_CHECK(hipMemCreate(&h, bytes, &prop, 0));
  *phys = reinterpret_cast<moe_phys_t>(h);
  return MOE_OK;
}

extern "C" int moe_vmm_map(int device, const moe_phys_t* phys, const size_t* bytes, int n,
                           void** va) {
  using namespace moe;
  if (!phys || !bytes || n < 1 || !va) return fail(MOE_ERR_ARG, "moe_vmm_map: bad arguments");
  size_t g = 0;
  int rc = moe_vmm_granularity(device, &g);
  if (rc) return rc;
  size_t total = 0;
  for (int i = 0; i < n; ++i) {
    if (!phys[i] || bytes[i] == 0 || bytes[i] % g != 0)
      return fail(MOE_ERR_ARG, "moe_vmm_map: piece %d is empty or not granular", i);
    total += bytes[i];
  }
  void* base = nullptr;
  MOE_HIP_CHECK(hipMemAddressReserve(&base, total, g, nullptr, 0));
  size_t off = 0;
  for (int i = 0; i < n; ++i) {
    hipError_t e = hipMemMap(static_cast<char*>(base) + off, bytes[i], 0,
                             reinterpret_cast<hipMemGenericAllocationHandle_t>(phys[i]), 0);
    if (e != hipSuccess) {
      for (size_t o = 0, j = 0; j < static_cast<size_t>(i); o += bytes[j], ++j)
        (void)hipMemUnmap(static_cast<char*>(base) + o, bytes[j]);
      (void)hipMemAddressFree(base, total);
      return hip_fail(e, "hipMemMap");
    }
    off += bytes[i];
  }
  hipMemAccessDesc acc = {};
  acc.location.type = hipMemLocationTypeDevice;
  acc.location.id = device;
  acc.flags = hipMemAccessFlagsProtReadWrite;
  hipError_t e = hipMemSetAccess(base, total, &acc, 1);
  if (e != hipSuccess) {
    for (size_t o = 0, j = 0; j < static_cast<size_t>(n); o += bytes[j], ++j)
      (void)hipMemUnmap(static_cast<char*>(base) + o, bytes[j]);
    (void)hipMemAddressFree(base, total);
    return hip_fail(e, "hipMemSetAccess");
  }
  *va = base;
  return MOE_OK;
}

extern "C" int moe_vmm_unmap(void* va, const size_t* bytes, int n) {
  using namespace moe;
  if (!va || !bytes || n < 1) return fail(MOE_ERR_ARG, "moe_vmm_unmap: bad arguments");
  size_t off = 0;
  for (int i = 0; i < n; ++i) {
    MOE_HIP_CHECK(hipMemUnmap(static_cast<char*>(va) + off, bytes[i]));
    off += bytes[i];
  }
  MOE_HIP_CHECK(hipMemAddressFree(va, off));
  return MOE_OK;
}

extern "C" int moe_vmm_release(moe_phys_t phys) {
  using namespace moe;
  if (!phys) return MOE_OK;
  MOE_HIP_CHECK(hipMemRelease(reinterpret_cast<hipMemGenericAllocationHandle_t>(phys)));
  return MOE_OK;
}
