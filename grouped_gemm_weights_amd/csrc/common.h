// Shared host/device helpers of the MoE library: error reporting, argument
// checks and small device utilities.  gfx950 (CDNA4) only: wave64.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <string>

#include "../../include/moe.h"

namespace moe {

constexpr int kWave = 64;

// Thread-local text of the last failure; set by fail(), read by moe_last_error().
std::string& last_error();

inline int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  last_error() = buf;
  return code;
}

// Debug mode (MOE_DEBUG_SYNC set to anything but "" or "0"): every call that enqueued work
// synchronises its stream before it returns; a failed kernel becomes MOE_ERR_HIP and a set
// status bit MOE_ERR_STATUS, each with a description.  rc != MOE_OK passes through.
int debug_check(int rc, const char* who, hipStream_t s, const int32_t* status);

inline int hip_fail(hipError_t e, const char* what) {
  return fail(MOE_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

#define MOE_HIP_CHECK(call)                                 \
  do {                                                      \
    hipError_t e_ = (call);                                 \
    if (e_ != hipSuccess) return ::moe::hip_fail(e_, #call); \
  } while (0)

// Check a kernel launch (launch-configuration errors surface here).
#define MOE_LAUNCH_CHECK(what)                                  \
  do {                                                          \
    hipError_t e_ = hipGetLastError();                          \
    if (e_ != hipSuccess) return ::moe::hip_fail(e_, what);     \
  } while (0)

inline hipStream_t as_stream(moe_stream_t s) { return reinterpret_cast<hipStream_t>(s); }
inline hipEvent_t as_event(moe_event_t e) { return reinterpret_cast<hipEvent_t>(e); }

inline size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }
inline int ceil_div(int a, int b) { return (a + b - 1) / b; }
inline int64_t ceil_div64(int64_t a, int64_t b) { return (a + b - 1) / b; }

inline int elem_size(moe_dtype dt) { return dt == MOE_BF16 ? 2 : 4; }

// ---------------------------------------------------------------------------
// device helpers
// ---------------------------------------------------------------------------

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// fp32 -> bf16 with round-to-nearest-even (the hardware conversion on gfx950).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  __bf16 h = static_cast<__bf16>(f);
  return __builtin_bit_cast(uint16_t, h);
}

__device__ __forceinline__ void status_or(int32_t* status, int32_t bits) {
  if (status) atomicOr(status, bits);
}

}  // namespace moe
