// Decode without a caller workspace: the split-KV partials go to a static
// device array of fixed size instead, so the call allocates nothing (for
// callers that cannot allocate device memory: code under HIP graph capture,
// tight serving loops, harnesses that forbid it).
//
// Each GPU the library runs on holds its own copy of `scratch` until the
// process ends.  Host code never uses the array's name as a device address:
// on the first call on a device, with that device current, its address is
// looked up once with hipGetSymbolAddress and kept per device; the kernels
// take that pointer as they take the workspace of sink_attn_decode.  Every
// call on a device shares the array: calls that overlap on one GPU (two
// streams, or two threads) race on it.  Nothing in it needs clearing: every
// split writes its whole partial before the merge reads it.
#include <hip/hip_runtime.h>

#include <mutex>

#include "internal.h"

namespace {

constexpr size_t kScratchBytes = SINK_ATTN_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::once_flag g_once[kMaxDevices];
void* g_scratch[kMaxDevices];
hipError_t g_status[kMaxDevices];

// The current device's copy of `scratch` (looked up once per device).
hipError_t scratch_for_current_device(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::call_once(g_once[dev], [dev] {
    void* p = nullptr;
    g_status[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    g_scratch[dev] = g_status[dev] == hipSuccess ? p : nullptr;
  });
  *out = g_scratch[dev];
  return g_status[dev];
}

}  // namespace

extern "C" int sink_attn_decode_noalloc(const sink_attn_decode_desc* desc, const void* q,
                                        const void* k_cache, const void* v_cache, void* o,
                                        float* lse, float* s, void* stream) {
  try {
    const size_t need = sink_attn_decode_workspace_size(desc);
    const int st = sink_attn_check_decode(desc, q, k_cache, v_cache, o, lse, s, need);
    if (st != SINK_ATTN_OK) return st;
    if (need > kScratchBytes)
      return sa::set_last_error(SINK_ATTN_WORKSPACE_TOO_SMALL,
                                "decode needs %zu bytes of split partials, more than the %zu bytes "
                                "of static scratch: use sink_attn_decode with a workspace or fewer "
                                "splits",
                                need, kScratchBytes);
    if (desc->batch == 0) return SINK_ATTN_OK;
    void* ws = nullptr;
    if (need > 0) {
      const hipError_t e = scratch_for_current_device(&ws);
      if (e != hipSuccess)
        return sa::set_last_error(SINK_ATTN_HIP_ERROR, "static scratch lookup: %s", hipGetErrorString(e));
    }
    return sink_attn_decode(desc, q, k_cache, v_cache, o, lse, s, ws, need, stream);
  } catch (...) {
    return sa::set_last_error(SINK_ATTN_HIP_ERROR, "unexpected exception in sink_attn_decode_noalloc");
  }
}
