// Backward main pass on matrix cores (bfloat16, head_dim 128).
#include "common.cuh"

namespace sa {

bool bwd_mfma_supported(const Prefill& p) {
  (void)p;
  return false;
}

hipError_t launch_bwd_mfma(const Prefill& p, const void* q, const void* k, const void* v,
                           const void* dout, const BwdWork& w, void* dk, void* dv, hipStream_t st) {
  (void)p; (void)q; (void)k; (void)v; (void)dout; (void)w; (void)dk; (void)dv; (void)st;
  return hipErrorNotSupported;
}

}  // namespace sa
