// Decode dispatch.
#include "common.cuh"

namespace sa {

hipError_t launch_decode_generic(const Decode& p, const void* q, const void* kc, const void* vc,
                                 void* o, float* lse, float* s, hipStream_t st);

int decode_auto_splits(const Decode& p) {
  (void)p;
  return 1;
}

bool decode_mfma_supported(const Decode& p) {
  (void)p;
  return false;
}

hipError_t launch_decode(const Decode& p, const void* q, const void* kc, const void* vc, void* o,
                         float* lse, float* s, float* ws, hipStream_t st) {
  (void)ws;
  return launch_decode_generic(p, q, kc, vc, o, lse, s, st);
}

}  // namespace sa
