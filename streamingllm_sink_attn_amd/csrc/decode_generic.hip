// Generic decode: one wavefront per (sequence, query head) walks the valid
// cache slots [0, cache_seqlens[b]) in slot order with an online softmax.
// Slots form an unordered set (a ring buffer keeps the first tokens and the
// recent window in any slot order), so there is no mask; the sink enters in
// the epilogue as s = sigma(L_orig - a_h) ("Attention Sink, Learnable Sink and
// dsink" s4).
#include "common.cuh"

namespace sa {

template <typename T>
__global__ __launch_bounds__(64) void decode_generic_kernel(Decode p, const void* __restrict__ q,
                                                            const void* __restrict__ kc,
                                                            const void* __restrict__ vc, void* o,
                                                            float* lse, float* s_out) {
  const int b = blockIdx.x;
  const int h = blockIdx.y;
  const int lane = threadIdx.x;
  const int g = h / (p.hq / p.hkv);
  const int D = p.d;
  const int nr = (D + 63) / 64;
  const int n = p.cache_seqlens ? min(p.cache_seqlens[b], p.slots) : p.slots;
  const size_t qrow = (static_cast<size_t>(b) * p.hq + h) * D;

  float qv[4], acc[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    int d = lane + 64 * r;
    qv[r] = (r < nr && d < D) ? Elem<T>::load(q, qrow + d) : 0.f;
    acc[r] = 0.f;
  }
  float m = -kInf, l = 0.f;
  for (int j = 0; j < n; ++j) {
    const size_t krow = ((static_cast<size_t>(b) * p.slots + j) * p.hkv + g) * D;
    float dot = 0.f;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      int d = lane + 64 * r;
      if (r < nr && d < D) dot += qv[r] * Elem<T>::load(kc, krow + d);
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) dot += __shfl_xor(dot, off);
    const float x = dot * p.scale;
    const float m_new = fmaxf(m, x);
    const float corr = __expf(m - m_new);
    const float pj = __expf(x - m_new);
    l = l * corr + pj;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      int d = lane + 64 * r;
      float vv = (r < nr && d < D) ? Elem<T>::load(vc, krow + d) : 0.f;
      acc[r] = acc[r] * corr + pj * vv;
    }
    m = m_new;
  }
  float L_orig, s_val, mul;
  const bool has_sink = p.sink != nullptr;
  if (l > 0.f) {
    L_orig = m + __logf(l);
    s_val = has_sink ? 1.f / (1.f + __expf(p.sink[h] - L_orig)) : 1.f;
    mul = s_val / l;
  } else {
    L_orig = -kInf;
    s_val = has_sink ? 0.f : 1.f;
    mul = 0.f;
  }
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    int d = lane + 64 * r;
    if (r < nr && d < D) Elem<T>::store(o, qrow + d, acc[r] * mul);
  }
  if (lane == 0) {
    lse[static_cast<size_t>(b) * p.hq + h] = L_orig;
    if (s_out) s_out[static_cast<size_t>(b) * p.hq + h] = s_val;
  }
}

hipError_t launch_decode_generic(const Decode& p, const void* q, const void* kc, const void* vc,
                                 void* o, float* lse, float* s, hipStream_t st) {
  if (p.batch == 0) return hipSuccess;
  dim3 grid(p.batch, p.hq);
  if (p.dtype == SINK_ATTN_F32)
    hipLaunchKernelGGL(decode_generic_kernel<float>, grid, dim3(64), 0, st, p, q, kc, vc, o, lse, s);
  else
    hipLaunchKernelGGL(decode_generic_kernel<uint16_t>, grid, dim3(64), 0, st, p, q, kc, vc, o, lse, s);
  return hipGetLastError();
}

}  // namespace sa
