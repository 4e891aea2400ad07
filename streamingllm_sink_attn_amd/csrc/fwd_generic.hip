// Generic forward: one wavefront per (query token, query head), any head_dim
// that is a multiple of 8 up to 256, float32 or bfloat16 storage.  Keys are
// walked one at a time with an online softmax (running max m and sum l); the
// sink enters only in the epilogue as the output scale
// s = sigma(L_orig - a_h) ("Attention Sink, Learnable Sink and dsink", s4).
// With gate0 != NULL it also writes the first-token gate (l - l_0) / l, the
// share of the real-token softmax not on the sample's first key ("Paper
// notes: Attention Sink and the native MoE in attention layers" s2, s5).
#include "common.cuh"
#include "row_keys.cuh"

namespace sa {

template <typename T>
__global__ __launch_bounds__(64) void fwd_generic_kernel(Prefill p, const void* __restrict__ q,
                                                         const void* __restrict__ k,
                                                         const void* __restrict__ v, void* o,
                                                         float* lse, float* s_out,
                                                         float* gate_out) {
  const int t = blockIdx.x;
  const int h = blockIdx.y;
  const int lane = threadIdx.x;
  const int b = find_sample(p.cu, p.batch, t);
  const int t0 = p.cu[b];
  const int i = t - t0;
  const int g = h / (p.hq / p.hkv);
  const int D = p.d;
  const int nr = (D + 63) / 64;

  float qv[4], acc[4];
  const size_t qrow = (static_cast<size_t>(t) * p.hq + h) * D;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    int d = lane + 64 * r;
    qv[r] = (r < nr && d < D) ? Elem<T>::load(q, qrow + d) : 0.f;
    acc[r] = 0.f;
  }
  float m = -kInf, l = 0.f;
  float l0 = 0.f;                        // probability mass of key 0 (same base as l)

  for_each_valid_key(p, b, i, g, [&](int j) {
    const size_t krow = (static_cast<size_t>(t0 + j) * p.hkv + g) * D;
    float dot = 0.f;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      int d = lane + 64 * r;
      if (r < nr && d < D) dot += qv[r] * Elem<T>::load(k, krow + d);
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) dot += __shfl_xor(dot, off);
    const float x = dot * p.scale;
    const float m_new = fmaxf(m, x);
    const float corr = __expf(m - m_new);
    const float pj = __expf(x - m_new);
    l = l * corr + pj;
    l0 = j == 0 ? pj : l0 * corr;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      int d = lane + 64 * r;
      float vv = (r < nr && d < D) ? Elem<T>::load(v, krow + d) : 0.f;
      acc[r] = acc[r] * corr + pj * vv;
    }
    m = m_new;
  });

  // Epilogue: L_orig = m + log l; s = sigma(L_orig - a_h); O = s * acc / l.
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
    lse[static_cast<size_t>(t) * p.hq + h] = L_orig;
    if (s_out) s_out[static_cast<size_t>(t) * p.hq + h] = s_val;
    if (gate_out) gate_out[static_cast<size_t>(t) * p.hq + h] = l > 0.f ? (l - l0) / l : 0.f;
  }
}

hipError_t launch_fwd_generic(const Prefill& p, const void* q, const void* k, const void* v,
                              void* o, float* lse, float* s, float* gate0, hipStream_t st) {
  if (p.total == 0) return hipSuccess;
  dim3 grid(p.total, p.hq);
  if (p.dtype == SINK_ATTN_F32)
    hipLaunchKernelGGL(fwd_generic_kernel<float>, grid, dim3(64), 0, st, p, q, k, v, o, lse, s, gate0);
  else
    hipLaunchKernelGGL(fwd_generic_kernel<uint16_t>, grid, dim3(64), 0, st, p, q, k, v, o, lse, s,
                       gate0);
  return hipGetLastError();
}

}  // namespace sa
