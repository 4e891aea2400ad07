// Generic backward main pass: one wavefront per (query token, query head).
// For every valid key j it rebuilds P_ij = e^{x_ij - L_new} with the sink
// already in L_new, forms dx_ij = P_ij (<dO_i, V_j> - Delta_i) ("Attention
// Sink, Learnable Sink and dsink" s8), writes dQ_i directly and adds
// alpha dx_ij Q_i and P_ij dO_i into float32 dK/dV accumulators (atomics:
// many rows share a key).
#include "common.cuh"
#include "row_keys.cuh"

namespace sa {

template <typename T>
__global__ __launch_bounds__(64) void bwd_generic_kernel(Prefill p, const void* __restrict__ q,
                                                         const void* __restrict__ k,
                                                         const void* __restrict__ v,
                                                         const void* __restrict__ dout,
                                                         BwdWork w, void* dq) {
  const int t = blockIdx.x;
  const int h = blockIdx.y;
  const int lane = threadIdx.x;
  const int b = find_sample(p.cu, p.batch, t);
  const int t0 = p.cu[b];
  const int i = t - t0;
  const int g = h / (p.hq / p.hkv);
  const int D = p.d;
  const int nr = (D + 63) / 64;
  const size_t row = static_cast<size_t>(t) * p.hq + h;

  float qv[4], dov[4], dqv[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    int d = lane + 64 * r;
    bool ok = r < nr && d < D;
    qv[r] = ok ? Elem<T>::load(q, row * D + d) : 0.f;
    dov[r] = ok ? Elem<T>::load(dout, row * D + d) : 0.f;
    dqv[r] = 0.f;
  }
  const float delta = w.delta[row];
  const float lnew = w.lnew[row];

  for_each_valid_key(p, b, i, g, [&](int j) {
    const size_t krow = (static_cast<size_t>(t0 + j) * p.hkv + g) * D;
    float kv[4], vv[4];
    float dot = 0.f, dpv = 0.f;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      int d = lane + 64 * r;
      bool ok = r < nr && d < D;
      kv[r] = ok ? Elem<T>::load(k, krow + d) : 0.f;
      vv[r] = ok ? Elem<T>::load(v, krow + d) : 0.f;
      dot += qv[r] * kv[r];
      dpv += dov[r] * vv[r];
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      dot += __shfl_xor(dot, off);
      dpv += __shfl_xor(dpv, off);
    }
    const float pj = exp2f(dot * p.scale * kLog2e - lnew);   // lnew in log2 units
    const float ds = pj * (dpv - delta);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      int d = lane + 64 * r;
      if (r < nr && d < D) {
        dqv[r] += ds * kv[r];
        atomicAdd(w.dk_acc + krow + d, p.scale * ds * qv[r]);
        atomicAdd(w.dv_acc + krow + d, pj * dov[r]);
      }
    }
  });

#pragma unroll
  for (int r = 0; r < 4; ++r) {
    int d = lane + 64 * r;
    if (r < nr && d < D) Elem<T>::store(dq, row * D + d, p.scale * dqv[r]);
  }
}

hipError_t launch_bwd_generic(const Prefill& p, const void* q, const void* k, const void* v,
                              const void* dout, const BwdWork& w, void* dq, hipStream_t st) {
  if (p.total == 0) return hipSuccess;
  dim3 grid(p.total, p.hq);
  if (p.dtype == SINK_ATTN_F32)
    hipLaunchKernelGGL(bwd_generic_kernel<float>, grid, dim3(64), 0, st, p, q, k, v, dout, w, dq);
  else
    hipLaunchKernelGGL(bwd_generic_kernel<uint16_t>, grid, dim3(64), 0, st, p, q, k, v, dout, w, dq);
  return hipGetLastError();
}

}  // namespace sa
