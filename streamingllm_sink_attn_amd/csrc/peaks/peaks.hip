// Microbenchmarks that ground the rooflines on the GPU the library runs on:
// the achievable HBM streaming-read rate, the dense bf16 matrix-core rate of
// v_mfma_f32_32x32x16_bf16 and the v_exp_f32 rate.  Built as their own
// library (libsinkattn_peaks.so); the attention path does not use them.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "sink_attn_peaks.h"

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Every lane reads 16-byte pieces in a grid-stride loop (consecutive lanes
// consecutive pieces), four loads in flight per lane, and folds them into one
// word per workgroup.
__global__ __launch_bounds__(256) void read_kernel(const u32x4* __restrict__ src, size_t n,
                                                   uint32_t* __restrict__ out) {
  __shared__ uint32_t red[256];
  uint32_t acc = 0u;
  const size_t stride = static_cast<size_t>(gridDim.x) * blockDim.x;
  size_t i = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  for (; i + 3 * stride < n; i += 4 * stride) {
    const u32x4 v0 = __builtin_nontemporal_load(src + i);
    const u32x4 v1 = __builtin_nontemporal_load(src + i + stride);
    const u32x4 v2 = __builtin_nontemporal_load(src + i + 2 * stride);
    const u32x4 v3 = __builtin_nontemporal_load(src + i + 3 * stride);
    acc ^= (v0[0] ^ v0[1] ^ v0[2] ^ v0[3]) ^ (v1[0] ^ v1[1] ^ v1[2] ^ v1[3]) ^
           (v2[0] ^ v2[1] ^ v2[2] ^ v2[3]) ^ (v3[0] ^ v3[1] ^ v3[2] ^ v3[3]);
  }
  for (; i < n; i += stride) {
    const u32x4 v = __builtin_nontemporal_load(src + i);
    acc ^= v[0] ^ v[1] ^ v[2] ^ v[3];
  }
  red[threadIdx.x] = acc;
  __syncthreads();
  for (int s = 128; s > 0; s >>= 1) {
    if (threadIdx.x < s) red[threadIdx.x] ^= red[threadIdx.x + s];
    __syncthreads();
  }
  if (threadIdx.x == 0) out[blockIdx.x] = red[0];
}

// Four independent accumulation chains per wavefront, so the matrix core
// never waits for a result.
__global__ __launch_bounds__(256) void mfma_kernel(int iters, float* __restrict__ out) {
  const int lane = threadIdx.x & 63;
  bf16x8 a, b;
  for (int e = 0; e < 8; ++e) {
    a[e] = static_cast<__bf16>(0.001f * (lane + e));
    b[e] = static_cast<__bf16>(0.002f * (lane - e));
  }
  f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
  for (int it = 0; it < iters; ++it) {
    c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c0, 0, 0, 0);
    c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c1, 0, 0, 0);
    c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c2, 0, 0, 0);
    c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c3, 0, 0, 0);
  }
  float s = 0.f;
  for (int i = 0; i < 16; ++i) s += c0[i] + c1[i] + c2[i] + c3[i];
  out[blockIdx.x * blockDim.x + threadIdx.x] = s;
}

// Eight independent chains of x <- exp2(x * m + k) per lane.
__global__ __launch_bounds__(256) void exp_kernel(int iters, float* __restrict__ out) {
  float x[8];
  for (int j = 0; j < 8; ++j) x[j] = -0.001f * (threadIdx.x + j);
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < 8; ++j) x[j] = __builtin_amdgcn_exp2f(__builtin_fmaf(x[j], -0.5f, -1.0f));
  }
  float s = 0.f;
  for (int j = 0; j < 8; ++j) s += x[j];
  out[blockIdx.x * blockDim.x + threadIdx.x] = s;
}

// Co-issue of matrix and vector work.  Each wavefront runs `iters`
// iterations of 16 v_mfma_f32_32x32x16_bf16 (four independent chains)
// and/or 32 independent FMAs (eight chains), and records its own s_memtime
// cycles.  Mode 0: MFMAs only; 1: FMAs only; 2: both in one wavefront, two
// FMAs after each MFMA; 3: wavefronts 0-3 only the MFMAs and wavefronts 4-7
// (the same four SIMDs) only the FMAs, each role a loop of its own behind a
// scalar branch.  One 512-lane workgroup per CU (launch bounds).
struct CoState {
  bf16x8 a, b;
  f32x16 c0, c1, c2, c3;
  float x[8];
};
template <bool MF, bool FM>
__device__ __forceinline__ void coissue_loop(CoState& st, int iters) {
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
#define SA_PEAKS_SLOT(C, J)                                                         \
  if constexpr (MF) st.C = __builtin_amdgcn_mfma_f32_32x32x16_bf16(st.a, st.b, st.C, 0, 0, 0); \
  __builtin_amdgcn_sched_barrier(0);                                                \
  if constexpr (FM) {                                                               \
    st.x[J] = __builtin_fmaf(st.x[J], 0.999f, 0.001f);                              \
    st.x[J + 1] = __builtin_fmaf(st.x[J + 1], 0.999f, 0.001f);                      \
  }                                                                                 \
  __builtin_amdgcn_sched_barrier(0);
      SA_PEAKS_SLOT(c0, 0)
      SA_PEAKS_SLOT(c1, 2)
      SA_PEAKS_SLOT(c2, 4)
      SA_PEAKS_SLOT(c3, 6)
#undef SA_PEAKS_SLOT
    }
  }
}
template <int MODE>
__global__ __launch_bounds__(512, 1) void coissue_kernel(int iters, float* __restrict__ out,
                                                         long long* __restrict__ cycles) {
  // 96 KB of LDS: one workgroup per CU, so each SIMD holds exactly wavefronts
  // w and w + 4 of it
  __shared__ uint32_t pad[24576];
  pad[threadIdx.x] = threadIdx.x;
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // scalar: roles branch
  CoState st;
  for (int e = 0; e < 8; ++e) {
    st.a[e] = static_cast<__bf16>(0.001f * (lane + e));
    st.b[e] = static_cast<__bf16>(0.002f * (lane - e));
  }
  st.c0 = st.c1 = st.c2 = st.c3 = f32x16{};
  for (int j = 0; j < 8; ++j) st.x[j] = 0.001f * (lane + j);
  const long long t0 = clock64();
  if constexpr (MODE == 0) coissue_loop<true, false>(st, iters);
  else if constexpr (MODE == 1) coissue_loop<false, true>(st, iters);
  else if constexpr (MODE == 2) coissue_loop<true, true>(st, iters);
  else {
    if (wv < 4) coissue_loop<true, false>(st, iters);
    else coissue_loop<false, true>(st, iters);
  }
  const long long t1 = clock64();
  float s = static_cast<float>(pad[threadIdx.x]);
  for (int i = 0; i < 16; ++i) s += st.c0[i] + st.c1[i] + st.c2[i] + st.c3[i];
  for (int j = 0; j < 8; ++j) s += st.x[j];
  out[blockIdx.x * blockDim.x + threadIdx.x] = s;
  if (lane == 0) cycles[blockIdx.x * 8 + wv] = t1 - t0;
}

// LDS read rate: 8 wavefronts per workgroup, each lane reading 16 loads per
// iteration from the first 64 KB of an LDS array at conflict-free addresses (consecutive
// lanes, consecutive 16- or 8-byte pieces), folded into one word.  Mode 0:
// ds_read_b128; 1: ds_read_b64; 2: ds_read_b64_tr_b16.  Records each
// wavefront's s_memtime cycles.
template <int MODE>
__global__ __launch_bounds__(512, 1) void lds_kernel(int iters, uint32_t* __restrict__ out,
                                                     long long* __restrict__ cycles) {
  typedef short i16x4 __attribute__((ext_vector_type(4)));
  typedef __attribute__((address_space(3))) char lds_c;
  __shared__ __attribute__((aligned(16))) uint32_t buf[24576];   // 96 KB: one workgroup per CU
  for (int i = threadIdx.x; i < 24576; i += blockDim.x) buf[i] = i * 2654435761u;
  __syncthreads();
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const uint32_t step = MODE == 0 ? 16u : 8u;
  const uint32_t base = ((wv * 64 + lane) * step) & 0xffffu;
  uint32_t acc = 0u;
  const long long t0 = clock64();
  for (int it = 0; it < iters; ++it) {
    asm volatile("" ::: "memory");
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const uint32_t ad = (base + r * 4096u) & (MODE == 0 ? 0xfff0u : 0xfff8u);
      const lds_c* pa = (const lds_c*)buf + ad;
      if (MODE == 0) {
        const u32x4 v = *reinterpret_cast<const __attribute__((address_space(3))) u32x4*>(pa);
        acc ^= v[0] ^ v[1] ^ v[2] ^ v[3];
      } else if (MODE == 1) {
        const uint64_t v = *reinterpret_cast<const __attribute__((address_space(3))) uint64_t*>(pa);
        acc ^= static_cast<uint32_t>(v) ^ static_cast<uint32_t>(v >> 29);
      } else {
        const i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) i16x4*)(const_cast<lds_c*>(pa)));
        acc ^= static_cast<uint32_t>(v[0]) ^ (static_cast<uint32_t>(v[1]) << 3) ^
               (static_cast<uint32_t>(v[2]) << 7) ^ (static_cast<uint32_t>(v[3]) << 11);
      }
    }
  }
  const long long t1 = clock64();
  out[blockIdx.x * blockDim.x + threadIdx.x] = acc;
  if (lane == 0) cycles[blockIdx.x * 8 + wv] = t1 - t0;
}

}  // namespace

extern "C" {

int sink_attn_peaks_read(const void* src, size_t bytes, uint32_t* out, int32_t grid, void* stream) {
  if (src == nullptr || out == nullptr || grid < 1 || bytes % 16 != 0) return 1;
  hipLaunchKernelGGL(read_kernel, dim3(grid), dim3(256), 0, static_cast<hipStream_t>(stream),
                     static_cast<const u32x4*>(src), bytes / 16, out);
  return hipGetLastError() == hipSuccess ? 0 : 4;
}

int sink_attn_peaks_mfma(int32_t iters, float* out, int32_t grid, void* stream) {
  if (out == nullptr || grid < 1 || iters < 1) return 1;
  hipLaunchKernelGGL(mfma_kernel, dim3(grid), dim3(256), 0, static_cast<hipStream_t>(stream), iters, out);
  return hipGetLastError() == hipSuccess ? 0 : 4;
}

int sink_attn_peaks_exp(int32_t iters, float* out, int32_t grid, void* stream) {
  if (out == nullptr || grid < 1 || iters < 1) return 1;
  hipLaunchKernelGGL(exp_kernel, dim3(grid), dim3(256), 0, static_cast<hipStream_t>(stream), iters, out);
  return hipGetLastError() == hipSuccess ? 0 : 4;
}

int sink_attn_peaks_coissue(int32_t mode, int32_t iters, float* out, long long* cycles, int32_t grid,
                            void* stream) {
  if (out == nullptr || cycles == nullptr || grid < 1 || iters < 1 || mode < 0 || mode > 3) return 1;
  hipStream_t st = static_cast<hipStream_t>(stream);
  switch (mode) {
    case 0: hipLaunchKernelGGL(coissue_kernel<0>, dim3(grid), dim3(512), 0, st, iters, out, cycles); break;
    case 1: hipLaunchKernelGGL(coissue_kernel<1>, dim3(grid), dim3(512), 0, st, iters, out, cycles); break;
    case 2: hipLaunchKernelGGL(coissue_kernel<2>, dim3(grid), dim3(512), 0, st, iters, out, cycles); break;
    default: hipLaunchKernelGGL(coissue_kernel<3>, dim3(grid), dim3(512), 0, st, iters, out, cycles); break;
  }
  return hipGetLastError() == hipSuccess ? 0 : 4;
}

int sink_attn_peaks_lds(int32_t mode, int32_t iters, uint32_t* out, long long* cycles, int32_t grid,
                        void* stream) {
  if (out == nullptr || cycles == nullptr || grid < 1 || iters < 1 || mode < 0 || mode > 2) return 1;
  hipStream_t st = static_cast<hipStream_t>(stream);
  switch (mode) {
    case 0: hipLaunchKernelGGL(lds_kernel<0>, dim3(grid), dim3(512), 0, st, iters, out, cycles); break;
    case 1: hipLaunchKernelGGL(lds_kernel<1>, dim3(grid), dim3(512), 0, st, iters, out, cycles); break;
    default: hipLaunchKernelGGL(lds_kernel<2>, dim3(grid), dim3(512), 0, st, iters, out, cycles); break;
  }
  return hipGetLastError() == hipSuccess ? 0 : 4;
}

}  // extern "C"
