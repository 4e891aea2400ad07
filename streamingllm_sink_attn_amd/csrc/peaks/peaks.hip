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

}  // extern "C"
