// Backward pieces shared by the generic and MFMA paths:
//   * preprocess: Delta = rowsum(dO * O_new), L_new = log(e^{L_orig} + e^{a_h}),
//     p_sink = e^{a_h - L_new} and the per-row sink-gradient term
//     -Delta * p_sink ("Attention Sink, Learnable Sink and dsink" s7 boxed
//     equation; s10 prefers e^{sink - lse_total} over 1 - s near s = 1);
//   * the reverse block lists (per KV block: the query blocks selecting it),
//     so that a KV-major backward visits each (KV block, query block) pair
//     once and never adds the sink term per visit (s10), built through a
//     selection bit matrix so the lists come out sorted;
//   * finish: dsink as a fixed-order sum of the per-row terms (deterministic),
//     and float32 accumulators converted to the output dtype.
#include "common.cuh"

namespace sa {

// 16 lanes per (token, head) row, 16-byte chunks.
template <typename T>
__global__ __launch_bounds__(256) void bwd_preprocess_kernel(Prefill p, const void* __restrict__ o,
                                                             const float* __restrict__ lse,
                                                             const void* __restrict__ dout,
                                                             BwdWork w) {
  constexpr int kPerChunk = 16 / sizeof(T);
  const int D = p.d;
  const int nchunks = D / kPerChunk;
  const size_t R = static_cast<size_t>(p.total) * p.hq;
  const int sub = threadIdx.x & 15;
  const size_t rows_per_step = static_cast<size_t>(gridDim.x) * (blockDim.x / 16);
  for (size_t row = static_cast<size_t>(blockIdx.x) * (blockDim.x / 16) + threadIdx.x / 16; row < R;
       row += rows_per_step) {
    float acc = 0.f;
    for (int c = sub; c < nchunks; c += 16) {
      const size_t off = row * D + static_cast<size_t>(c) * kPerChunk;
      // read once here: non-temporal, so the stream does not displace the
      // tiles the backward kernels reuse from the caches
      u32x4 ov = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(static_cast<const T*>(o) + off));
      u32x4 dv = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(static_cast<const T*>(dout) + off));
      if constexpr (sizeof(T) == 4) {
#pragma unroll
        for (int e = 0; e < 4; ++e) acc += __uint_as_float(ov[e]) * __uint_as_float(dv[e]);
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          acc += __uint_as_float(ov[e] << 16) * __uint_as_float(dv[e] << 16);
          acc += __uint_as_float(ov[e] & 0xffff0000u) * __uint_as_float(dv[e] & 0xffff0000u);
        }
      }
    }
#pragma unroll
    for (int off = 8; off >= 1; off >>= 1) acc += __shfl_xor(acc, off, 16);
    if (sub == 0) {
      const int h = static_cast<int>(row % p.hq);
      const float L = lse[row];
      float lnew, ps;
      if (p.sink != nullptr) {
        const float a = p.sink[h];
        if (L == -kInf) {
          lnew = a;
        } else {
          const float mx = fmaxf(L, a);
          lnew = mx + log1pf(expf(-fabsf(L - a)));
        }
        ps = expf(a - lnew);
      } else {
        lnew = (L == -kInf) ? kInf : L;   // +inf makes every recomputed P exactly 0
        ps = 0.f;
      }
      w.delta[row] = acc;
      w.lnew[row] = lnew * kLog2e;         // kept in log2 units for exp2
      w.dsink_terms[row] = -acc * ps;
    }
  }
}

__global__ __launch_bounds__(256) void fill_zero_kernel(float* __restrict__ ptr, size_t n) {
  const size_t stride = static_cast<size_t>(gridDim.x) * blockDim.x * 4;
  for (size_t i = (static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x) * 4; i < n; i += stride) {
    if (i + 4 <= n) {
      *reinterpret_cast<f32x4*>(ptr + i) = f32x4{0.f, 0.f, 0.f, 0.f};
    } else {
      for (size_t e = i; e < n; ++e) ptr[e] = 0.f;
    }
  }
}

static int grid_for(size_t work, int per_block) {
  size_t g = (work + per_block - 1) / per_block;
  if (g > 8192) g = 8192;
  if (g < 1) g = 1;
  return static_cast<int>(g);
}

__global__ __launch_bounds__(256) void fill_zero_bytes_kernel(uint8_t* __restrict__ ptr, size_t n) {
  const size_t stride = static_cast<size_t>(gridDim.x) * blockDim.x;
  for (size_t i = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n; i += stride)
    ptr[i] = 0;
}

hipError_t launch_fill_zero(float* ptr, size_t n, hipStream_t st) {
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(fill_zero_kernel, dim3(grid_for(n, 1024)), dim3(256), 0, st, ptr, n);
  return hipGetLastError();
}

hipError_t launch_fill_zero_bytes(uint8_t* ptr, size_t n, hipStream_t st) {
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(fill_zero_bytes_kernel, dim3(grid_for(n, 256)), dim3(256), 0, st, ptr, n);
  return hipGetLastError();
}

hipError_t launch_bwd_preprocess(const Prefill& p, const void* o, const float* lse,
                                 const void* dout, const BwdWork& w, bool zero_dkv, hipStream_t st) {
  if (p.total == 0) return hipSuccess;
  const size_t R = static_cast<size_t>(p.total) * p.hq;
  const int grid = grid_for(R, 16);
  if (p.dtype == SINK_ATTN_F32)
    hipLaunchKernelGGL(bwd_preprocess_kernel<float>, dim3(grid), dim3(256), 0, st, p, o, lse, dout, w);
  else
    hipLaunchKernelGGL(bwd_preprocess_kernel<uint16_t>, dim3(grid), dim3(256), 0, st, p, o, lse,
                       dout, w);
  if (zero_dkv) {
    const size_t n = static_cast<size_t>(p.total) * p.hkv * p.d;
    hipLaunchKernelGGL(fill_zero_kernel, dim3(grid_for(n, 1024)), dim3(256), 0, st, w.dk_acc, n);
    hipLaunchKernelGGL(fill_zero_kernel, dim3(grid_for(n, 1024)), dim3(256), 0, st, w.dv_acc, n);
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Reverse block lists.  For global KV block kbg (= sample offset + local kb)
// and KV head g: the sample-local query blocks qb >= kb whose row selects kb,
// in increasing qb order (so the fill is deterministic).
// ---------------------------------------------------------------------------
__device__ __forceinline__ void locate_block(const int32_t* cu, int batch, int kbg, int* b_out,
                                             int* off_out) {
  int off = 0;
  for (int b = 0; b < batch; ++b) {
    const int n = (cu[b + 1] - cu[b] + kBlock - 1) / kBlock;
    if (kbg < off + n) { *b_out = b; *off_out = off; return; }
    off += n;
  }
  *b_out = batch - 1; *off_out = off;
}

// Bit matrix of the selections: word w of (global KV block kbg, KV head g)
// holds bit qb % 32 for every sample-local query block qb in [32w, 32w + 32)
// whose row selects the KV block (qb >= kb only; duplicates collapse).  One
// thread per block-list entry.
__global__ __launch_bounds__(256) void block_bits_kernel(Prefill p, BwdWork w, int words) {
  const size_t idx = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (idx >= static_cast<size_t>(p.nqb) * p.hkv * p.max_blocks) return;
  const int e = static_cast<int>(idx % p.max_blocks);
  const int g = static_cast<int>((idx / p.max_blocks) % p.hkv);
  const int qbg = static_cast<int>(idx / (static_cast<size_t>(p.max_blocks) * p.hkv));
  int b, off;
  locate_block(p.cu, p.batch, qbg, &b, &off);
  const int qb = qbg - off;
  const int nqb_b = (p.cu[b + 1] - p.cu[b] + kBlock - 1) / kBlock;
  const int kb = p.blocks[(static_cast<size_t>(qbg) * p.hkv + g) * p.max_blocks + e];
  if (kb < 0 || kb > qb || kb >= nqb_b || (qb >> 5) >= words) return;
  atomicOr(w.csr_bits + (static_cast<size_t>(off + kb) * p.hkv + g) * words + (qb >> 5), 1u << (qb & 31));
}

// Per (KV block, KV head): the list length (kFill = false), or the list itself
// in increasing query-block order (kFill = true, deterministic).
template <bool kFill>
__global__ __launch_bounds__(256) void block_csr_kernel(Prefill p, BwdWork w, int words) {
  const int idx = blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= p.nqb * p.hkv) return;
  const uint32_t* bits = w.csr_bits + static_cast<size_t>(idx) * words;
  if (!kFill) {
    int n = 0;
    for (int i = 0; i < words; ++i) n += __builtin_popcount(bits[i]);
    w.csr_off[idx + 1] = n;
    return;
  }
  int32_t* dst = w.csr_idx + w.csr_off[idx];
  int n = 0;
  for (int i = 0; i < words; ++i) {
    uint32_t m = bits[i];
    while (m != 0u) {
      dst[n++] = 32 * i + __builtin_ctz(m);
      m &= m - 1u;
    }
  }
}

// Exclusive scan of csr_off[1..n] in place (csr_off[0] = 0), one workgroup.
__global__ __launch_bounds__(1024) void csr_scan_kernel(int32_t* off, int n) {
  __shared__ int32_t part[1024];
  const int tid = threadIdx.x;
  const int per = (n + 1023) / 1024;
  const int a = tid * per, e = min(n, a + per);
  int32_t sum = 0;
  for (int i = a; i < e; ++i) sum += off[i + 1];
  part[tid] = sum;
  __syncthreads();
  for (int d = 1; d < 1024; d <<= 1) {
    int32_t v = tid >= d ? part[tid - d] : 0;
    __syncthreads();
    part[tid] += v;
    __syncthreads();
  }
  int32_t run = tid ? part[tid - 1] : 0;
  for (int i = a; i < e; ++i) {
    const int32_t c = off[i + 1];
    off[i + 1] = run + c;
    run += c;
  }
  if (tid == 0) off[0] = 0;
}

hipError_t launch_scan(int32_t* off, int n, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(csr_scan_kernel, dim3(1), dim3(1024), 0, st, off, n);
  return hipGetLastError();
}

int block_csr_words(const Prefill& p) {
  const int max_nqb = (p.max_seqlen + kBlock - 1) / kBlock;
  return (max_nqb + 31) / 32;
}

hipError_t launch_block_csr(const Prefill& p, const BwdWork& w, hipStream_t st) {
  const int n = p.nqb * p.hkv;
  if (n == 0) return hipSuccess;
  const int words = block_csr_words(p);
  const size_t nbits = static_cast<size_t>(n) * words;
  hipLaunchKernelGGL(fill_zero_kernel, dim3(grid_for(nbits, 1024)), dim3(256), 0, st,
                     reinterpret_cast<float*>(w.csr_bits), nbits);
  const size_t entries = static_cast<size_t>(n) * p.max_blocks;
  hipLaunchKernelGGL(block_bits_kernel, dim3(static_cast<unsigned>((entries + 255) / 256)), dim3(256), 0,
                     st, p, w, words);
  const int grid = (n + 255) / 256;
  hipLaunchKernelGGL(block_csr_kernel<false>, dim3(grid), dim3(256), 0, st, p, w, words);
  hipLaunchKernelGGL(csr_scan_kernel, dim3(1), dim3(1024), 0, st, w.csr_off, n);
  hipLaunchKernelGGL(block_csr_kernel<true>, dim3(grid), dim3(256), 0, st, p, w, words);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Finish: dsink[h] = sum_t terms[t, h] in a fixed order; accumulators -> dtype.
// ---------------------------------------------------------------------------
// Column sums in two passes, both in a fixed order: per slab of kDsinkRows
// rows, partial sums of every column (reads are contiguous across the
// columns of a row), then per column the sum of the slabs' partials, times a
// scale.  dsink uses them on the per-row terms (scale 1); the head importance
// on a per-row gate (scale 1 / rows).
constexpr int kDsinkRows = 64;

__global__ __launch_bounds__(256) void column_sum_partial_kernel(const float* __restrict__ terms, int T,
                                                            int hq, float* __restrict__ part) {
  __shared__ float red[256];
  const int t0 = blockIdx.x * kDsinkRows;
  const int t1 = min(T, t0 + kDsinkRows);
  for (int hc = 0; hc < hq; hc += 256) {
    const int ncol = min(256, hq - hc);
    const int rpp = 256 / ncol;                       // rows per pass
    const int r = threadIdx.x / ncol, h = threadIdx.x % ncol;
    float acc = 0.f;
    if (r < rpp)
      for (int t = t0 + r; t < t1; t += rpp) acc += terms[static_cast<size_t>(t) * hq + hc + h];
    red[threadIdx.x] = acc;
    __syncthreads();
    if (threadIdx.x < ncol) {
      float sum = 0.f;
      for (int k = 0; k < rpp; ++k) sum += red[k * ncol + threadIdx.x];
      part[static_cast<size_t>(blockIdx.x) * hq + hc + threadIdx.x] = sum;
    }
    __syncthreads();
  }
}

// One workgroup per head: thread t sums slabs t, t + 256, ... in order, then
// a fixed tree over the 256 partial sums.
__global__ __launch_bounds__(256) void column_sum_final_kernel(const float* __restrict__ part, int nslab,
                                                               int hq, float scale,
                                                               float* __restrict__ out) {
  __shared__ float red[256];
  const int h = blockIdx.x;
  float acc = 0.f;
  for (int k = threadIdx.x; k < nslab; k += 256) acc += part[static_cast<size_t>(k) * hq + h];
  red[threadIdx.x] = acc;
  __syncthreads();
  for (int st = 128; st > 0; st >>= 1) {
    if (threadIdx.x < st) red[threadIdx.x] += red[threadIdx.x + st];
    __syncthreads();
  }
  if (threadIdx.x == 0) out[h] = red[0] * scale;
}

int dsink_slabs(int total) { return (total + kDsinkRows - 1) / kDsinkRows; }

hipError_t launch_column_sum(const float* x, int rows, int cols, float scale, float* part,
                             float* out, hipStream_t st) {
  if (cols <= 0) return hipSuccess;
  const int nslab = dsink_slabs(rows);
  if (nslab > 0)
    hipLaunchKernelGGL(column_sum_partial_kernel, dim3(nslab), dim3(256), 0, st, x, rows, cols, part);
  hipLaunchKernelGGL(column_sum_final_kernel, dim3(cols), dim3(256), 0, st, part, nslab, cols, scale,
                     out);
  return hipGetLastError();
}

template <typename T>
__global__ __launch_bounds__(256) void convert_kernel(const float* __restrict__ src, void* dst,
                                                      size_t n) {
  const size_t stride = static_cast<size_t>(gridDim.x) * blockDim.x * 4;
  for (size_t i = (static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x) * 4; i < n; i += stride) {
    if (i + 4 <= n) {
      f32x4 x = *reinterpret_cast<const f32x4*>(src + i);
      if constexpr (sizeof(T) == 4) {
        *reinterpret_cast<f32x4*>(static_cast<float*>(dst) + i) = x;
      } else {
        uint16_t* d = static_cast<uint16_t*>(dst) + i;
        u32x2 packed;
        packed[0] = static_cast<uint32_t>(f32_to_bf16(x[0])) | (static_cast<uint32_t>(f32_to_bf16(x[1])) << 16);
        packed[1] = static_cast<uint32_t>(f32_to_bf16(x[2])) | (static_cast<uint32_t>(f32_to_bf16(x[3])) << 16);
        *reinterpret_cast<u32x2*>(d) = packed;
      }
    } else {
      for (size_t e = i; e < n; ++e) Elem<T>::store(dst, e, src[e]);
    }
  }
}

template <typename T>
static void convert(const float* src, void* dst, size_t n, hipStream_t st) {
  if (n == 0) return;
  hipLaunchKernelGGL(convert_kernel<T>, dim3(grid_for(n, 1024)), dim3(256), 0, st, src, dst, n);
}

hipError_t launch_bwd_finish(const Prefill& p, const BwdWork& w, float* dsink, void* dk, void* dv,
                             bool dkv_from_acc, hipStream_t st) {
  if (dsink != nullptr) launch_column_sum(w.dsink_terms, p.total, p.hq, 1.f, w.dsink_part, dsink, st);
  const size_t nkv = static_cast<size_t>(p.total) * p.hkv * p.d;
  const bool f32 = p.dtype == SINK_ATTN_F32;
  if (dkv_from_acc) {
    if (f32) {
      convert<float>(w.dk_acc, dk, nkv, st);
      convert<float>(w.dv_acc, dv, nkv, st);
    } else {
      convert<uint16_t>(w.dk_acc, dk, nkv, st);
      convert<uint16_t>(w.dv_acc, dv, nkv, st);
    }
  }
  return hipGetLastError();
}

}  // namespace sa
