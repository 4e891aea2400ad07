// Device-side helpers shared by the kernels: vector types, bf16 conversion,
// the valid-key predicate and the key-tile schedule.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "internal.h"

namespace sa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kInf = __builtin_inff();
constexpr int kBlock = SINK_ATTN_BLOCK_SIZE;

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}
// Round to nearest even (finite inputs; NaN keeps a quiet NaN).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  __bf16 h = static_cast<__bf16>(f);
  return __builtin_bit_cast(uint16_t, h);
}

template <typename T> struct Elem;
template <> struct Elem<float> {
  static __device__ __forceinline__ float load(const void* p, size_t i) {
    return static_cast<const float*>(p)[i];
  }
  static __device__ __forceinline__ void store(void* p, size_t i, float v) {
    static_cast<float*>(p)[i] = v;
  }
};
template <> struct Elem<uint16_t> {
  static __device__ __forceinline__ float load(const void* p, size_t i) {
    return bf16_to_f32(static_cast<const uint16_t*>(p)[i]);
  }
  static __device__ __forceinline__ void store(void* p, size_t i, float v) {
    static_cast<uint16_t*>(p)[i] = f32_to_bf16(v);
  }
};

// Sample containing packed token t (cu is nondecreasing, cu[0] = 0).
__device__ __forceinline__ int find_sample(const int32_t* cu, int batch, int t) {
  int lo = 0, hi = batch - 1;
  while (lo < hi) {
    int mid = (lo + hi + 1) >> 1;
    if (cu[mid] <= t) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// First block_indices row of sample b: rows are packed sample by sample,
// ceil(L / kBlock) rows per sample.
__device__ __forceinline__ int q_block_offset(const int32_t* cu, int b) {
  int off = 0;
  for (int i = 0; i < b; ++i) off += (cu[i + 1] - cu[i] + kBlock - 1) / kBlock;
  return off;
}

// Causal order plus the StreamingLLM window: query i sees key j iff j <= i
// and, with a window, j is one of the first n_sink tokens or i - j < window.
// (Sample-local indices; block selection is checked per block.)
__device__ __forceinline__ bool key_visible(int i, int j, int n_sink, int window) {
  return j <= i && (window <= 0 || j < n_sink || i - j < window);
}

// Whether entry e of a row is the first occurrence of its block id.
__device__ __forceinline__ bool first_occurrence(const int32_t* row, int e) {
  int kb = row[e];
  for (int x = 0; x < e; ++x)
    if (row[x] == kb) return false;
  return true;
}

// ---------------------------------------------------------------------------
// Key-tile schedule of a group of query rows [p0, p1) (sample-local, p1 <= L)
// for 64-key tiles, without block selection: the union of the first-token
// tiles and the window tiles, or every causal tile when there is no window.
// Ranges: [0, r0_end) and [r1_begin, r1_end), r0_end <= r1_begin.
// ---------------------------------------------------------------------------
struct TileRanges {
  int r0_end, r1_begin, r1_end;
  __device__ __forceinline__ int count() const { return r0_end + (r1_end - r1_begin); }
  __device__ __forceinline__ int at(int n) const { return n < r0_end ? n : r1_begin + (n - r0_end); }
};

__device__ __forceinline__ TileRanges window_tiles(int p0, int p1, int n_sink, int window, int bn) {
  TileRanges r;
  int last = (p1 - 1) / bn;             // causal: keys <= p1 - 1
  if (window <= 0) {
    r.r0_end = 0; r.r1_begin = 0; r.r1_end = last + 1;
    return r;
  }
  int wfirst = p0 - window + 1;         // oldest key in any row's window
  int w_tile = wfirst <= 0 ? 0 : wfirst / bn;
  int s_end = n_sink > 0 ? (n_sink - 1) / bn + 1 : 0;
  if (s_end > last + 1) s_end = last + 1;
  if (w_tile <= s_end) {
    r.r0_end = 0; r.r1_begin = 0; r.r1_end = last + 1;
  } else {
    r.r0_end = s_end; r.r1_begin = w_tile; r.r1_end = last + 1;
  }
  return r;
}

// Per-tile classification for rows [p0, p1) against keys [k0, k0 + bn):
// 0 = no valid pair, 1 = every pair valid, 2 = mixed (needs the element mask).
// Keys at or beyond L are never valid; callers pass p1 <= L.
__device__ __forceinline__ int classify_tile(int p0, int p1, int k0, int bn, int n_sink,
                                             int window) {
  int k1 = k0 + bn - 1;
  if (k0 > p1 - 1) return 0;                          // all keys in the future
  if (window > 0) {
    bool any = (k0 < n_sink) || (p0 - k1 < window);
    if (!any) return 0;
    bool all_win = (k1 < n_sink) || (p1 - 1 - k0 < window);
    if (k1 <= p0 && all_win) return 1;
    return 2;
  }
  return k1 <= p0 ? 1 : 2;
}

}  // namespace sa
