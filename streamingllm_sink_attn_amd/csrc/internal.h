// Internal declarations shared by the C-ABI layer and the kernel sources.
// Host-visible structs hold only plain pointers and sizes; kernels take them
// by value.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "sink_attn.h"

namespace sa {

// Everything a prefill kernel needs to know about the problem.
struct Prefill {
  const int32_t* cu;          // [batch+1]
  int batch, total, max_seqlen;
  int hq, hkv, d, dtype;
  float scale;
  int n_sink, window;         // window <= 0: no window (n_sink ignored)
  const int32_t* blocks;      // [nqb, hkv, max_blocks] or nullptr
  int nqb, max_blocks;
  const float* sink;          // [hq] or nullptr
  // [batch] or nullptr: rows before qstart[b] of sample b are not needed
  // (a workgroup whose rows all lie before it exits; the forward only).
  const int32_t* qstart = nullptr;
  // [batch] or nullptr: the Q, O, LSE and s rows of sample b start at row
  // qo_base[b] instead of cu[b] (K and V stay at cu[b]); the forward only.
  const int32_t* qo_base = nullptr;
};

// Backward workspace carve-up (float32 unless noted).
struct BwdWork {
  float* delta;      // [T, Hq]  rowsum(dO * O)
  float* lnew;       // [T, Hq]  log2(e) * log(Z + e^a) (or of L_orig; +inf for empty rows without a sink)
  float* dsink_terms;// [T, Hq]  -Delta * p_sink per row
  float* dsink_part; // [ceil(T/64), Hq] per-slab partial sums of the terms
  float* dk_acc;     // generic path: [T, Hkv, D]; MFMA path: [max split tiles, 64, D] (split key tiles)
  float* dv_acc;     // as dk_acc
  int32_t* csr_off;  // [nqb*Hkv + 1]  (block mode) per (KV block, KV head) list offsets
  int32_t* csr_idx;  // [nqb*Hkv*max_blocks] query blocks selecting each KV block
  uint32_t* csr_bits;// [nqb*Hkv*words] selection bit matrix the lists are built from
  int32_t* plan;     // [batch*nkt*Hkv + 1] (MFMA path) chunks per key tile -> offsets
  int32_t* split_slot;// [batch*nkt*Hkv + 1] (MFMA path) accumulator slot of each split key tile
  int max_split;     // (MFMA path) slots of dk_acc / dv_acc
  int32_t* queues;   // [8] work counters of the key-major pass
};

struct Decode {
  const int32_t* cache_seqlens;
  int batch, slots, hq, hkv, d, dtype;
  float scale;
  const float* sink;
  int splits;
};

// Rolling KV cache of StreamingLLM: n_sink first tokens plus a ring of the
// last `window` tokens; quantized = the ring in 8-bit e4m3 with per-(slot,
// KV head) float32 scales, the first tokens bfloat16.
struct KvCache {
  int batch, n_sink, window, hkv, d, quantized;
  void* k;                    // !quantized: bf16 [B, n_sink + window, Hkv, D]
  void* v;
  void* sink_k;               // quantized: bf16 [B, n_sink, Hkv, D]
  void* sink_v;
  uint8_t* win_k;             // quantized: e4m3 [B, window, Hkv, D]
  uint8_t* win_v;
  float* win_k_scale;         // quantized: [B, Hkv, window]
  float* win_v_scale;
};

// Keys and values of a chunked prefill read in place (bf16 cache, D = 128):
// sample 2b of the forward launch is stream b's keys in position order
// [kept first tokens | ring tokens, oldest first | chunk]; sample 2b + 1 is
// padding with no query row.  Key tiles inside one run are read from the
// cache or the chunk; the few tiles holding a seam (see stream_rows.cuh)
// are copied first to the staging tiles sk / sv.
constexpr int kSeamSlots = 3;
constexpr int kSeamRows = 64;
struct CacheKv {
  const uint16_t* k;          // bf16 [B, slots, Hkv, D]
  const uint16_t* v;
  const uint16_t* kn;         // bf16 [B, chunk, Hkv, D]
  const uint16_t* vn;
  uint16_t* sk;               // bf16 [B, 3, 64, Hkv, D] staged seam tiles
  uint16_t* sv;
  const int32_t* n_seen;      // [B] tokens each stream held before the chunk
  int batch, hkv, slots, n_sink, window, chunk;
};

// ---- launchers (each returns hipGetLastError() of its launches) ----
// gate0: float32 [T, Hq] first-token gate, or nullptr (not computed).
hipError_t launch_fwd_generic(const Prefill& p, const void* q, const void* k, const void* v,
                              void* o, float* lse, float* s, float* gate0, hipStream_t st);
hipError_t launch_fwd_mfma(const Prefill& p, const void* q, const void* k, const void* v,
                           void* o, float* lse, float* s, float* gate0, hipStream_t st);
bool fwd_mfma_supported(const Prefill& p);
// The matrix-core forward with K and V read in place from a rolling cache and
// a chunk (p describes the 2B samples; p.qstart and p.qo_base are set).
hipError_t launch_fwd_mfma_cache(const Prefill& p, const CacheKv& ckv, const void* q, void* o, float* lse,
                                 float* s, hipStream_t st);

// zero_dkv: also zero the float32 dK/dV accumulators of every row (generic path).
hipError_t launch_bwd_preprocess(const Prefill& p, const void* o, const float* lse,
                                 const void* dout, const BwdWork& w, bool zero_dkv, hipStream_t st);
hipError_t launch_bwd_generic(const Prefill& p, const void* q, const void* k, const void* v,
                              const void* dout, const BwdWork& w, void* dq, hipStream_t st);
// Key-major dK/dV pass: its planning (chunk plan, split-slot scan, zeroed
// split accumulators; reads only the inputs and the reverse block lists),
// then the persistent kernel and the split-tile finish; and the query-major
// dQ kernel.  dK/dV and dQ read only the inputs and the preprocess's L_new
// and Delta and write disjoint outputs, so they may run on two streams at
// once, and the planning beside the preprocess.
hipError_t launch_bwd_dkdv_plan(const Prefill& p, const BwdWork& w, void* dk, void* dv, hipStream_t st);
hipError_t launch_bwd_dkdv(const Prefill& p, const void* q, const void* k, const void* v,
                           const void* dout, const BwdWork& w, void* dk, void* dv, hipStream_t st);
hipError_t launch_bwd_dq(const Prefill& p, const void* q, const void* k, const void* v,
                         const void* dout, const BwdWork& w, void* dq, hipStream_t st);
bool bwd_mfma_supported(const Prefill& p);
int bwd_num_tiles(const Prefill& p);        // key tiles of the key-major pass
// Upper bound on the key tiles whose work is split over several work items
// (they accumulate dK/dV in float32 slots); a tile beyond the bound is not
// split (correct, only less balanced).
int bwd_max_split_tiles(const Prefill& p);
hipError_t launch_block_csr(const Prefill& p, const BwdWork& w, hipStream_t st);
int block_csr_words(const Prefill& p);      // 32-bit words per reverse-list bit row
int dsink_slabs(int total);                 // row slabs of the dsink reduction
// out[c] = scale * sum_r x[r, c] over the rows of x [rows, cols], in a fixed
// order (per-slab partials in part [dsink_slabs(rows), cols], then slabs in
// order): deterministic.
hipError_t launch_column_sum(const float* x, int rows, int cols, float scale, float* part,
                             float* out, hipStream_t st);
hipError_t launch_bwd_finish(const Prefill& p, const BwdWork& w, float* dsink, void* dk, void* dv,
                             bool dkv_from_acc, hipStream_t st);

hipError_t launch_decode(const Decode& p, const void* q, const void* kc, const void* vc,
                         void* o, float* lse, float* s, float* ws, hipStream_t st);
int decode_auto_splits(const Decode& p);
bool decode_mfma_supported(const Decode& p);

hipError_t launch_visit_map(const Prefill& p, uint8_t* out, hipStream_t st);

// Append `chunk` tokens per sequence (k_new, v_new bf16 [B, chunk, Hkv, D],
// stream positions n_seen[b] + c) into the cache.
// Chunked prefill against the cache: the packed per-sequence samples (K, V,
// and Q rows when qp is set; cu of 2*batch + 1 entries, qstart and qo_base of
// 2*batch) and the copy of the chunk rows' outputs back to [batch, chunk, ...]
// order (for the generic forward, which reads and writes packed rows).
hipError_t launch_kvcache_prefill_gather(const KvCache& c, const void* q, const void* k_new,
                                         const void* v_new, int chunk, int hq, const int32_t* n_seen,
                                         int lmax, void* kp, void* vp, void* qp, int32_t* cu,
                                         int32_t* qstart, int32_t* qo_base, hipStream_t st);
// A chunked prefill whose keys are read in place: the sample bounds cu
// (2B + 1), qstart and qo_base (2B each), as the gather writes them, and the
// staged seam tiles of ckv.
hipError_t launch_kvcache_prefill_plan(const CacheKv& ckv, int lmax, int32_t* cu, int32_t* qstart,
                                       int32_t* qo_base, hipStream_t st);
hipError_t launch_kvcache_prefill_scatter(const KvCache& c, int chunk, int hq, const int32_t* n_seen,
                                          int lmax, const void* op, const float* lsep, const float* sp,
                                          void* o, float* lse, float* s, hipStream_t st);
hipError_t launch_kvcache_append(const KvCache& c, const void* k_new, const void* v_new, int chunk,
                                 const int32_t* n_seen, hipStream_t st);
// Decode over the 8-bit cache: p.cache_seqlens holds the tokens appended so
// far per sequence (the current one included); p.slots is unused.
hipError_t launch_kvcache_decode_q8(const Decode& p, const KvCache& c, const void* q, void* o,
                                    float* lse, float* s, float* ws, hipStream_t st);
int kvcache_q8_auto_splits(const Decode& p, const KvCache& c);

// Records the detail sink_attn_last_error() returns on this thread; returns
// status.
int set_last_error(int status, const char* fmt, ...);

// Fill kernels (used instead of hipMemsetAsync so callers may capture graphs).
hipError_t launch_fill_zero(float* ptr, size_t n, hipStream_t st);
hipError_t launch_fill_zero_bytes(uint8_t* ptr, size_t n, hipStream_t st);

}  // namespace sa
