/*
 * sink_attn.h - C ABI of the MI355X (gfx950) sink-attention library.
 *
 * Scaled-dot-product attention with a per-query-head learnable sink logit a_h
 * that adds e^{a_h} to the softmax denominator, as derived in "Attention Sink,
 * Learnable Sink and dsink: from the meaning of the output to the backward
 * gradient" (notes.kuangjux.top), referred to below as [Notes]:
 *
 *   x_ij   = alpha * <Q_ih, K_j,g(h)>                       [Notes] s1
 *   L_orig = log sum_{j valid} e^{x_ij}                     [Notes] s4
 *   s_ih   = sigma(L_orig - a_h) = Z / (Z + e^{a_h})        [Notes] s4
 *   O_ih   = s_ih * sum_j softmax_j(x_ij) V_j,g(h)          [Notes] s4 (O_new = s O_orig)
 *   dsink_h = -sum_i Delta_ih (1 - s_ih),
 *             Delta_ih = sum_d dO_ihd O_ihd                 [Notes] s7 (boxed)
 *   dQ/dK/dV from dx_ij = P_ij (<dO_ih, V_j> - Delta_ih),
 *             with P built from L_new = log(Z + e^{a_h})    [Notes] s8
 *
 * The valid key set of query i (head h) is: same packed sample, causal order
 * (j <= i), and, when window > 0, either one of the first n_sink tokens of the
 * sample or within the recent window (i - j < window), as StreamingLLM keeps
 * the first tokens plus a recent window ([Notes] s2; "What is Attention Sink?
 * ... StreamingLLM" (model.playoffer.cn), core idea).  With block_indices the
 * selected blocks are further narrowed by the window, causal order and sample
 * boundaries ([Notes] s2, responsibilities of block_indices).
 *
 * Conventions shared by every call:
 *   - All tensors are device pointers, caller-owned, contiguous row-major and
 *     16-byte aligned.  Packed prefill tensors: Q, O, dO, dQ [T, Hq, D];
 *     K, V, dK, dV [T, Hkv, D]; lse, s [T, Hq] float32.
 *   - GQA: query head h reads KV head g(h) = h / (Hq / Hkv); Hq % Hkv == 0.
 *   - dtype SINK_ATTN_BF16: Q/K/V/O/dO/dQ/dK/dV are bfloat16, arithmetic in
 *     float32 (bfloat16 MFMA with float32 accumulation).  SINK_ATTN_F32: all
 *     of them float32.  lse, s, learnable_sink and dsink are always float32.
 *   - The sink logit is used as is: it is not multiplied by softmax_scale, and
 *     it is in natural-log units ([Notes] s7, second pitfall).
 *   - learnable_sink == NULL disables the sink (s = 1 exactly); a value of 0
 *     still adds e^0 = 1 ([Notes] s4).
 *   - lse is L_orig, the log-sum-exp over real keys only, in natural log.  The
 *     backward takes this L_orig and forms L_new itself, so the two are never
 *     mixed ([Notes] s9-10).
 *   - A query with no valid key gets O = 0, lse = -inf and s = 0 with a sink
 *     (s = 1 without); it contributes nothing to any gradient.
 *   - Outputs are overwritten, never accumulated (dQ, dK, dV, dsink included).
 *     dsink is the plain sum over every query row of the call; summing it
 *     across calls or processes is the caller's job ([Notes] s7, s9).
 *   - The library never allocates, frees or synchronises.  Work is enqueued
 *     on `stream` (a hipStream_t; NULL = the null stream).  Scratch memory is
 *     the caller's `workspace`, of at least the size the matching
 *     *_workspace_size() call returns; its contents on entry do not matter
 *     (sink_attn_decode_noalloc uses a fixed static array instead).
 *   - No call reads device memory from the host.  Device-side preconditions
 *     (monotone cu_seqlens with cu_seqlens[0] = 0 and cu_seqlens[batch] =
 *     total_tokens, every length <= max_seqlen, block ids < the sample's block
 *     count, 1 <= cache_seqlens[b] <= slots) are documented, not checked;
 *     breaking them gives unspecified results.
 *   - Every entry point returns a sink_attn_status; nothing aborts and no C++
 *     exception crosses this boundary.  sink_attn_last_error() describes the
 *     last failure on the calling thread.
 */
#ifndef SINK_ATTN_H
#define SINK_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum sink_attn_status {
  SINK_ATTN_OK = 0,
  SINK_ATTN_INVALID_ARGUMENT = 1,    /* NULL required pointer, bad sizes, misalignment, ... */
  SINK_ATTN_UNSUPPORTED = 2,         /* dtype / head_dim / block_size outside what is built */
  SINK_ATTN_WORKSPACE_TOO_SMALL = 3,
  SINK_ATTN_HIP_ERROR = 4            /* a kernel launch failed */
} sink_attn_status;

typedef enum sink_attn_dtype {
  SINK_ATTN_BF16 = 0,
  SINK_ATTN_F32 = 1
} sink_attn_dtype;

/* Largest supported head_dim; head_dim must be a multiple of 8. */
#define SINK_ATTN_MAX_HEAD_DIM 256
/* block_indices blocks are always this many tokens. */
#define SINK_ATTN_BLOCK_SIZE 64

/*
 * Shape and mask of a packed variable-length prefill problem.
 *
 * cu_seqlens     device int32 [batch + 1]: sample b holds packed tokens
 *                [cu_seqlens[b], cu_seqlens[b+1]).
 * batch          number of samples (>= 0; 0 makes every call a no-op).
 * total_tokens   T, host copy of cu_seqlens[batch].
 * max_seqlen     host upper bound on every sample length (sizes the grids).
 * num_q_heads    Hq; num_kv_heads Hkv (Hq % Hkv == 0); head_dim D.
 * dtype          sink_attn_dtype of Q/K/V/O/dO/dQ/dK/dV.
 * softmax_scale  alpha (> 0, finite), usually 1/sqrt(D).
 * n_sink         first tokens of each sample kept visible by the window (>= 0).
 * window         recent-window length W; <= 0 disables the window (and n_sink).
 * block_indices  NULL (dense), or device int32 [num_q_blocks, Hkv, max_blocks]:
 *                row (qb, g) lists the sample-local KV blocks selected for
 *                query block qb and KV head g; rows are ordered by sample, then
 *                by sample-local query block of block_size tokens, so
 *                num_q_blocks = sum_b ceil(L_b / block_size).  Entries are in
 *                [-1, ceil(L_b / block_size)), -1 is padding, duplicates are
 *                allowed and count once.
 * block_size     must be SINK_ATTN_BLOCK_SIZE when block_indices != NULL.
 * learnable_sink device float32 [Hq], or NULL (no sink).
 */
typedef struct sink_attn_prefill_desc {
  const int32_t* cu_seqlens;
  int32_t batch;
  int32_t total_tokens;
  int32_t max_seqlen;
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t head_dim;
  int32_t dtype;
  float softmax_scale;
  int32_t n_sink;
  int32_t window;
  const int32_t* block_indices;
  int32_t num_q_blocks;
  int32_t block_size;
  int32_t max_blocks;
  const float* learnable_sink;
} sink_attn_prefill_desc;

/*
 * One query per sequence against a rolling KV cache.
 *
 * cache_seqlens  device int32 [batch]: slots [0, cache_seqlens[b]) are valid;
 *                NULL = all `slots` valid.  Slots are an unordered set: a ring
 *                buffer keeps the first n_sink tokens and the recent window in
 *                whatever slot order ("Attention Sink" (lijianxiong.space),
 *                H2O section, circular cache), and the current token's K/V is
 *                already in the cache, so no causal or window mask applies.
 * batch, slots   B and S; the caches are [B, S, Hkv, D], q and o [B, Hq, D],
 *                lse and s [B, Hq].
 * num_splits     KV splits per (sequence, KV head) merged by their LSE;
 *                0 = choose automatically.  The result does not depend on it
 *                beyond rounding.
 */
typedef struct sink_attn_decode_desc {
  const int32_t* cache_seqlens;
  int32_t batch;
  int32_t slots;
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t head_dim;
  int32_t dtype;
  float softmax_scale;
  const float* learnable_sink;
  int32_t num_splits;
} sink_attn_decode_desc;

/*
 * StreamingLLM's rolling KV cache ("What is Attention Sink? ... StreamingLLM"
 * (model.playoffer.cn), core idea: the first tokens of the stream (4
 * recommended) stay for good, a sliding window keeps the most recent ones and
 * a new token replaces the oldest window token; "Attention Sink"
 * (lijianxiong.space), H2O section: the recent part as a circular queue).
 * The token at stream position p lives in sink slot p when p < n_sink, else
 * in ring slot (p - n_sink) mod window.
 *
 * quantized = 0: one bfloat16 cache per K and V, [B, n_sink + window, Hkv, D]
 *   (slots [0, n_sink) the first tokens, n_sink + r ring slot r): the layout
 *   sink_attn_decode reads.
 * quantized = 1 (head_dim 128): the first tokens stay bfloat16 and the ring
 *   is 8-bit, as the same page's engineering notes describe for KV-cache
 *   quantisers that keep the first tokens in high precision:
 *     sink_k, sink_v            bfloat16 [B, n_sink, Hkv, D];
 *     win_k, win_v              e4m3 codes [B, window, Hkv, D] (OCP layout: 1
 *                               sign, 4 exponent bits of bias 7, 3 mantissa
 *                               bits; 448 the largest value);
 *     win_k_scale, win_v_scale  float32 [B, Hkv, window]; a ring row's value
 *                               is code * scale, with scale = amax / 448 and
 *                               code = e4m3(x * (448 / amax)) rounded to
 *                               nearest even (a zero row: scale 0, codes 0).
 * All pointers are device memory owned by the caller, 16-byte aligned;
 * unused ones may be NULL.
 */
typedef struct sink_attn_kvcache_desc {
  int32_t batch;
  int32_t n_sink;         /* first tokens kept for good (>= 0) */
  int32_t window;         /* most recent tokens kept in the ring (>= 1) */
  int32_t num_kv_heads;
  int32_t head_dim;       /* multiple of 8 up to SINK_ATTN_MAX_HEAD_DIM; 128 when quantized */
  int32_t quantized;      /* 0 or 1, see above */
  void* k;                /* quantized = 0 */
  void* v;
  void* sink_k;           /* quantized = 1 */
  void* sink_v;
  void* win_k;
  void* win_v;
  float* win_k_scale;
  float* win_v_scale;
} sink_attn_kvcache_desc;

/*
 * Append a chunk of new tokens to every sequence's cache.
 *   k_new, v_new  bfloat16 [B, chunk, Hkv, D]: the new tokens in stream order.
 *   n_seen        device int32 [B] (>= 0, n_seen[b] + chunk < 2^31): tokens
 *                 each stream held before this call; token c of sequence b
 *                 has stream position n_seen[b] + c (a negative count reads
 *                 as 0).
 * Each token is written to its slot (quantized ring rows with their scales),
 * overwriting the token that slot held; a chunk token that a later token of
 * the same chunk would overwrite at once is not written, so no slot has two
 * writers.  The caller advances n_seen by chunk for the next call.
 */
int sink_attn_kvcache_append(const sink_attn_kvcache_desc* cache, const void* k_new,
                             const void* v_new, int32_t chunk, const int32_t* n_seen,
                             void* stream);

/*
 * Decode one query per sequence over its cache: [Notes] s1 and s4 on the
 * slots written so far, split-KV merged by log-sum-exp (as sink_attn_decode).
 *   q         bfloat16 [B, num_q_heads, D].
 *   n_tokens  device int32 [B]: tokens appended to each stream so far, the
 *             current token included; the valid slots are the first
 *             min(n_tokens, n_sink) sink slots and the first
 *             min(max(n_tokens - n_sink, 0), window) ring slots.
 *   o         output bfloat16 [B, num_q_heads, D]; lse, s float32 [B, num_q_heads]
 *             as sink_attn_decode (s may be NULL).
 *   workspace sink_attn_kvcache_decode_workspace_size bytes.
 */
int sink_attn_kvcache_decode(const sink_attn_kvcache_desc* cache, const void* q,
                             int32_t num_q_heads, const int32_t* n_tokens, float softmax_scale,
                             const float* learnable_sink, int32_t num_splits,
                             void* o, float* lse, float* s,
                             void* workspace, size_t workspace_bytes, void* stream);

/*
 * Chunked prefill against the cache: a chunk of `chunk` new tokens per
 * sequence attends, with the sink ([Notes] s1, s4), to the keys StreamingLLM
 * keeps for each of its positions ("What is Attention Sink? ... StreamingLLM"
 * (model.playoffer.cn), core idea: the first n_sink tokens and a sliding
 * window of the most recent ones).  Row c of sequence b is stream position
 * p = n_seen[b] + c and sees key position k when k <= p and (k < n_sink or
 * p - k < window): the cached first tokens and ring tokens (as they were
 * before this chunk) and the chunk's own earlier tokens.  This equals row p
 * of sink_attn_fwd over the whole stream with that n_sink and window.  The
 * 8-bit ring enters as code * scale rounded to bfloat16.
 *   q             bfloat16 [B, chunk, num_q_heads, D].
 *   k_new, v_new  bfloat16 [B, chunk, Hkv, D]: the chunk's keys and values.
 *   n_seen        device int32 [B] (>= 0, n_seen[b] + chunk < 2^31): tokens
 *                 the cache has taken so far (a negative count reads as 0).
 *   o             output bfloat16 [B, chunk, num_q_heads, D]; lse, s float32
 *                 [B, chunk, num_q_heads] as sink_attn_fwd (s may be NULL).
 *   workspace     sink_attn_kvcache_prefill_workspace_size bytes, 256-byte
 *                 aligned: the bounds of the per-sequence samples, and for
 *                 the 8-bit cache or head_dim other than 128 the samples
 *                 themselves (B x (n_sink + window + chunk) packed rows of K
 *                 and V; of Q and O too for head_dim other than 128).  With
 *                 the bfloat16 cache and head_dim 128 the keys and values
 *                 are read in place from the cache and k_new / v_new, and
 *                 the workspace holds only copies of the at most three
 *                 64-row key tiles per sequence that span a seam (first
 *                 tokens to ring, the ring's wrap, ring to chunk).
 * The cache is read, not written: append the chunk afterwards with
 * sink_attn_kvcache_append and the same n_seen (appending first could evict
 * ring tokens the chunk's earlier rows still see).
 */
size_t sink_attn_kvcache_prefill_workspace_size(const sink_attn_kvcache_desc* cache, int32_t chunk,
                                                int32_t num_q_heads);
int sink_attn_check_kvcache_prefill(const sink_attn_kvcache_desc* cache, const void* q,
                                    int32_t num_q_heads, const void* k_new, const void* v_new,
                                    int32_t chunk, const int32_t* n_seen, float softmax_scale,
                                    const void* o, const float* lse, const float* s,
                                    size_t workspace_bytes);
int sink_attn_kvcache_prefill(const sink_attn_kvcache_desc* cache, const void* q, int32_t num_q_heads,
                              const void* k_new, const void* v_new, int32_t chunk,
                              const int32_t* n_seen, float softmax_scale, const float* learnable_sink,
                              void* o, float* lse, float* s, void* workspace, size_t workspace_bytes,
                              void* stream);

/*
 * Forward.  [Notes] s1 (scores, probabilities, output) and s4 (the sink as an
 * output scale).
 *   q, k, v   inputs (layouts above).
 *   o         output [T, Hq, D], dtype of q.
 *   lse       output float32 [T, Hq], L_orig (required: the backward needs it).
 *   s         output float32 [T, Hq] (real-token share, the output scale and
 *             the implicit per-head gate G = sigma(LSE - sink) of "Paper notes:
 *             Attention Sink and the native MoE in attention layers" s2, s5);
 *             NULL = not written.
 */
int sink_attn_fwd(const sink_attn_prefill_desc* desc,
                  const void* q, const void* k, const void* v,
                  void* o, float* lse, float* s,
                  void* workspace, size_t workspace_bytes, void* stream);

/*
 * Forward with the first-token gate of vanilla attention.  "Paper notes:
 * Attention Sink and the native MoE in attention layers" (lvdousha26.github.io)
 * s2: a sink whose value vector is zero scales the head's output by
 * G = 1 - A_sink; s5: for vanilla attention, where the sample's first token
 * plays the sink, that gate comes from the log-sum-exp as
 * G = sigma(LSE_not0 - x_i0), with no attention matrix stored.
 *   gate0   output float32 [T, Hq]: the share of the real-token softmax that
 *           is not on the sample's first key,
 *             sum_{j valid, j != 0} e^{x_ij} / sum_{j valid} e^{x_ij},
 *           1 when the first key is not valid for the query, 0 for a query
 *           with no valid key.  NULL = not written (the call is then
 *           sink_attn_fwd).  It does not depend on learnable_sink, whose own
 *           gate sigma(LSE - sink) is s.
 * Every other argument, output and error as sink_attn_fwd.
 */
int sink_attn_fwd_gated(const sink_attn_prefill_desc* desc,
                        const void* q, const void* k, const void* v,
                        void* o, float* lse, float* s, float* gate0,
                        void* workspace, size_t workspace_bytes, void* stream);

/*
 * Head importance, "Paper notes: Attention Sink and the native MoE in
 * attention layers" s4: Imp_h, the mean of a per-row gate over the rows.
 *   gate       device float32 [rows, num_heads] (s of sink attention, or
 *              gate0 of sink_attn_fwd_gated).
 *   imp        output device float32 [num_heads]:
 *                imp[h] = (1 / rows) sum_r gate[r, h],
 *              summed in a fixed order (deterministic); 0 when rows == 0.
 *   workspace  at least sink_attn_head_importance_workspace_size(rows,
 *              num_heads) bytes (NULL allowed when that is 0).
 */
int sink_attn_head_importance(const float* gate, int32_t rows, int32_t num_heads,
                              float* imp, void* workspace, size_t workspace_bytes,
                              void* stream);

/*
 * Backward.  [Notes] s7 (dsink, Delta) and s8 (sink-aware dQ/dK/dV).
 *   o, lse    the forward's outputs for the same inputs (o is O_new).
 *   dout      upstream gradient dO [T, Hq, D], dtype of q.
 *   dq        output [T, Hq, D]; dk, dv outputs [T, Hkv, D] (summed over the
 *             query heads of each KV group).
 *   dsink     output float32 [Hq]; required when desc->learnable_sink is
 *             non-NULL and must be NULL otherwise.  Reduced in a fixed order
 *             (deterministic).  The caller casts it to the parameter dtype.
 * Streams: on the matrix-core path the dQ pass runs on a second stream the
 * library owns (one per device, default priority, created by the first call
 * on that device made outside graph capture) beside the dK/dV pass on
 * `stream`; it is forked from `stream` after the preprocess and joined back
 * before the call returns, so all work of the call is ordered before later
 * work on `stream` (under capture: graph edges).  Concurrent calls on one
 * device take turns through the fork and join.  SINK_ATTN_SERIAL_BWD=1 in
 * the environment (read on every call) keeps everything on `stream`; the
 * results are the same either way.
 */
int sink_attn_bwd(const sink_attn_prefill_desc* desc,
                  const void* q, const void* k, const void* v,
                  const void* o, const float* lse, const void* dout,
                  void* dq, void* dk, void* dv, float* dsink,
                  void* workspace, size_t workspace_bytes, void* stream);

/*
 * Decode: split-KV over the rolling cache, partial (max, sum, acc) per split
 * merged by their log-sum-exp, then the sink epilogue of [Notes] s4.
 *   q         [B, Hq, D]; k_cache, v_cache [B, S, Hkv, D]; dtype of q.
 *   o         output [B, Hq, D]; lse output float32 [B, Hq] (L_orig);
 *   s         output float32 [B, Hq] or NULL.
 */
int sink_attn_decode(const sink_attn_decode_desc* desc,
                     const void* q, const void* k_cache, const void* v_cache,
                     void* o, float* lse, float* s,
                     void* workspace, size_t workspace_bytes, void* stream);

/*
 * Decode that allocates nothing, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid allocation).  The same call and results as sink_attn_decode, with
 * the split partials in a static device array the library holds on each GPU
 * it runs on (SINK_ATTN_NOALLOC_SCRATCH_BYTES, kept until the process ends)
 * instead of a caller workspace.  A problem whose sink_attn_decode_workspace_size
 * exceeds that size returns SINK_ATTN_WORKSPACE_TOO_SMALL (lower num_splits,
 * or use sink_attn_decode).  Every call on one GPU shares the array: calls
 * that overlap on one GPU (other streams or threads) race on it and must be
 * ordered by the caller.  The first call on a device looks the array up on
 * that device (no allocation).
 */
#define SINK_ATTN_NOALLOC_SCRATCH_BYTES ((size_t)16 << 20)
int sink_attn_decode_noalloc(const sink_attn_decode_desc* desc,
                             const void* q, const void* k_cache, const void* v_cache,
                             void* o, float* lse, float* s, void* stream);

/* Workspace bytes each call needs for this problem (0 = none).  Pure host. */
size_t sink_attn_fwd_workspace_size(const sink_attn_prefill_desc* desc);
size_t sink_attn_bwd_workspace_size(const sink_attn_prefill_desc* desc);
size_t sink_attn_decode_workspace_size(const sink_attn_decode_desc* desc);
size_t sink_attn_head_importance_workspace_size(int32_t rows, int32_t num_heads);
size_t sink_attn_kvcache_decode_workspace_size(const sink_attn_kvcache_desc* cache,
                                               int32_t num_q_heads, int32_t num_splits);

/*
 * Pure host validation of the scalar arguments and pointers of the matching
 * call (the pointers are checked for NULL and alignment, never dereferenced).
 * Returns what the call itself would return before launching anything.
 */
int sink_attn_check_fwd(const sink_attn_prefill_desc* desc,
                        const void* q, const void* k, const void* v,
                        const void* o, const float* lse, const float* s,
                        size_t workspace_bytes);
int sink_attn_check_bwd(const sink_attn_prefill_desc* desc,
                        const void* q, const void* k, const void* v,
                        const void* o, const float* lse, const void* dout,
                        const void* dq, const void* dk, const void* dv, const float* dsink,
                        size_t workspace_bytes);
int sink_attn_check_decode(const sink_attn_decode_desc* desc,
                           const void* q, const void* k_cache, const void* v_cache,
                           const void* o, const float* lse, const float* s,
                           size_t workspace_bytes);
int sink_attn_check_fwd_gated(const sink_attn_prefill_desc* desc,
                              const void* q, const void* k, const void* v,
                              const void* o, const float* lse, const float* s,
                              const float* gate0, size_t workspace_bytes);
int sink_attn_check_head_importance(const float* gate, int32_t rows, int32_t num_heads,
                                    const float* imp, size_t workspace_bytes);
int sink_attn_check_kvcache_append(const sink_attn_kvcache_desc* cache, const void* k_new,
                                   const void* v_new, int32_t chunk, const int32_t* n_seen);
int sink_attn_check_kvcache_decode(const sink_attn_kvcache_desc* cache, const void* q,
                                   int32_t num_q_heads, const int32_t* n_tokens,
                                   float softmax_scale, int32_t num_splits, const void* o,
                                   const float* lse, const float* s, size_t workspace_bytes);

/* Static description of a status code; never NULL. */
const char* sink_attn_strerror(int status);
/* Detail of the last non-OK status returned on this thread ("" if none). */
const char* sink_attn_last_error(void);

/*
 * Kernel path chosen for a prefill problem: 1 = bfloat16 MFMA kernels
 * (D = 128), 0 = the generic kernels.  Pure host; for tests and reports.
 */
int sink_attn_prefill_path(const sink_attn_prefill_desc* desc);

/*
 * Test hook: writes the valid-key mask exactly as the forward kernels'
 * tile schedule and per-element predicate see it.  out is device uint8,
 * samples in order, each sample b holding Hkv row-major [L_b, L_b] masks
 * (1 = the key is visited and valid).  Requires max_seqlen <= 4096.
 * The bytes needed are Hkv * sum_b L_b^2 (the caller knows the lengths).
 */
int sink_attn_debug_visit_map(const sink_attn_prefill_desc* desc, uint8_t* out,
                              size_t out_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* SINK_ATTN_H */
