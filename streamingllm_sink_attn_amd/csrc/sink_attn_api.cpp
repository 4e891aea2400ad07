// C-ABI entry points: host-side validation, workspace carve-up and dispatch
// to the kernels.  Nothing here reads device memory, allocates device memory,
// frees or synchronises; the only resources created are the backward's
// second stream and its two events, once per device.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <utility>

#include "internal.h"

namespace {

thread_local char g_last_error[512] = "";

int fail(int status, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return status;
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

constexpr size_t kAlign = 256;
size_t round_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

// The backward's second stream, one per device.  The caller's stream forks to
// it at the start of the call; it runs the key-major pass's planning (which
// reads only the inputs) while the caller's stream runs the preprocess, then
// waits for the preprocess and runs the query-major dQ kernel while the
// caller's stream, once the planning is done, runs the key-major dK/dV
// kernel: dQ and dK/dV read only the inputs, L_new and Delta and write
// disjoint outputs, and the CUs that one kernel's last, unevenly finishing
// workgroups leave idle take the other's.  It joins back into the caller's
// stream before the call returns, so every output is ordered on the caller's
// stream as with one stream (under HIP graph capture the events become graph
// edges).  Default
// priority.  Created by the first backward call on a device whose stream is
// not being captured; before that, if creating it failed, or with
// SINK_ATTN_SERIAL_BWD=1 in the environment, both passes run on the caller's
// stream.  One call at a time per device goes through the fork and join (the
// events are shared); a call made while the side stream belongs to another
// thread's unfinished capture also runs on one stream.
struct BwdSide {
  std::mutex mu;
  bool tried = false, ok = false;
  hipStream_t stream = nullptr;
  hipEvent_t fork = nullptr, planned = nullptr, prepped = nullptr, join = nullptr;
};
constexpr int kMaxSideDevices = 64;
BwdSide g_bwd_side[kMaxSideDevices];

bool serial_bwd_requested() {
  const char* e = std::getenv("SINK_ATTN_SERIAL_BWD");
  return e != nullptr && e[0] == '1';
}

// The current device's side stream, created on first use outside capture,
// returned with its mutex held in *lock; nullptr when the backward runs on
// one stream.
BwdSide* bwd_side(hipStream_t st, std::unique_lock<std::mutex>* lock) {
  if (serial_bwd_requested()) return nullptr;
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxSideDevices) return nullptr;
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  unsigned long long cid = 0;
  if (hipStreamGetCaptureInfo(st, &cs, &cid) != hipSuccess) return nullptr;
  BwdSide& side = g_bwd_side[dev];
  std::unique_lock<std::mutex> held(side.mu);
  if (!side.tried) {
    if (cs != hipStreamCaptureStatusNone) return nullptr;
    side.tried = true;
    side.ok = hipStreamCreateWithFlags(&side.stream, hipStreamNonBlocking) == hipSuccess &&
              hipEventCreateWithFlags(&side.fork, hipEventDisableTiming) == hipSuccess &&
              hipEventCreateWithFlags(&side.planned, hipEventDisableTiming) == hipSuccess &&
              hipEventCreateWithFlags(&side.prepped, hipEventDisableTiming) == hipSuccess &&
              hipEventCreateWithFlags(&side.join, hipEventDisableTiming) == hipSuccess;
  }
  if (!side.ok) return nullptr;
  // A side stream that joined a capture stays in it until the capture ends:
  // use it only from that same capture, else run on one stream.
  hipStreamCaptureStatus ss = hipStreamCaptureStatusNone;
  unsigned long long sid = 0;
  if (hipStreamGetCaptureInfo(side.stream, &ss, &sid) != hipSuccess) return nullptr;
  if (ss != hipStreamCaptureStatusNone && (cs != hipStreamCaptureStatusActive || sid != cid)) return nullptr;
  *lock = std::move(held);
  return &side;
}

// Longest sample allowed with block lists (the forward's block bitmap).
constexpr int kMaxBlockSeqlen = 8192 * SINK_ATTN_BLOCK_SIZE;

int check_prefill_desc(const sink_attn_prefill_desc* d) {
  if (d == nullptr) return fail(SINK_ATTN_INVALID_ARGUMENT, "desc is NULL");
  if (d->batch < 0) return fail(SINK_ATTN_INVALID_ARGUMENT, "batch < 0");
  if (d->batch > 0 && d->cu_seqlens == nullptr)
    return fail(SINK_ATTN_INVALID_ARGUMENT, "cu_seqlens is NULL");
  if (d->total_tokens < 0) return fail(SINK_ATTN_INVALID_ARGUMENT, "total_tokens < 0");
  if (d->max_seqlen < 0) return fail(SINK_ATTN_INVALID_ARGUMENT, "max_seqlen < 0");
  if (d->total_tokens > 0 && d->max_seqlen < 1)
    return fail(SINK_ATTN_INVALID_ARGUMENT, "max_seqlen must be >= 1 when total_tokens > 0");
  if (d->total_tokens > 0 && d->batch == 0)
    return fail(SINK_ATTN_INVALID_ARGUMENT, "total_tokens > 0 with batch == 0");
  if (d->num_q_heads < 1 || d->num_kv_heads < 1)
    return fail(SINK_ATTN_INVALID_ARGUMENT, "head counts must be >= 1");
  if (d->num_q_heads % d->num_kv_heads != 0)
    return fail(SINK_ATTN_INVALID_ARGUMENT, "num_q_heads %% num_kv_heads != 0");
  if (d->num_q_heads > 65535) return fail(SINK_ATTN_UNSUPPORTED, "num_q_heads > 65535");
  if (d->dtype != SINK_ATTN_BF16 && d->dtype != SINK_ATTN_F32)
    return fail(SINK_ATTN_UNSUPPORTED, "dtype %d not supported", d->dtype);
  if (d->head_dim < 8 || d->head_dim > SINK_ATTN_MAX_HEAD_DIM || d->head_dim % 8 != 0)
    return fail(SINK_ATTN_UNSUPPORTED, "head_dim %d not supported (multiple of 8, 8..%d)",
                d->head_dim, SINK_ATTN_MAX_HEAD_DIM);
  if (!(d->softmax_scale > 0.f) || !std::isfinite(d->softmax_scale))
    return fail(SINK_ATTN_INVALID_ARGUMENT, "softmax_scale must be finite and > 0");
  if (d->n_sink < 0) return fail(SINK_ATTN_INVALID_ARGUMENT, "n_sink < 0");
  if (d->block_indices != nullptr) {
    if (d->block_size != SINK_ATTN_BLOCK_SIZE)
      return fail(SINK_ATTN_UNSUPPORTED, "block_size %d not supported (must be %d)", d->block_size,
                  SINK_ATTN_BLOCK_SIZE);
    if (d->max_blocks < 1) return fail(SINK_ATTN_INVALID_ARGUMENT, "max_blocks < 1");
    if (d->num_q_blocks < 0) return fail(SINK_ATTN_INVALID_ARGUMENT, "num_q_blocks < 0");
    const long long need_min = (static_cast<long long>(d->total_tokens) + SINK_ATTN_BLOCK_SIZE - 1) /
                               SINK_ATTN_BLOCK_SIZE;
    if (d->num_q_blocks < need_min)
      return fail(SINK_ATTN_INVALID_ARGUMENT, "num_q_blocks %d < ceil(total_tokens / %d)",
                  d->num_q_blocks, SINK_ATTN_BLOCK_SIZE);
    if (d->max_seqlen > kMaxBlockSeqlen)
      return fail(SINK_ATTN_UNSUPPORTED, "max_seqlen > %d with block_indices", kMaxBlockSeqlen);
  }
  return SINK_ATTN_OK;
}

sa::Prefill to_prefill(const sink_attn_prefill_desc* d) {
  sa::Prefill p;
  p.cu = d->cu_seqlens;
  p.batch = d->batch;
  p.total = d->total_tokens;
  p.max_seqlen = d->max_seqlen;
  p.hq = d->num_q_heads;
  p.hkv = d->num_kv_heads;
  p.d = d->head_dim;
  p.dtype = d->dtype;
  p.scale = d->softmax_scale;
  p.n_sink = d->n_sink;
  p.window = d->window;
  p.blocks = d->block_indices;
  p.nqb = d->block_indices ? d->num_q_blocks : 0;
  p.max_blocks = d->block_indices ? d->max_blocks : 0;
  p.sink = d->learnable_sink;
  return p;
}

size_t elem_size(int dtype) { return dtype == SINK_ATTN_F32 ? 4 : 2; }

// Backward workspace layout (each section 256-byte aligned).
struct BwdLayout {
  size_t delta, lnew, terms, dsink_part, dk_acc, dv_acc, csr_off, csr_idx, csr_bits, plan, split_slot,
      queues, total;
  int max_split;
};

BwdLayout bwd_layout(const sa::Prefill& p) {
  BwdLayout l{};
  const size_t rows = static_cast<size_t>(p.total) * p.hq;
  const size_t kv = static_cast<size_t>(p.total) * p.hkv * p.d;
  const bool mfma = sa::bwd_mfma_supported(p);
  size_t off = 0;
  l.delta = off; off += round_up(rows * 4);
  l.lnew = off; off += round_up(rows * 4);
  l.terms = off; off += round_up(rows * 4);
  l.dsink_part = off; off += round_up(static_cast<size_t>(sa::dsink_slabs(p.total)) * p.hq * 4);
  // float32 dK/dV: every row on the generic path, split key tiles only on the
  // matrix-core path (64 rows of D per tile)
  l.max_split = mfma ? sa::bwd_max_split_tiles(p) : 0;
  const size_t acc = mfma ? static_cast<size_t>(l.max_split) * 64 * p.d : kv;
  l.dk_acc = off; off += round_up(acc * 4);
  l.dv_acc = off; off += round_up(acc * 4);
  const size_t nl = p.blocks ? static_cast<size_t>(p.nqb) * p.hkv : 0;
  l.csr_off = off; off += (p.blocks && mfma) ? round_up((nl + 1) * 4) : 0;
  l.csr_idx = off; off += (p.blocks && mfma) ? round_up(nl * p.max_blocks * 4) : 0;
  l.csr_bits = off;
  off += (p.blocks && mfma) ? round_up(nl * static_cast<size_t>(sa::block_csr_words(p)) * 4) : 0;
  l.plan = off; off += mfma ? round_up((static_cast<size_t>(sa::bwd_num_tiles(p)) + 1) * 4) : 0;
  l.split_slot = off; off += mfma ? round_up((static_cast<size_t>(sa::bwd_num_tiles(p)) + 1) * 4) : 0;
  l.queues = off; off += mfma ? round_up(8 * 4) : 0;
  l.total = off;
  return l;
}

int check_decode_desc(const sink_attn_decode_desc* d) {
  if (d == nullptr) return fail(SINK_ATTN_INVALID_ARGUMENT, "desc is NULL");
  if (d->batch < 0) return fail(SINK_ATTN_INVALID_ARGUMENT, "batch < 0");
  if (d->batch > 0 && d->slots < 1) return fail(SINK_ATTN_INVALID_ARGUMENT, "slots < 1");
  if (d->num_q_heads < 1 || d->num_kv_heads < 1)
    return fail(SINK_ATTN_INVALID_ARGUMENT, "head counts must be >= 1");
  if (d->num_q_heads % d->num_kv_heads != 0)
    return fail(SINK_ATTN_INVALID_ARGUMENT, "num_q_heads %% num_kv_heads != 0");
  if (d->num_q_heads > 65535) return fail(SINK_ATTN_UNSUPPORTED, "num_q_heads > 65535");
  if (d->dtype != SINK_ATTN_BF16 && d->dtype != SINK_ATTN_F32)
    return fail(SINK_ATTN_UNSUPPORTED, "dtype %d not supported", d->dtype);
  if (d->head_dim < 8 || d->head_dim > SINK_ATTN_MAX_HEAD_DIM || d->head_dim % 8 != 0)
    return fail(SINK_ATTN_UNSUPPORTED, "head_dim %d not supported", d->head_dim);
  if (!(d->softmax_scale > 0.f) || !std::isfinite(d->softmax_scale))
    return fail(SINK_ATTN_INVALID_ARGUMENT, "softmax_scale must be finite and > 0");
  if (d->batch > 65535) return fail(SINK_ATTN_UNSUPPORTED, "batch > 65535");
  if (d->num_splits < 0 || d->num_splits > 256)
    return fail(SINK_ATTN_INVALID_ARGUMENT, "num_splits must be in [0, 256]");
  return SINK_ATTN_OK;
}

sa::Decode to_decode(const sink_attn_decode_desc* d) {
  sa::Decode p;
  p.cache_seqlens = d->cache_seqlens;
  p.batch = d->batch;
  p.slots = d->slots;
  p.hq = d->num_q_heads;
  p.hkv = d->num_kv_heads;
  p.d = d->head_dim;
  p.dtype = d->dtype;
  p.scale = d->softmax_scale;
  p.sink = d->learnable_sink;
  p.splits = d->num_splits;
  if (p.splits == 0) p.splits = sa::decode_auto_splits(p);
  if (p.splits > p.slots && p.slots > 0) p.splits = p.slots;
  if (p.splits < 1) p.splits = 1;
  return p;
}

size_t decode_ws_bytes(const sa::Decode& p) {
  // one split: the split kernel applies the sink epilogue and writes O itself
  if (!sa::decode_mfma_supported(p) || p.splits <= 1) return 0;
  // per (sequence, query head, split): acc[D] + (m, l)
  return round_up(static_cast<size_t>(p.batch) * p.hq * p.splits * (p.d + 2) * 4);
}

int check_ptr(const void* ptr, const char* name, size_t align, bool required) {
  if (ptr == nullptr) {
    if (required) return fail(SINK_ATTN_INVALID_ARGUMENT, "%s is NULL", name);
    return SINK_ATTN_OK;
  }
  if (!aligned(ptr, align))
    return fail(SINK_ATTN_INVALID_ARGUMENT, "%s is not %zu-byte aligned", name, align);
  return SINK_ATTN_OK;
}

#define SA_TRY(expr)                 \
  do {                               \
    int _st = (expr);                \
    if (_st != SINK_ATTN_OK) return _st; \
  } while (0)

int hip_status(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(SINK_ATTN_HIP_ERROR, "%s: %s", what, hipGetErrorString(e));
  return SINK_ATTN_OK;
}

int check_kvcache_desc(const sink_attn_kvcache_desc* c) {
  if (c == nullptr) return fail(SINK_ATTN_INVALID_ARGUMENT, "cache desc is NULL");
  if (c->batch < 0) return fail(SINK_ATTN_INVALID_ARGUMENT, "batch < 0");
  if (c->batch > 65535) return fail(SINK_ATTN_UNSUPPORTED, "batch > 65535");
  if (c->n_sink < 0) return fail(SINK_ATTN_INVALID_ARGUMENT, "n_sink < 0");
  if (c->window < 1) return fail(SINK_ATTN_INVALID_ARGUMENT, "window < 1");
  if (c->num_kv_heads < 1) return fail(SINK_ATTN_INVALID_ARGUMENT, "num_kv_heads < 1");
  if (c->head_dim < 8 || c->head_dim > SINK_ATTN_MAX_HEAD_DIM || c->head_dim % 8 != 0)
    return fail(SINK_ATTN_UNSUPPORTED, "head_dim %d not supported", c->head_dim);
  if (c->quantized != 0 && c->quantized != 1)
    return fail(SINK_ATTN_INVALID_ARGUMENT, "quantized must be 0 or 1");
  if (c->quantized && c->head_dim != 128)
    return fail(SINK_ATTN_UNSUPPORTED, "the 8-bit cache needs head_dim 128");
  if (static_cast<long long>(c->n_sink) + c->window > (1LL << 30))
    return fail(SINK_ATTN_UNSUPPORTED, "n_sink + window too large");
  const bool need = c->batch > 0;
  if (!c->quantized) {
    SA_TRY(check_ptr(c->k, "cache k", 16, need));
    SA_TRY(check_ptr(c->v, "cache v", 16, need));
  } else {
    SA_TRY(check_ptr(c->sink_k, "sink_k", 16, need && c->n_sink > 0));
    SA_TRY(check_ptr(c->sink_v, "sink_v", 16, need && c->n_sink > 0));
    SA_TRY(check_ptr(c->win_k, "win_k", 16, need));
    SA_TRY(check_ptr(c->win_v, "win_v", 16, need));
    SA_TRY(check_ptr(c->win_k_scale, "win_k_scale", 16, need));
    SA_TRY(check_ptr(c->win_v_scale, "win_v_scale", 16, need));
  }
  return SINK_ATTN_OK;
}

sa::KvCache to_kvcache(const sink_attn_kvcache_desc* c) {
  sa::KvCache k;
  k.batch = c->batch;
  k.n_sink = c->n_sink;
  k.window = c->window;
  k.hkv = c->num_kv_heads;
  k.d = c->head_dim;
  k.quantized = c->quantized;
  k.k = c->k;
  k.v = c->v;
  k.sink_k = c->sink_k;
  k.sink_v = c->sink_v;
  k.win_k = static_cast<uint8_t*>(c->win_k);
  k.win_v = static_cast<uint8_t*>(c->win_v);
  k.win_k_scale = c->win_k_scale;
  k.win_v_scale = c->win_v_scale;
  return k;
}

// The decode problem of a cache decode call (splits resolved).
sa::Decode kvcache_decode_problem(const sink_attn_kvcache_desc* c, int32_t hq,
                                  const int32_t* n_tokens, float scale, const float* sink,
                                  int32_t num_splits) {
  sa::Decode p;
  p.cache_seqlens = n_tokens;
  p.batch = c->batch;
  p.slots = c->n_sink + c->window;
  p.hq = hq;
  p.hkv = c->num_kv_heads;
  p.d = c->head_dim;
  p.dtype = SINK_ATTN_BF16;
  p.scale = scale;
  p.sink = sink;
  p.splits = num_splits;
  if (p.splits == 0)
    p.splits = c->quantized ? sa::kvcache_q8_auto_splits(p, to_kvcache(c)) : sa::decode_auto_splits(p);
  if (p.splits > p.slots && p.slots > 0) p.splits = p.slots;
  if (p.splits < 1) p.splits = 1;
  return p;
}

}  // namespace

namespace sa {
int set_last_error(int status, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return status;
}
}  // namespace sa

extern "C" {

const char* sink_attn_strerror(int status) {
  switch (status) {
    case SINK_ATTN_OK: return "ok";
    case SINK_ATTN_INVALID_ARGUMENT: return "invalid argument";
    case SINK_ATTN_UNSUPPORTED: return "unsupported configuration";
    case SINK_ATTN_WORKSPACE_TOO_SMALL: return "workspace too small";
    case SINK_ATTN_HIP_ERROR: return "HIP error";
    default: return "unknown status";
  }
}

const char* sink_attn_last_error(void) { return g_last_error; }

size_t sink_attn_fwd_workspace_size(const sink_attn_prefill_desc* desc) {
  (void)desc;
  return 0;
}

size_t sink_attn_bwd_workspace_size(const sink_attn_prefill_desc* desc) {
  if (check_prefill_desc(desc) != SINK_ATTN_OK) return 0;
  return bwd_layout(to_prefill(desc)).total;
}

size_t sink_attn_decode_workspace_size(const sink_attn_decode_desc* desc) {
  if (check_decode_desc(desc) != SINK_ATTN_OK) return 0;
  return decode_ws_bytes(to_decode(desc));
}

int sink_attn_prefill_path(const sink_attn_prefill_desc* desc) {
  if (check_prefill_desc(desc) != SINK_ATTN_OK) return -1;
  return sa::fwd_mfma_supported(to_prefill(desc)) ? 1 : 0;
}

int sink_attn_check_fwd(const sink_attn_prefill_desc* desc, const void* q, const void* k,
                        const void* v, const void* o, const float* lse, const float* s,
                        size_t workspace_bytes) {
  SA_TRY(check_prefill_desc(desc));
  const bool need = desc->total_tokens > 0;
  SA_TRY(check_ptr(q, "q", 16, need));
  SA_TRY(check_ptr(k, "k", 16, need));
  SA_TRY(check_ptr(v, "v", 16, need));
  SA_TRY(check_ptr(o, "o", 16, need));
  SA_TRY(check_ptr(lse, "lse", 4, need));
  SA_TRY(check_ptr(s, "s", 4, false));
  SA_TRY(check_ptr(desc->learnable_sink, "learnable_sink", 4, false));
  SA_TRY(check_ptr(desc->block_indices, "block_indices", 4, false));
  if (workspace_bytes < sink_attn_fwd_workspace_size(desc))
    return fail(SINK_ATTN_WORKSPACE_TOO_SMALL, "workspace too small");
  return SINK_ATTN_OK;
}

int sink_attn_check_bwd(const sink_attn_prefill_desc* desc, const void* q, const void* k,
                        const void* v, const void* o, const float* lse, const void* dout,
                        const void* dq, const void* dk, const void* dv, const float* dsink,
                        size_t workspace_bytes) {
  SA_TRY(check_prefill_desc(desc));
  const bool need = desc->total_tokens > 0;
  SA_TRY(check_ptr(q, "q", 16, need));
  SA_TRY(check_ptr(k, "k", 16, need));
  SA_TRY(check_ptr(v, "v", 16, need));
  SA_TRY(check_ptr(o, "o", 16, need));
  SA_TRY(check_ptr(lse, "lse", 4, need));
  SA_TRY(check_ptr(dout, "dout", 16, need));
  SA_TRY(check_ptr(dq, "dq", 16, need));
  SA_TRY(check_ptr(dk, "dk", 16, need));
  SA_TRY(check_ptr(dv, "dv", 16, need));
  SA_TRY(check_ptr(desc->learnable_sink, "learnable_sink", 4, false));
  SA_TRY(check_ptr(desc->block_indices, "block_indices", 4, false));
  if (desc->learnable_sink != nullptr && dsink == nullptr)
    return fail(SINK_ATTN_INVALID_ARGUMENT, "dsink is NULL while learnable_sink is set");
  if (desc->learnable_sink == nullptr && dsink != nullptr)
    return fail(SINK_ATTN_INVALID_ARGUMENT, "dsink is set while learnable_sink is NULL");
  SA_TRY(check_ptr(dsink, "dsink", 4, false));
  if (workspace_bytes < sink_attn_bwd_workspace_size(desc))
    return fail(SINK_ATTN_WORKSPACE_TOO_SMALL, "workspace too small: %zu < %zu", workspace_bytes,
                sink_attn_bwd_workspace_size(desc));
  return SINK_ATTN_OK;
}

int sink_attn_check_decode(const sink_attn_decode_desc* desc, const void* q, const void* k_cache,
                           const void* v_cache, const void* o, const float* lse, const float* s,
                           size_t workspace_bytes) {
  SA_TRY(check_decode_desc(desc));
  const bool need = desc->batch > 0;
  SA_TRY(check_ptr(q, "q", 16, need));
  SA_TRY(check_ptr(k_cache, "k_cache", 16, need));
  SA_TRY(check_ptr(v_cache, "v_cache", 16, need));
  SA_TRY(check_ptr(o, "o", 16, need));
  SA_TRY(check_ptr(lse, "lse", 4, need));
  SA_TRY(check_ptr(s, "s", 4, false));
  SA_TRY(check_ptr(desc->learnable_sink, "learnable_sink", 4, false));
  SA_TRY(check_ptr(desc->cache_seqlens, "cache_seqlens", 4, false));
  if (workspace_bytes < sink_attn_decode_workspace_size(desc))
    return fail(SINK_ATTN_WORKSPACE_TOO_SMALL, "workspace too small: %zu < %zu", workspace_bytes,
                sink_attn_decode_workspace_size(desc));
  return SINK_ATTN_OK;
}

int sink_attn_check_fwd_gated(const sink_attn_prefill_desc* desc, const void* q, const void* k,
                              const void* v, const void* o, const float* lse, const float* s,
                              const float* gate0, size_t workspace_bytes) {
  SA_TRY(sink_attn_check_fwd(desc, q, k, v, o, lse, s, workspace_bytes));
  SA_TRY(check_ptr(gate0, "gate0", 4, false));
  return SINK_ATTN_OK;
}

int sink_attn_fwd_gated(const sink_attn_prefill_desc* desc, const void* q, const void* k,
                        const void* v, void* o, float* lse, float* s, float* gate0,
                        void* workspace, size_t workspace_bytes, void* stream) {
  try {
    SA_TRY(sink_attn_check_fwd_gated(desc, q, k, v, o, lse, s, gate0, workspace_bytes));
    (void)workspace;
    const sa::Prefill p = to_prefill(desc);
    if (p.total == 0) return SINK_ATTN_OK;
    hipStream_t st = static_cast<hipStream_t>(stream);
    hipError_t e = sa::fwd_mfma_supported(p)
                       ? sa::launch_fwd_mfma(p, q, k, v, o, lse, s, gate0, st)
                       : sa::launch_fwd_generic(p, q, k, v, o, lse, s, gate0, st);
    return hip_status(e, "sink_attn_fwd launch");
  } catch (...) {
    return fail(SINK_ATTN_HIP_ERROR, "unexpected exception in sink_attn_fwd");
  }
}

int sink_attn_fwd(const sink_attn_prefill_desc* desc, const void* q, const void* k, const void* v,
                  void* o, float* lse, float* s, void* workspace, size_t workspace_bytes,
                  void* stream) {
  return sink_attn_fwd_gated(desc, q, k, v, o, lse, s, nullptr, workspace, workspace_bytes, stream);
}

size_t sink_attn_head_importance_workspace_size(int32_t rows, int32_t num_heads) {
  if (rows <= 0 || num_heads <= 0) return 0;
  return round_up(static_cast<size_t>(sa::dsink_slabs(rows)) * num_heads * 4);
}

int sink_attn_check_head_importance(const float* gate, int32_t rows, int32_t num_heads,
                                    const float* imp, size_t workspace_bytes) {
  if (rows < 0) return fail(SINK_ATTN_INVALID_ARGUMENT, "rows < 0");
  if (num_heads < 1) return fail(SINK_ATTN_INVALID_ARGUMENT, "num_heads < 1");
  SA_TRY(check_ptr(gate, "gate", 4, rows > 0));
  SA_TRY(check_ptr(imp, "imp", 4, true));
  const size_t need = sink_attn_head_importance_workspace_size(rows, num_heads);
  if (workspace_bytes < need)
    return fail(SINK_ATTN_WORKSPACE_TOO_SMALL, "workspace too small: %zu < %zu", workspace_bytes, need);
  return SINK_ATTN_OK;
}

int sink_attn_head_importance(const float* gate, int32_t rows, int32_t num_heads, float* imp,
                              void* workspace, size_t workspace_bytes, void* stream) {
  try {
    SA_TRY(sink_attn_check_head_importance(gate, rows, num_heads, imp, workspace_bytes));
    if (sink_attn_head_importance_workspace_size(rows, num_heads) > 0 && workspace == nullptr)
      return fail(SINK_ATTN_INVALID_ARGUMENT, "workspace is NULL");
    hipStream_t st = static_cast<hipStream_t>(stream);
    const float scale = rows > 0 ? 1.f / static_cast<float>(rows) : 0.f;
    hipError_t e = sa::launch_column_sum(gate, rows, num_heads, scale, static_cast<float*>(workspace),
                                         imp, st);
    return hip_status(e, "sink_attn_head_importance launch");
  } catch (...) {
    return fail(SINK_ATTN_HIP_ERROR, "unexpected exception in sink_attn_head_importance");
  }
}

int sink_attn_bwd(const sink_attn_prefill_desc* desc, const void* q, const void* k, const void* v,
                  const void* o, const float* lse, const void* dout, void* dq, void* dk, void* dv,
                  float* dsink, void* workspace, size_t workspace_bytes, void* stream) {
  try {
    SA_TRY(sink_attn_check_bwd(desc, q, k, v, o, lse, dout, dq, dk, dv, dsink, workspace_bytes));
    const sa::Prefill p = to_prefill(desc);
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (p.total == 0) {
      if (dsink != nullptr) {
        // No rows: dsink is an empty sum.
        hipError_t e = sa::launch_fill_zero(dsink, p.hq, st);
        return hip_status(e, "sink_attn_bwd dsink clear");
      }
      return SINK_ATTN_OK;
    }
    const BwdLayout lay = bwd_layout(p);
    char* base = static_cast<char*>(workspace);
    sa::BwdWork w;
    w.delta = reinterpret_cast<float*>(base + lay.delta);
    w.lnew = reinterpret_cast<float*>(base + lay.lnew);
    w.dsink_terms = reinterpret_cast<float*>(base + lay.terms);
    w.dsink_part = reinterpret_cast<float*>(base + lay.dsink_part);
    w.dk_acc = reinterpret_cast<float*>(base + lay.dk_acc);
    w.dv_acc = reinterpret_cast<float*>(base + lay.dv_acc);
    w.csr_off = reinterpret_cast<int32_t*>(base + lay.csr_off);
    w.csr_idx = reinterpret_cast<int32_t*>(base + lay.csr_idx);
    w.csr_bits = reinterpret_cast<uint32_t*>(base + lay.csr_bits);
    w.plan = reinterpret_cast<int32_t*>(base + lay.plan);
    w.split_slot = reinterpret_cast<int32_t*>(base + lay.split_slot);
    w.max_split = lay.max_split;
    w.queues = reinterpret_cast<int32_t*>(base + lay.queues);
    const bool mfma = sa::bwd_mfma_supported(p);
    hipError_t e;
    if (mfma) {
      std::unique_lock<std::mutex> lock;
      BwdSide* side = bwd_side(st, &lock);
      e = hipSuccess;
      bool forked = false;
      if (side != nullptr) {
        e = hipEventRecord(side->fork, st);
        if (e == hipSuccess) e = hipStreamWaitEvent(side->stream, side->fork, 0);
        forked = e == hipSuccess;
      }
      hipStream_t ss = forked ? side->stream : st;
      if (e == hipSuccess && p.blocks != nullptr) e = sa::launch_block_csr(p, w, ss);
      if (e == hipSuccess) e = sa::launch_bwd_dkdv_plan(p, w, dk, dv, ss);
      if (e == hipSuccess && forked) e = hipEventRecord(side->planned, ss);
      if (e == hipSuccess) e = sa::launch_bwd_preprocess(p, o, lse, dout, w, /*zero_dkv=*/false, st);
      if (e == hipSuccess && forked) {
        e = hipEventRecord(side->prepped, st);
        if (e == hipSuccess) e = hipStreamWaitEvent(ss, side->prepped, 0);
      }
      if (e == hipSuccess) e = sa::launch_bwd_dq(p, q, k, v, dout, w, dq, ss);
      if (e == hipSuccess && forked) e = hipStreamWaitEvent(st, side->planned, 0);
      if (e == hipSuccess) e = sa::launch_bwd_dkdv(p, q, k, v, dout, w, dk, dv, st);
      if (e == hipSuccess) e = sa::launch_bwd_finish(p, w, dsink, dk, dv, /*dkv_from_acc=*/false, st);
      if (forked) {
        // join even after an error, so a capture is never left forked
        hipError_t j = hipEventRecord(side->join, ss);
        if (j == hipSuccess) j = hipStreamWaitEvent(st, side->join, 0);
        if (e == hipSuccess) e = j;
      }
    } else {
      e = sa::launch_bwd_preprocess(p, o, lse, dout, w, /*zero_dkv=*/true, st);
      if (e == hipSuccess) e = sa::launch_bwd_generic(p, q, k, v, dout, w, dq, st);
      if (e == hipSuccess) e = sa::launch_bwd_finish(p, w, dsink, dk, dv, /*dkv_from_acc=*/true, st);
    }
    return hip_status(e, "sink_attn_bwd launch");
  } catch (...) {
    return fail(SINK_ATTN_HIP_ERROR, "unexpected exception in sink_attn_bwd");
  }
}

int sink_attn_check_kvcache_append(const sink_attn_kvcache_desc* cache, const void* k_new,
                                   const void* v_new, int32_t chunk, const int32_t* n_seen) {
  SA_TRY(check_kvcache_desc(cache));
  if (chunk < 0) return fail(SINK_ATTN_INVALID_ARGUMENT, "chunk < 0");
  const long long rows = static_cast<long long>(cache->batch) * chunk * cache->num_kv_heads;
  if (rows > 0x7fffffffLL) return fail(SINK_ATTN_UNSUPPORTED, "batch * chunk * num_kv_heads too large");
  const bool need = rows > 0;
  SA_TRY(check_ptr(k_new, "k_new", 16, need));
  SA_TRY(check_ptr(v_new, "v_new", 16, need));
  SA_TRY(check_ptr(n_seen, "n_seen", 4, need));
  return SINK_ATTN_OK;
}

int sink_attn_kvcache_append(const sink_attn_kvcache_desc* cache, const void* k_new,
                             const void* v_new, int32_t chunk, const int32_t* n_seen, void* stream) {
  try {
    SA_TRY(sink_attn_check_kvcache_append(cache, k_new, v_new, chunk, n_seen));
    if (static_cast<long long>(cache->batch) * chunk == 0) return SINK_ATTN_OK;
    hipError_t e = sa::launch_kvcache_append(to_kvcache(cache), k_new, v_new, chunk, n_seen,
                                             static_cast<hipStream_t>(stream));
    return hip_status(e, "sink_attn_kvcache_append launch");
  } catch (...) {
    return fail(SINK_ATTN_HIP_ERROR, "unexpected exception in sink_attn_kvcache_append");
  }
}

size_t sink_attn_kvcache_decode_workspace_size(const sink_attn_kvcache_desc* cache,
                                               int32_t num_q_heads, int32_t num_splits) {
  if (check_kvcache_desc(cache) != SINK_ATTN_OK || num_q_heads < 1 || num_splits < 0) return 0;
  const sa::Decode p = kvcache_decode_problem(cache, num_q_heads, nullptr, 1.f, nullptr, num_splits);
  if (!cache->quantized) return decode_ws_bytes(p);
  return p.splits > 1 ? round_up(static_cast<size_t>(p.batch) * p.hq * p.splits * (p.d + 2) * 4) : 0;
}

int sink_attn_check_kvcache_decode(const sink_attn_kvcache_desc* cache, const void* q,
                                   int32_t num_q_heads, const int32_t* n_tokens, float softmax_scale,
                                   int32_t num_splits, const void* o, const float* lse, const float* s,
                                   size_t workspace_bytes) {
  SA_TRY(check_kvcache_desc(cache));
  if (num_q_heads < 1 || num_q_heads % cache->num_kv_heads != 0)
    return fail(SINK_ATTN_INVALID_ARGUMENT, "num_q_heads must be a positive multiple of num_kv_heads");
  if (num_q_heads > 65535) return fail(SINK_ATTN_UNSUPPORTED, "num_q_heads > 65535");
  if (!(softmax_scale > 0.f) || !std::isfinite(softmax_scale))
    return fail(SINK_ATTN_INVALID_ARGUMENT, "softmax_scale must be finite and > 0");
  if (num_splits < 0 || num_splits > 256)
    return fail(SINK_ATTN_INVALID_ARGUMENT, "num_splits must be in [0, 256]");
  const bool need = cache->batch > 0;
  SA_TRY(check_ptr(q, "q", 16, need));
  SA_TRY(check_ptr(n_tokens, "n_tokens", 4, need));
  SA_TRY(check_ptr(o, "o", 16, need));
  SA_TRY(check_ptr(lse, "lse", 4, need));
  SA_TRY(check_ptr(s, "s", 4, false));
  const size_t ws = sink_attn_kvcache_decode_workspace_size(cache, num_q_heads, num_splits);
  if (workspace_bytes < ws)
    return fail(SINK_ATTN_WORKSPACE_TOO_SMALL, "workspace too small: %zu < %zu", workspace_bytes, ws);
  return SINK_ATTN_OK;
}

int sink_attn_kvcache_decode(const sink_attn_kvcache_desc* cache, const void* q, int32_t num_q_heads,
                             const int32_t* n_tokens, float softmax_scale,
                             const float* learnable_sink, int32_t num_splits, void* o, float* lse,
                             float* s, void* workspace, size_t workspace_bytes, void* stream) {
  try {
    SA_TRY(sink_attn_check_kvcache_decode(cache, q, num_q_heads, n_tokens, softmax_scale, num_splits,
                                          o, lse, s, workspace_bytes));
    SA_TRY(check_ptr(learnable_sink, "learnable_sink", 4, false));
    if (cache->batch == 0) return SINK_ATTN_OK;
    const sa::Decode p = kvcache_decode_problem(cache, num_q_heads, n_tokens, softmax_scale,
                                                learnable_sink, num_splits);
    hipStream_t st = static_cast<hipStream_t>(stream);
    float* ws = static_cast<float*>(workspace);
    hipError_t e = cache->quantized
                       ? sa::launch_kvcache_decode_q8(p, to_kvcache(cache), q, o, lse, s, ws, st)
                       : sa::launch_decode(p, q, cache->k, cache->v, o, lse, s, ws, st);
    return hip_status(e, "sink_attn_kvcache_decode launch");
  } catch (...) {
    return fail(SINK_ATTN_HIP_ERROR, "unexpected exception in sink_attn_kvcache_decode");
  }
}

// Chunked prefill: workspace sections of the packed per-sequence samples.
// With head_dim 128 the matrix-core forward reads Q and writes the outputs in
// the caller's [B, chunk] layout (direct); otherwise the generic forward works
// on packed Q / O copies.  With the bfloat16 cache as well (inplace) it also
// reads K and V straight from the cache and the chunk: kp / vp then hold only
// the staged seam tiles, 3 x 64 rows per stream.
struct PrefillLayout {
  size_t cu, qstart, qo_base, kp, vp, qp, op, lsep, sp, total;
  long long lmax;
  bool direct, inplace;
};

PrefillLayout kvcache_prefill_layout(const sink_attn_kvcache_desc* c, int32_t chunk, int32_t hq) {
  PrefillLayout l{};
  l.lmax = static_cast<long long>(c->n_sink) + c->window + chunk;
  l.direct = c->head_dim == 128;
  l.inplace = l.direct && !c->quantized;
  const size_t rows = l.inplace ? static_cast<size_t>(c->batch) * sa::kSeamSlots * sa::kSeamRows
                                : static_cast<size_t>(c->batch) * static_cast<size_t>(l.lmax);
  const size_t D = static_cast<size_t>(c->head_dim);
  const size_t qrows = l.direct ? 0 : static_cast<size_t>(c->batch) * static_cast<size_t>(l.lmax);
  size_t off = 0;
  l.cu = off; off += round_up((2 * static_cast<size_t>(c->batch) + 1) * 4);
  l.qstart = off; off += round_up(2 * static_cast<size_t>(c->batch) * 4);
  l.qo_base = off; off += round_up(2 * static_cast<size_t>(c->batch) * 4);
  l.kp = off; off += round_up(rows * c->num_kv_heads * D * 2);
  l.vp = off; off += round_up(rows * c->num_kv_heads * D * 2);
  l.qp = off; off += round_up(qrows * hq * D * 2);
  l.op = off; off += round_up(qrows * hq * D * 2);
  l.lsep = off; off += round_up(qrows * hq * 4);
  l.sp = off; off += round_up(qrows * hq * 4);
  l.total = off;
  return l;
}

size_t sink_attn_kvcache_prefill_workspace_size(const sink_attn_kvcache_desc* cache, int32_t chunk,
                                                int32_t num_q_heads) {
  if (check_kvcache_desc(cache) != SINK_ATTN_OK || chunk < 0 || num_q_heads < 1) return 0;
  if (static_cast<long long>(cache->batch) * chunk == 0) return 0;
  return kvcache_prefill_layout(cache, chunk, num_q_heads).total;
}

int sink_attn_check_kvcache_prefill(const sink_attn_kvcache_desc* cache, const void* q,
                                    int32_t num_q_heads, const void* k_new, const void* v_new,
                                    int32_t chunk, const int32_t* n_seen, float softmax_scale,
                                    const void* o, const float* lse, const float* s,
                                    size_t workspace_bytes) {
  SA_TRY(check_kvcache_desc(cache));
  if (chunk < 0) return fail(SINK_ATTN_INVALID_ARGUMENT, "chunk < 0");
  if (num_q_heads < 1 || num_q_heads % cache->num_kv_heads != 0)
    return fail(SINK_ATTN_INVALID_ARGUMENT, "num_q_heads must be a positive multiple of num_kv_heads");
  if (num_q_heads > 65535) return fail(SINK_ATTN_UNSUPPORTED, "num_q_heads > 65535");
  if (!(softmax_scale > 0.f) || !std::isfinite(softmax_scale))
    return fail(SINK_ATTN_INVALID_ARGUMENT, "softmax_scale must be finite and > 0");
  const long long lmax = static_cast<long long>(cache->n_sink) + cache->window + chunk;
  const long long rows = static_cast<long long>(cache->batch) * lmax;
  // packed rows, and the forward's grid (at most lmax/32 position tiles x
  // 2*batch samples x num_q_heads head groups), within 32 bits
  if (rows > 0x7fffffffLL || 2LL * cache->batch * ((lmax + 31) / 32) * num_q_heads > 0x7fffffffLL ||
      static_cast<long long>(cache->batch) * chunk * num_q_heads > 0x7fffffffLL ||
      rows * cache->num_kv_heads > 0x7fffffffLL)
    return fail(SINK_ATTN_UNSUPPORTED, "batch x (n_sink + window + chunk) too large");
  const bool need = static_cast<long long>(cache->batch) * chunk > 0;
  SA_TRY(check_ptr(q, "q", 16, need));
  SA_TRY(check_ptr(k_new, "k_new", 16, need));
  SA_TRY(check_ptr(v_new, "v_new", 16, need));
  SA_TRY(check_ptr(n_seen, "n_seen", 4, need));
  SA_TRY(check_ptr(o, "o", 16, need));
  SA_TRY(check_ptr(lse, "lse", 4, need));
  SA_TRY(check_ptr(s, "s", 4, false));
  const size_t ws = sink_attn_kvcache_prefill_workspace_size(cache, chunk, num_q_heads);
  if (workspace_bytes < ws)
    return fail(SINK_ATTN_WORKSPACE_TOO_SMALL, "workspace too small: %zu < %zu", workspace_bytes, ws);
  return SINK_ATTN_OK;
}

int sink_attn_kvcache_prefill(const sink_attn_kvcache_desc* cache, const void* q, int32_t num_q_heads,
                              const void* k_new, const void* v_new, int32_t chunk,
                              const int32_t* n_seen, float softmax_scale, const float* learnable_sink,
                              void* o, float* lse, float* s, void* workspace, size_t workspace_bytes,
                              void* stream) {
  try {
    SA_TRY(sink_attn_check_kvcache_prefill(cache, q, num_q_heads, k_new, v_new, chunk, n_seen,
                                           softmax_scale, o, lse, s, workspace_bytes));
    SA_TRY(check_ptr(learnable_sink, "learnable_sink", 4, false));
    if (static_cast<long long>(cache->batch) * chunk == 0) return SINK_ATTN_OK;
    SA_TRY(check_ptr(workspace, "workspace", 256, true));
    const PrefillLayout l = kvcache_prefill_layout(cache, chunk, num_q_heads);
    char* ws = static_cast<char*>(workspace);
    int32_t* cu = reinterpret_cast<int32_t*>(ws + l.cu);
    int32_t* qstart = reinterpret_cast<int32_t*>(ws + l.qstart);
    float* lsep = reinterpret_cast<float*>(ws + l.lsep);
    float* sp = reinterpret_cast<float*>(ws + l.sp);
    const sa::KvCache kc = to_kvcache(cache);
    hipStream_t st = static_cast<hipStream_t>(stream);
    const int lmax = static_cast<int>(l.lmax);
    int32_t* qo_base = l.direct ? reinterpret_cast<int32_t*>(ws + l.qo_base) : nullptr;
    sa::CacheKv ckv;
    ckv.k = static_cast<const uint16_t*>(cache->k);
    ckv.v = static_cast<const uint16_t*>(cache->v);
    ckv.kn = static_cast<const uint16_t*>(k_new);
    ckv.vn = static_cast<const uint16_t*>(v_new);
    ckv.sk = reinterpret_cast<uint16_t*>(ws + l.kp);
    ckv.sv = reinterpret_cast<uint16_t*>(ws + l.vp);
    ckv.n_seen = n_seen;
    ckv.batch = cache->batch;
    ckv.hkv = cache->num_kv_heads;
    ckv.slots = cache->n_sink + cache->window;
    ckv.n_sink = cache->n_sink;
    ckv.window = cache->window;
    ckv.chunk = chunk;
    hipError_t e = l.inplace
                       ? sa::launch_kvcache_prefill_plan(ckv, lmax, cu, qstart, qo_base, st)
                       : sa::launch_kvcache_prefill_gather(kc, q, k_new, v_new, chunk, num_q_heads, n_seen, lmax,
                                                           ws + l.kp, ws + l.vp, l.direct ? nullptr : ws + l.qp,
                                                           cu, qstart, qo_base, st);
    if (e == hipSuccess) {
      sa::Prefill p;
      p.cu = cu;
      p.batch = 2 * cache->batch;
      p.total = cache->batch * lmax;
      p.max_seqlen = lmax;
      p.hq = num_q_heads;
      p.hkv = cache->num_kv_heads;
      p.d = cache->head_dim;
      p.dtype = SINK_ATTN_BF16;
      p.scale = softmax_scale;
      p.n_sink = cache->n_sink;
      p.window = cache->window;
      p.blocks = nullptr;
      p.nqb = 0;
      p.max_blocks = 0;
      p.sink = learnable_sink;
      p.qstart = qstart;
      p.qo_base = qo_base;
      if (l.direct != sa::fwd_mfma_supported(p))
        return fail(SINK_ATTN_HIP_ERROR, "internal: chunked prefill path mismatch");
      e = l.inplace  ? sa::launch_fwd_mfma_cache(p, ckv, q, o, lse, s, st)
          : l.direct ? sa::launch_fwd_mfma(p, q, ws + l.kp, ws + l.vp, o, lse, s, nullptr, st)
                   : sa::launch_fwd_generic(p, ws + l.qp, ws + l.kp, ws + l.vp, ws + l.op, lsep, sp, nullptr, st);
    }
    if (e == hipSuccess && !l.direct)
      e = sa::launch_kvcache_prefill_scatter(kc, chunk, num_q_heads, n_seen, lmax, ws + l.op, lsep, sp, o,
                                             lse, s, st);
    return hip_status(e, "sink_attn_kvcache_prefill launch");
  } catch (...) {
    return fail(SINK_ATTN_HIP_ERROR, "unexpected exception in sink_attn_kvcache_prefill");
  }
}

int sink_attn_decode(const sink_attn_decode_desc* desc, const void* q, const void* k_cache,
                     const void* v_cache, void* o, float* lse, float* s, void* workspace,
                     size_t workspace_bytes, void* stream) {
  try {
    SA_TRY(sink_attn_check_decode(desc, q, k_cache, v_cache, o, lse, s, workspace_bytes));
    const sa::Decode p = to_decode(desc);
    if (p.batch == 0) return SINK_ATTN_OK;
    hipStream_t st = static_cast<hipStream_t>(stream);
    hipError_t e = sa::launch_decode(p, q, k_cache, v_cache, o, lse, s,
                                     static_cast<float*>(workspace), st);
    return hip_status(e, "sink_attn_decode launch");
  } catch (...) {
    return fail(SINK_ATTN_HIP_ERROR, "unexpected exception in sink_attn_decode");
  }
}

int sink_attn_debug_visit_map(const sink_attn_prefill_desc* desc, uint8_t* out, size_t out_bytes,
                              void* stream) {
  try {
    SA_TRY(check_prefill_desc(desc));
    if (desc->max_seqlen > 4096)
      return fail(SINK_ATTN_UNSUPPORTED, "visit map needs max_seqlen <= 4096");
    if (desc->total_tokens == 0) return SINK_ATTN_OK;
    SA_TRY(check_ptr(out, "out", 1, true));
    const size_t need = static_cast<size_t>(desc->num_kv_heads) * desc->max_seqlen *
                        static_cast<size_t>(desc->total_tokens);
    if (out_bytes < need)
      return fail(SINK_ATTN_INVALID_ARGUMENT, "out_bytes %zu < Hkv*max_seqlen*total_tokens = %zu",
                  out_bytes, need);
    hipStream_t st = static_cast<hipStream_t>(stream);
    hipError_t e = sa::launch_fill_zero_bytes(out, out_bytes, st);
    if (e == hipSuccess) e = sa::launch_visit_map(to_prefill(desc), out, st);
    return hip_status(e, "sink_attn_debug_visit_map launch");
  } catch (...) {
    return fail(SINK_ATTN_HIP_ERROR, "unexpected exception in sink_attn_debug_visit_map");
  }
}

}  // extern "C"
