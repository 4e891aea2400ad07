// Rolling KV cache of StreamingLLM: the first n_sink tokens of a stream stay
// for good and the most recent `window` tokens live in a ring ("What is
// Attention Sink? ... StreamingLLM" (model.playoffer.cn), core idea: a fixed
// first-token segment plus a sliding window whose oldest token a new one
// replaces; "Attention Sink" (lijianxiong.space), H2O section: the recent part
// as a circular queue).  The token at stream position p goes to sink slot p
// when p < n_sink, else to ring slot (p - n_sink) mod window.
//
// Optional 8-bit ring: the same page's engineering notes keep the first
// tokens, which take a large share of the attention, in high precision when
// the KV cache is quantised.  Ring rows are e4m3 (OCP: 4 exponent bits, 3
// mantissa bits, 448 the largest value) with one float32 scale per (slot,
// KV head) row: scale = amax / 448, code = e4m3(x * (448 / amax)), rounded to
// nearest even by the hardware conversion; a zero row gets scale 0.
#include "common.cuh"
#include "stream_rows.cuh"

namespace sa {
namespace kvc {

constexpr float kE4m3Max = 448.f;

// 8 lanes per (sequence b, chunk token c, KV head g), every load of a lane
// issued before its first store: writes the K and V rows of the token to its
// slot, or nothing when a later token of the same chunk takes that slot (only
// the last `window` non-first tokens survive, so no slot gets two writers).
constexpr int kAppendLanes = 8;      // lanes per row
constexpr int kAppendPieces = 2;     // 16-byte pieces of K and of V per lane and pass

// Copies a K row and a V row of n 16-byte pieces with kAppendLanes lanes:
// pieces sub, sub + 8, ... (each load instruction reads 128 contiguous bytes),
// every load of a pass issued before its stores.
__device__ __forceinline__ void copy_rows(const uint16_t* ks, const uint16_t* vs, uint16_t* kd, uint16_t* vd,
                                          int n, int sub) {
  for (int e0 = 0; e0 < n; e0 += kAppendLanes * kAppendPieces) {
    u32x4 kr[kAppendPieces], vr[kAppendPieces];
#pragma unroll
    for (int j = 0; j < kAppendPieces; ++j) {
      const int e = e0 + sub + kAppendLanes * j;
      if (e < n) {
        kr[j] = *reinterpret_cast<const u32x4*>(ks + 8 * e);
        vr[j] = *reinterpret_cast<const u32x4*>(vs + 8 * e);
      }
    }
#pragma unroll
    for (int j = 0; j < kAppendPieces; ++j) {
      const int e = e0 + sub + kAppendLanes * j;
      if (e < n) {
        *reinterpret_cast<u32x4*>(kd + 8 * e) = kr[j];
        *reinterpret_cast<u32x4*>(vd + 8 * e) = vr[j];
      }
    }
  }
}
template <bool QUANT>
__global__ __launch_bounds__(256) void append_kernel(KvCache c, const uint16_t* __restrict__ k_new,
                                                     const uint16_t* __restrict__ v_new, int chunk,
                                                     const int32_t* __restrict__ n_seen) {
  const size_t unit = static_cast<size_t>(blockIdx.x) * (256 / kAppendLanes) + threadIdx.x / kAppendLanes;
  const int sub = threadIdx.x % kAppendLanes;
  if (unit >= static_cast<size_t>(c.batch) * chunk * c.hkv) return;
  const int g = static_cast<int>(unit % c.hkv);
  const int cc = static_cast<int>((unit / c.hkv) % chunk);
  const int b = static_cast<int>(unit / (static_cast<size_t>(c.hkv) * chunk));
  const int D = c.d;
  const long long p0 = max(n_seen[b], 0);               // a negative count reads as an empty stream
  const long long p = p0 + cc;
  const long long total = p0 + chunk;
  if (p >= c.n_sink && p < total - c.window) return;      // evicted within this chunk (uniform per row)
  const size_t src = ((static_cast<size_t>(b) * chunk + cc) * c.hkv + g) * D;
  const bool is_sink = p < c.n_sink;
  const int ring = is_sink ? 0 : static_cast<int>((p - c.n_sink) % c.window);

  if (!QUANT || is_sink) {
    uint16_t* dk;
    uint16_t* dv;
    if (!QUANT) {
      const int slot = is_sink ? static_cast<int>(p) : c.n_sink + ring;
      const size_t dst = ((static_cast<size_t>(b) * (c.n_sink + c.window) + slot) * c.hkv + g) * D;
      dk = static_cast<uint16_t*>(c.k) + dst;
      dv = static_cast<uint16_t*>(c.v) + dst;
    } else {
      const size_t dst = ((static_cast<size_t>(b) * c.n_sink + p) * c.hkv + g) * D;
      dk = static_cast<uint16_t*>(c.sink_k) + dst;
      dv = static_cast<uint16_t*>(c.sink_v) + dst;
    }
    copy_rows(k_new + src, v_new + src, dk, dv, D / 8, sub);
    return;
  }

  // 8-bit ring row (head_dim 128): lane sub holds values 16 sub .. 16 sub + 15
  // of the K row and of the V row; amax over the row, then the codes, two per
  // conversion, 16 contiguous bytes per lane.
  const size_t dst = ((static_cast<size_t>(b) * c.window + ring) * c.hkv + g) * D;
  const size_t sidx = (static_cast<size_t>(b) * c.hkv + g) * c.window + ring;
  u32x4 raw[2][2];                                       // [K, V][piece]
#pragma unroll
  for (int which = 0; which < 2; ++which)
#pragma unroll
    for (int j = 0; j < 2; ++j)
      raw[which][j] = *reinterpret_cast<const u32x4*>((which == 0 ? k_new : v_new) + src + 16 * sub + 8 * j);
#pragma unroll
  for (int which = 0; which < 2; ++which) {
    float xv[16];
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        xv[8 * j + 2 * q] = __uint_as_float(raw[which][j][q] << 16);
        xv[8 * j + 2 * q + 1] = __uint_as_float(raw[which][j][q] & 0xffff0000u);
      }
    float amax = 0.f;
#pragma unroll
    for (int j = 0; j < 16; ++j) amax = fmaxf(amax, fabsf(xv[j]));
#pragma unroll
    for (int off = kAppendLanes / 2; off >= 1; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off, kAppendLanes));
    const float scale = amax > 0.f ? amax / kE4m3Max : 0.f;
    const float inv = amax > 0.f ? kE4m3Max / amax : 0.f;
    u32x4 codes = {0u, 0u, 0u, 0u};
    if (amax > 0.f) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        int w = __builtin_amdgcn_cvt_pk_fp8_f32(xv[4 * j] * inv, xv[4 * j + 1] * inv, 0, false);
        w = __builtin_amdgcn_cvt_pk_fp8_f32(xv[4 * j + 2] * inv, xv[4 * j + 3] * inv, w, true);
        codes[j] = static_cast<uint32_t>(w);
      }
    }
    *reinterpret_cast<u32x4*>((which == 0 ? c.win_k : c.win_v) + dst + 16 * sub) = codes;
    if (sub == 0) (which == 0 ? c.win_k_scale : c.win_v_scale)[sidx] = scale;
  }
}

// ---------------------------------------------------------------------------
// Chunked prefill against the cache.  Query row c of sequence b is stream
// position P0 + c (P0 = n_seen[b], the tokens the cache has taken so far); it
// sees the keys StreamingLLM keeps for that position: the first n_sink tokens
// and the positions within the window, from the cache (before this chunk is
// appended) and from the chunk itself, causally.  Each sequence is laid out
// as one packed sample of the prefill forward:
//   [ns cached first tokens | nw ring tokens in position order | C chunk tokens]
// (ns = min(P0, n_sink), nw = min(max(P0 - n_sink, 0), window)).  Local index
// differences then equal position differences for every key the window can
// reach and the first-token keys keep local index = position, so the prefill
// mask of that sample is the StreamingLLM mask of the stream.  Sequence b owns
// rows [b*Lmax, (b+1)*Lmax), Lmax = n_sink + window + C: the sample, then a
// padding sample for the rest of the segment whose rows all lie before its
// qstart (the forward skips them).
// ---------------------------------------------------------------------------
struct Seg {
  int ns, nw, L;
};
__device__ __forceinline__ Seg segment(const KvCache& c, int p0, int chunk) {
  Seg s;
  p0 = max(p0, 0);                                    // negative counts read as an empty stream
  s.ns = min(p0, c.n_sink);
  s.nw = min(max(p0 - c.n_sink, 0), c.window);
  s.L = s.ns + s.nw + chunk;
  return s;
}

// Chunked prefill with keys read in place.  Block (b, i, part): seam kind
// i of stream b (see stream_rows.cuh), rows 4 part .. 4 part + 3 of its
// tile, copied to staging slot i when that kind owns the tile; block
// (b, 0, 0) also writes the bounds of the stream's sample (2b: first tokens,
// ring, chunk) and of the padding sample after it (2b + 1, no query rows),
// and where the chunk rows sit in the caller's [B, chunk] Q and outputs.
constexpr int kStageParts = sa::kSeamRows / 4;
__global__ __launch_bounds__(256) void prefill_plan_kernel(CacheKv ckv, int lmax, int32_t* __restrict__ cu,
                                                           int32_t* __restrict__ qstart,
                                                           int32_t* __restrict__ qo_base) {
  const int part = blockIdx.x % kStageParts;
  const int i = (blockIdx.x / kStageParts) % sa::kSeamSlots;
  const int b = blockIdx.x / (kStageParts * sa::kSeamSlots);
  sa::StreamRows sr;
  sr.init(ckv.n_seen[b], ckv.n_sink, ckv.window, ckv.chunk);
  if (i == 0 && part == 0 && threadIdx.x == 0) {
    cu[2 * b] = b * lmax;
    cu[2 * b + 1] = b * lmax + sr.L;
    qstart[2 * b] = sr.L - ckv.chunk;
    qstart[2 * b + 1] = lmax - sr.L;
    qo_base[2 * b] = b * ckv.chunk - (sr.L - ckv.chunk);
    qo_base[2 * b + 1] = 0;
    if (b == ckv.batch - 1) cu[2 * ckv.batch] = ckv.batch * lmax;
  }
  const int kt = sr.seam_tile(i);
  int unused;
  if (kt < 0 || sr.tile_kind(kt, &unused) != 2 || sr.seam_slot(kt) != i) return;
  const int kvs = ckv.hkv * 128;
  const int pieces = kvs / 8;                         // 16-byte pieces of a row
  const size_t stage0 = (static_cast<size_t>(b) * sa::kSeamSlots + i) * sa::kSeamRows;
  for (int e = threadIdx.x; e < 4 * pieces; e += blockDim.x) {
    const int rr = 4 * part + e / pieces;             // row inside the tile
    const int r = kt * sa::kSeamRows + rr;
    if (r >= sr.L) break;                             // rows beyond the stream: never read
    int row;
    const bool in_cache = sr.source(r, &row);
    const size_t src = (in_cache ? static_cast<size_t>(b) * ckv.slots + row
                                 : static_cast<size_t>(b) * ckv.chunk + row) * kvs + 8 * (e % pieces);
    const size_t dst = (stage0 + rr) * kvs + 8 * (e % pieces);
    *reinterpret_cast<u32x4*>(ckv.sk + dst) = *reinterpret_cast<const u32x4*>((in_cache ? ckv.k : ckv.kn) + src);
    *reinterpret_cast<u32x4*>(ckv.sv + dst) = *reinterpret_cast<const u32x4*>((in_cache ? ckv.v : ckv.vn) + src);
  }
}

// 16 lanes per (sequence b, segment row i, KV head g): the K and V row of the
// key at row i (cache or chunk) and, for chunk rows with qp set, the G query
// rows.  Also writes the samples' bounds (cu: 2B + 1, qstart: 2B) and, when
// qo_base is set, where each sample's rows sit in the caller's [B, chunk]
// Q and outputs (the forward then reads and writes those directly).
template <bool QUANT>
__global__ __launch_bounds__(256) void prefill_gather_kernel(KvCache c, const uint16_t* __restrict__ q,
                                                             const uint16_t* __restrict__ k_new,
                                                             const uint16_t* __restrict__ v_new, int chunk,
                                                             int hq, const int32_t* __restrict__ n_seen,
                                                             int lmax, uint16_t* __restrict__ kp,
                                                             uint16_t* __restrict__ vp,
                                                             uint16_t* __restrict__ qp, int32_t* __restrict__ cu,
                                                             int32_t* __restrict__ qstart,
                                                             int32_t* __restrict__ qo_base) {
  const size_t unit = static_cast<size_t>(blockIdx.x) * (256 / kAppendLanes) + threadIdx.x / kAppendLanes;
  const int sub = threadIdx.x % kAppendLanes;
  const size_t units = static_cast<size_t>(c.batch) * lmax * c.hkv;
  if (unit >= units) return;
  const int g = static_cast<int>(unit % c.hkv);
  const int i = static_cast<int>((unit / c.hkv) % lmax);
  const int b = static_cast<int>(unit / (static_cast<size_t>(c.hkv) * lmax));
  const int D = c.d;
  const int p0 = n_seen[b];
  const Seg sg = segment(c, p0, chunk);
  if (i == 0 && g == 0 && sub == 0) {
    cu[2 * b] = b * lmax;
    cu[2 * b + 1] = b * lmax + sg.L;
    qstart[2 * b] = sg.L - chunk;
    qstart[2 * b + 1] = lmax - sg.L;
    if (qo_base != nullptr) {                         // chunk row cc read and written at b*chunk + cc
      qo_base[2 * b] = b * chunk - (sg.L - chunk);
      qo_base[2 * b + 1] = 0;
    }
    if (b == c.batch - 1) cu[2 * c.batch] = c.batch * lmax;
  }
  if (i >= sg.L) return;
  const size_t dst = ((static_cast<size_t>(b) * lmax + i) * c.hkv + g) * D;
  const int nchunk8 = D / 8;                          // 16-byte pieces of a bf16 row
  if (i >= sg.ns + sg.nw) {                           // a chunk token
    const int cc = i - sg.ns - sg.nw;
    const size_t src = ((static_cast<size_t>(b) * chunk + cc) * c.hkv + g) * D;
    copy_rows(k_new + src, v_new + src, kp + dst, vp + dst, nchunk8, sub);
    const int G = qp != nullptr ? hq / c.hkv : 0;    // Q rows only for a packed copy
    for (int hh = 0; hh < G; ++hh) {
      const int h = g * G + hh;
      const size_t qs = ((static_cast<size_t>(b) * chunk + cc) * hq + h) * D;
      const size_t qd = ((static_cast<size_t>(b) * lmax + i) * hq + h) * D;
      for (int e = sub; e < nchunk8; e += kAppendLanes)
        *reinterpret_cast<u32x4*>(qp + qd + 8 * e) = *reinterpret_cast<const u32x4*>(q + qs + 8 * e);
    }
    return;
  }
  const bool first = i < sg.ns;
  // position of the key and its ring slot
  const int ring = first ? 0 : ((p0 - sg.nw + (i - sg.ns)) - c.n_sink) % c.window;
  if (!QUANT || first) {
    const uint16_t* sk;
    const uint16_t* sv;
    if (!QUANT) {
      const int slot = first ? i : c.n_sink + ring;
      const size_t o = ((static_cast<size_t>(b) * (c.n_sink + c.window) + slot) * c.hkv + g) * D;
      sk = static_cast<const uint16_t*>(c.k) + o;
      sv = static_cast<const uint16_t*>(c.v) + o;
    } else {
      const size_t o = ((static_cast<size_t>(b) * c.n_sink + i) * c.hkv + g) * D;
      sk = static_cast<const uint16_t*>(c.sink_k) + o;
      sv = static_cast<const uint16_t*>(c.sink_v) + o;
    }
    copy_rows(sk, sv, kp + dst, vp + dst, nchunk8, sub);
    return;
  }
  // 8-bit ring row (head_dim 128): code * scale in float32, rounded to
  // bfloat16; lane sub converts pieces sub and sub + 8 of K and of V, its
  // loads issued before its stores.
  const size_t o = ((static_cast<size_t>(b) * c.window + ring) * c.hkv + g) * D;
  const size_t si = (static_cast<size_t>(b) * c.hkv + g) * c.window + ring;
  u32x2 w[2][2];                                      // [K, V][piece]
#pragma unroll
  for (int which = 0; which < 2; ++which)
#pragma unroll
    for (int j = 0; j < 2; ++j)
      w[which][j] = *reinterpret_cast<const u32x2*>((which == 0 ? c.win_k : c.win_v) + o +
                                                    8 * (sub + kAppendLanes * j));
  const float scs[2] = {c.win_k_scale[si], c.win_v_scale[si]};
#pragma unroll
  for (int which = 0; which < 2; ++which) {
    uint16_t* out = (which == 0 ? kp : vp) + dst;
#pragma unroll
    for (int jp = 0; jp < 2; ++jp) {
      u32x4 r;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t word = w[which][jp][j >> 1];
        const auto f = (j & 1) ? __builtin_amdgcn_cvt_pk_f32_fp8(word, true)
                               : __builtin_amdgcn_cvt_pk_f32_fp8(word, false);
        bf16x2 v2 = {static_cast<__bf16>(f[0] * scs[which]), static_cast<__bf16>(f[1] * scs[which])};
        r[j] = __builtin_bit_cast(uint32_t, v2);
      }
      *reinterpret_cast<u32x4*>(out + 8 * (sub + kAppendLanes * jp)) = r;
    }
  }
}

// 16 lanes per (sequence b, chunk row c, query head h): O, LSE and s of the
// chunk rows from the packed forward's outputs.
__global__ __launch_bounds__(256) void prefill_scatter_kernel(KvCache c, int chunk, int hq,
                                                              const int32_t* __restrict__ n_seen, int lmax,
                                                              const uint16_t* __restrict__ op,
                                                              const float* __restrict__ lsep,
                                                              const float* __restrict__ sp,
                                                              uint16_t* __restrict__ o, float* __restrict__ lse,
                                                              float* __restrict__ s) {
  const size_t unit = static_cast<size_t>(blockIdx.x) * 16 + (threadIdx.x >> 4);
  const int sub = threadIdx.x & 15;
  if (unit >= static_cast<size_t>(c.batch) * chunk * hq) return;
  const int h = static_cast<int>(unit % hq);
  const int cc = static_cast<int>((unit / hq) % chunk);
  const int b = static_cast<int>(unit / (static_cast<size_t>(hq) * chunk));
  const Seg sg = segment(c, n_seen[b], chunk);
  const size_t src = (static_cast<size_t>(b) * lmax + (sg.L - chunk) + cc) * hq + h;
  const size_t dst = unit;                            // (b * chunk + cc) * hq + h
  const int D = c.d;
  for (int e = sub; e < D / 8; e += 16)
    *reinterpret_cast<u32x4*>(o + dst * D + 8 * e) = *reinterpret_cast<const u32x4*>(op + src * D + 8 * e);
  if (sub == 0) {
    lse[dst] = lsep[src];
    if (s != nullptr) s[dst] = sp[src];
  }
}
}  // namespace kvc

hipError_t launch_kvcache_append(const KvCache& c, const void* k_new, const void* v_new, int chunk,
                                 const int32_t* n_seen, hipStream_t st) {
  const long long rows = static_cast<long long>(c.batch) * chunk * c.hkv;
  if (rows <= 0) return hipSuccess;
  auto kern = c.quantized ? kvc::append_kernel<true> : kvc::append_kernel<false>;
  constexpr int per_block = 256 / kvc::kAppendLanes;        // rows per workgroup
  hipLaunchKernelGGL(kern, dim3(static_cast<unsigned>((rows + per_block - 1) / per_block)), dim3(256), 0, st,
                     c, static_cast<const uint16_t*>(k_new), static_cast<const uint16_t*>(v_new), chunk,
                     n_seen);
  return hipGetLastError();
}

hipError_t launch_kvcache_prefill_gather(const KvCache& c, const void* q, const void* k_new,
                                         const void* v_new, int chunk, int hq, const int32_t* n_seen,
                                         int lmax, void* kp, void* vp, void* qp, int32_t* cu,
                                         int32_t* qstart, int32_t* qo_base, hipStream_t st) {
  const size_t units = static_cast<size_t>(c.batch) * lmax * c.hkv;
  if (units == 0) return hipSuccess;
  auto kern = c.quantized ? kvc::prefill_gather_kernel<true> : kvc::prefill_gather_kernel<false>;
  constexpr int per_block = 256 / kvc::kAppendLanes;        // rows per workgroup
  hipLaunchKernelGGL(kern, dim3(static_cast<unsigned>((units + per_block - 1) / per_block)), dim3(256), 0, st, c,
                     static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k_new),
                     static_cast<const uint16_t*>(v_new), chunk, hq, n_seen, lmax, static_cast<uint16_t*>(kp),
                     static_cast<uint16_t*>(vp), static_cast<uint16_t*>(qp), cu, qstart, qo_base);
  return hipGetLastError();
}

hipError_t launch_kvcache_prefill_plan(const CacheKv& ckv, int lmax, int32_t* cu, int32_t* qstart,
                                       int32_t* qo_base, hipStream_t st) {
  if (ckv.batch == 0) return hipSuccess;
  const long long grid = static_cast<long long>(ckv.batch) * sa::kSeamSlots * kvc::kStageParts;
  hipLaunchKernelGGL(kvc::prefill_plan_kernel, dim3(static_cast<unsigned>(grid)), dim3(256), 0, st, ckv, lmax,
                     cu, qstart, qo_base);
  return hipGetLastError();
}

hipError_t launch_kvcache_prefill_scatter(const KvCache& c, int chunk, int hq, const int32_t* n_seen,
                                          int lmax, const void* op, const float* lsep, const float* sp,
                                          void* o, float* lse, float* s, hipStream_t st) {
  const size_t units = static_cast<size_t>(c.batch) * chunk * hq;
  if (units == 0) return hipSuccess;
  hipLaunchKernelGGL(kvc::prefill_scatter_kernel, dim3(static_cast<unsigned>((units + 15) / 16)), dim3(256), 0,
                     st, c, chunk, hq, n_seen, lmax, static_cast<const uint16_t*>(op), lsep, sp,
                     static_cast<uint16_t*>(o), lse, s);
  return hipGetLastError();
}

}  // namespace sa
