// Forward for bfloat16, head_dim 128, on gfx950 matrix cores.
//
// What is computed is the forward of "Attention Sink, Learnable Sink and
// dsink" (notes.kuangjux.top): scores x = alpha <Q, K> (s1), softmax over the
// valid keys, O = sum P V (s1), with the sink applied as the output scale
// s = sigma(L_orig - a_h) and O_new = s O_orig (s4).  lse is L_orig.
//
// Work decomposition (geometry and schedule in qmajor.cuh):
//   * A workgroup is 4 wavefronts (one per SIMD) of one KV head, two
//     workgroups per CU; each wavefront owns 32 query rows of one query
//     head.  Two independent workgroups per CU rather than one of 8
//     wavefronts: their barriers do not couple, so one workgroup's mask, max
//     and barrier time overlaps the other's matrix work (measured: the same
//     rate at a lower clock on the GQA workload, 5-12% faster on the window
//     and chunked workloads, for twice the K/V tile loads).  Keys come in 64-key
//     tiles loaded straight into LDS (buffer loads issued from asm blocks so
//     they overlap a whole step; see qmajor.cuh), and only the
//     tiles the mask can reach are visited: every causal tile, or the
//     first-token tiles plus the window tiles, or the union of the selected
//     blocks.  Each wavefront classifies a tile as empty (skipped), full, or
//     mixed (element mask).
//   * Scores are computed transposed, S^T = K Q^T, with
//     v_mfma_f32_32x32x16_bf16: in the 32x32 result each lane holds 16 keys
//     of ONE query (its column), so the online-softmax max and sum stay in
//     registers plus one v_permlane32_swap between the lane halves.  The same
//     registers, converted to bf16, are the B operand of O^T += V^T P^T; the
//     V^T operand comes from the staged V tile by ds_read_b64_tr_b16.
//   * Software pipeline over three tiles: a step masks the scores of tile
//     j+1 and takes their row max, then runs one straight-line block of 16
//     slots, each holding a score MFMA of tile j+2 (K fragments read two
//     slots ahead), two exponentials of tile j+1 with their row sum, an
//     O += V P MFMA of tile j and two more exponentials.  A wavefront's
//     independent vector ALU work issues while its own MFMAs execute, so the
//     exponentials no longer wait for the score MFMAs of their tile.  K runs
//     two tiles ahead of V; K and V each have two LDS buffers.
//   * Online softmax with lazy rescaling: the exponent base only moves when a
//     row's max grows by more than 2^8 (P <= 256), which is exact because O
//     and l always share the same base.
//   * LDS addresses: the per-lane swizzled offsets are computed once; the
//     loop is unrolled by two so buffer offsets are instruction immediates.
//   * Optional first-token gate (instantiation GATE): the share of the
//     real-token softmax that is not on the sample's first key, 1 - A_0, the
//     vanilla-attention gate of "Paper notes: Attention Sink and the native
//     MoE in attention layers" s2 (G = 1 - A_sink) and s5 (its LSE form).
//     Key 0 of a sample is element (M-tile 0, i 0) of the lanes of half 0 in
//     key tile 0, so its probability is kept beside the row sum (rescaled
//     with it) and the epilogue writes (l - l_0) / l.
//   * Keys and values in place (instantiation CACHE, chunked prefill against
//     a rolling cache): a sample's key rows are the stream's kept first
//     tokens, its ring tokens oldest first, then the new chunk.  A 64-row
//     tile inside one contiguous run (first tokens, ring rows on one side of
//     the wrap, chunk rows) loads as any tile, from a per-tile base in the
//     cache or the chunk; the at most three tiles of a stream that hold a
//     seam load from copies staged beforehand (stream_rows.cuh).
#include <cstdlib>
#include <type_traits>

#include "qmajor.cuh"
#include "stream_rows.cuh"

namespace sa {
namespace fwd128 {

using namespace qm;

constexpr float kRescaleLog2 = 8.f;    // lazy-rescale threshold (log2 units)
constexpr int FNW = 4;                 // wavefronts per workgroup (two workgroups per CU)
constexpr int FQW = 32;                // query rows per wavefront

typedef __attribute__((address_space(3))) char lds_char;

__device__ __forceinline__ float xhalf_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __builtin_fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xhalf_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ bf16x8 lds_frag(const lds_char* base, int byte_off) {
  return __builtin_bit_cast(bf16x8, *reinterpret_cast<const __attribute__((address_space(3))) u32x4*>(base + byte_off));
}
__device__ __forceinline__ u32x2 lds_tr(const lds_char* base, int byte_off) {
  return __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                                       (__attribute__((address_space(3))) i16x4*)(base + byte_off)));
}

template <bool GATE, bool CACHE>
__global__ __launch_bounds__(64 * FNW, 2) void fwd_kernel(Prefill p, Geo geo,
                                                          const uint16_t* __restrict__ Q,
                                                          const uint16_t* __restrict__ K,
                                                          const uint16_t* __restrict__ V,
                                                          uint16_t* __restrict__ O,
                                                          float* __restrict__ lse_out,
                                                          float* __restrict__ s_out,
                                                          float* __restrict__ gate_out, CacheKv ckv) {
  __shared__ __attribute__((aligned(16))) uint16_t kbuf[2][TILE];
  __shared__ __attribute__((aligned(16))) uint16_t vbuf[2][TILE];
  __shared__ uint32_t bitmap[BITMAP_LDS_WORDS];

  const WgCoord wc = wg_coord(geo, p.batch, blockIdx.x);
  const int t0 = p.cu[wc.b];
  const int L = p.cu[wc.b + 1] - t0;
  const int p0 = wc.pt * geo.P;
  if (p0 >= L) return;                               // uniform over the workgroup
  const int p1 = min(L, p0 + geo.P);
  const int qs = p.qstart != nullptr ? p.qstart[wc.b] : 0;   // rows before qs: not needed
  if (p1 <= qs) return;
  const int tq = p.qo_base != nullptr ? p.qo_base[wc.b] : t0;   // row of local 0 in Q, O, LSE, s

  const int tid = threadIdx.x;
  // wavefront index as a scalar, so per-wavefront tile decisions are
  // uniform branches rather than exec-masked regions
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int gq = lane >> 5;
  const int G = p.hq / p.hkv;
  const int g = wc.g;
  const int h = g * G + wc.hg * geo.hw + w / geo.wph;
  const int wq0 = p0 + (w % geo.wph) * FQW;
  const int wq1 = min(L, wq0 + FQW);
  const int qi = wq0 + l32;                          // this lane's query row
  const int qoff = p.blocks ? q_block_offset(p.cu, wc.b) : 0;

  // Q^T as the B operand: lane (query l32, half gq) holds dims gq*64 + ks*8
  // .. +8 for k-step ks (the K fragments use the same order).
  bf16x8 qf[8];
  if (qi < L && qi >= qs) {
    const uint16_t* src = Q + (static_cast<size_t>(tq + qi) * p.hq + h) * D + gq * 64;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks)
      qf[ks] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(src + ks * 8));
  } else {
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) qf[ks] = __builtin_bit_cast(bf16x8, u32x4{0u, 0u, 0u, 0u});
  }
  // Loaded before any tile DMA is in flight (the compiler counts only its own
  // loads): consuming the fragments here makes it wait for them up front.
  asm volatile("" ::"v"(qf[0]), "v"(qf[1]), "v"(qf[2]), "v"(qf[3]), "v"(qf[4]), "v"(qf[5]),
               "v"(qf[6]), "v"(qf[7]));

  // Per-lane swizzled LDS byte offsets (tile rows are 256 bytes).
  //   K fragment (mt, ks): row mt*32 + l32, logical chunk gq*8 + ks.
  //   V^T fragment (cc, dt): rows 16cc + ra0 and 16cc + ra0 + 8, logical
  //   chunk dt*4 + c4, byte 2*(d & 7) inside it (see tr_frag in qmajor.cuh).
  int koff[8], voa[4], vob[4];
  {
    const int sk = swz16(l32);
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) koff[ks] = l32 * 256 + (((gq * 8 + ks) ^ sk) << 4);
    const int l16 = lane & 15, grp = lane >> 4;
    const int ra0 = 4 * (grp >> 1) + (l16 >> 2);
    const int d4 = 16 * (grp & 1) + 4 * (l16 & 3);           // dim offset inside the 32-dim block
    const int c4 = d4 >> 3, off = (d4 & 7) * 2;
    const int sa_ = swz16(ra0), sb_ = swz16(ra0 + 8);
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) {
      voa[dt] = ra0 * 256 + (((dt * 4 + c4) ^ sa_) << 4) + off;
      vob[dt] = (ra0 + 8) * 256 + (((dt * 4 + c4) ^ sb_) << 4) + off;
    }
  }

  Sched sc = make_sched(p, L, qoff, g, p0, p1, bitmap);

  const float c = p.scale * kLog2e;                  // exp(scale*x) = exp2(c*x)
  const float thr = kRescaleLog2 / c;                // raw-score rescale threshold
  f32x16 oacc[4];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int i = 0; i < 16; ++i) oacc[dt][i] = 0.f;
  float mrun = -kInf, lsum = 0.f;
  float l0 = 0.f;                                    // GATE: P of the sample's first key

  const int kvs = p.hkv * D;
  const uint16_t* Kg = CACHE ? nullptr : K + static_cast<size_t>(t0) * kvs + g * D;
  const uint16_t* Vg = CACHE ? nullptr : V + static_cast<size_t>(t0) * kvs + g * D;
  DmaTiles<FNW> ld;
  ld.init(w, lane, kvs);
  const uint32_t kbuf0 = lds_address(&kbuf[0][0]), vbuf0 = lds_address(&vbuf[0][0]);
  // CACHE: sample 2 sb is stream sb's keys (first tokens, ring, chunk); each
  // key tile is read from one base (wave-uniform): a contiguous run of the
  // cache or of the chunk, or the stream's staged copy of a seam tile.
  int c_sb = 0;
  StreamRows sr{};
  if constexpr (CACHE) {
    c_sb = wc.b >> 1;
    sr.init(ckv.n_seen[c_sb], ckv.n_sink, ckv.window, ckv.chunk);
  }
  auto cache_base = [&](const uint16_t* cbase, const uint16_t* nbase, const uint16_t* sbase,
                        int kt) -> const uint16_t* {
    int row;
    const int kind = sr.tile_kind(kt, &row);
    size_t r;
    const uint16_t* base;
    if (kind == 0) {
      base = nbase;
      r = static_cast<size_t>(c_sb) * ckv.chunk + row;
    } else if (kind == 1) {
      base = cbase;
      r = static_cast<size_t>(c_sb) * ckv.slots + row;
    } else {
      base = sbase;
      r = (static_cast<size_t>(c_sb) * kSeamSlots + sr.seam_slot(kt)) * kSeamRows;
    }
    return base + r * kvs + g * D;
  };
  auto issue_k = [&](int kt, int st) {
    const int k0 = kt * BN;
    const uint32_t lds = kbuf0 + static_cast<uint32_t>(st * TILE * 2);
    ld.load(CACHE ? cache_base(ckv.k, ckv.kn, ckv.sk, kt) : Kg + static_cast<size_t>(k0) * kvs, L - k0, lds);
  };
  auto issue_v = [&](int kt, int st) {
    const int k0 = kt * BN;
    const uint32_t lds = vbuf0 + static_cast<uint32_t>(st * TILE * 2);
    ld.load(CACHE ? cache_base(ckv.v, ckv.vn, ckv.sv, kt) : Vg + static_cast<size_t>(k0) * kvs, L - k0, lds);
  };
  auto tile_class = [&](int kt) { return kt >= 0 ? wave_tile_class(p, sc, p0, wq0, wq1, kt) : 0; };

  // S^T of a tile from K buffer ST.  The two 32-key halves alternate (two
  // independent accumulation chains) and every K fragment is read two MFMAs
  // ahead, in an order the scheduling barriers keep.
  auto scores = [&](auto ST, f32x16 (&s)[2]) __attribute__((always_inline)) {
    const lds_char* kb = (const lds_char*)(kbuf[decltype(ST)::value]);
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int i = 0; i < 16; ++i) s[mt][i] = 0.f;
    bf16x8 f[3];
    f[0] = lds_frag(kb, koff[0]);
    f[1] = lds_frag(kb, koff[0] + 8192);
#pragma unroll
    for (int x = 0; x < 16; ++x) {
      if (x + 2 < 16) f[(x + 2) % 3] = lds_frag(kb, koff[(x + 2) >> 1] + ((x + 2) & 1) * 8192);
      __builtin_amdgcn_sched_barrier(0);
      s[x & 1] = mfma32(f[x % 3], qf[x >> 1], s[x & 1]);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  // Element mask of a mixed tile: element i of M-tile mt is key
  // kb + dk with kb = k0 + 4gq and dk = 32mt + 8(i/4) + i%4 fixed per
  // element.  The pair is visible iff dk <= a (causal) and, with a window,
  // dk > wb (inside the window) or dk < cs (a kept first token), with a, wb,
  // cs per lane: one or two compares and a select per element.
  auto mask = [&](int kt, f32x16 (&s)[2]) __attribute__((always_inline)) {
    const int kb = kt * BN + 4 * gq;
    const int a = qi - kb;
    // a window longer than qi + 1 keys, or none, covers the same keys as
    // qi + 1 (all causal keys): visible iff a - wlen < dk <= a
    const int wlen = p.window > 0 ? min(p.window, qi + 1) : qi + 1;
    // per element: dk + nb < span with nb = -wb - 1; nb is pinned here so
    // the compiler does not hoist 32 per-element sums out of the loop
    int nb = wlen - a - 1;
    asm volatile("" : "+v"(nb));
    const uint32_t span = static_cast<uint32_t>(wlen);
    if (p.window <= 0 || kt * BN >= p.n_sink) {      // uniform: no kept token here
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int dk = 32 * mt + 8 * (i >> 2) + (i & 3);
          s[mt][i] = static_cast<uint32_t>(dk + nb) < span ? s[mt][i] : -kInf;
        }
    } else {
      const int cs = min(p.n_sink - kb, a + 1);      // kept first tokens: dk < cs
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int dk = 32 * mt + 8 * (i >> 2) + (i & 3);
          const bool vis = static_cast<uint32_t>(dk + nb) < span || dk < cs;
          s[mt][i] = vis ? s[mt][i] : -kInf;
        }
    }
  };
  // Row max of a tile and the lazy rescale to a new base of O, l and the
  // not yet accumulated probabilities pend (which share the old base).
  auto update_max = [&](const f32x16 (&s)[2], bool dead, bf16x8 (&pend)[4]) __attribute__((always_inline)) {
    float m0 = -kInf;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int i = 0; i < 16; ++i) m0 = __builtin_fmaxf(m0, s[mt][i]);
    m0 = dead ? -kInf : xhalf_max(m0);
    if (__ballot(m0 > mrun + thr) != 0) {
      const float mnew = __builtin_fmaxf(mrun, m0);
      const float f = (mrun == -kInf) ? 0.f : __builtin_amdgcn_exp2f((mrun - mnew) * c);
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int i = 0; i < 16; ++i) oacc[dt][i] *= f;
#pragma unroll
      for (int cc = 0; cc < 4; ++cc) {
        u32x4 u = __builtin_bit_cast(u32x4, pend[cc]);
#pragma unroll
        for (int e = 0; e < 4; ++e)
          u[e] = pack_bf16x2(__uint_as_float(u[e] << 16) * f, __uint_as_float(u[e] & 0xffff0000u) * f);
        pend[cc] = __builtin_bit_cast(bf16x8, u);
      }
      lsum *= f;
      if constexpr (GATE) l0 *= f;
      mrun = mnew;
    }
  };
  // P = 2^(c x - mb) in bf16 as four k-steps, l += sum P.  first: this is
  // key tile 0 (GATE keeps the first key's P).
  auto probs = [&](f32x16 (&s)[2], float mb, bool first, bf16x8 (&pf)[4]) __attribute__((always_inline)) {
    float ls = 0.f;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float e = __builtin_amdgcn_exp2f(__builtin_fmaf(s[mt][i], c, -mb));
        s[mt][i] = e;
        ls += e;
      }
    lsum += ls;
    if constexpr (GATE) {
      if (first) l0 += gq == 0 ? s[0][0] : 0.f;     // uniform branch
    }
#pragma unroll
    for (int cc = 0; cc < 4; ++cc) pf[cc] = pack_kstep(s[cc >> 1], cc & 1);
  };
  // O^T += V^T P^T from V buffer ST.
  auto pv = [&](auto ST, const bf16x8 (&pf)[4]) __attribute__((always_inline)) {
    const lds_char* vb = (const lds_char*)(vbuf[decltype(ST)::value]);
#pragma unroll
    for (int cc = 0; cc < 4; ++cc)
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) {
        const u32x2 a = lds_tr(vb, voa[dt] + cc * 4096);
        const u32x2 b = lds_tr(vb, vob[dt] + cc * 4096);
        oacc[dt] = mfma32(__builtin_bit_cast(bf16x8, u32x4{a[0], a[1], b[0], b[1]}), pf[cc], oacc[dt]);
      }
  };

  // Mask the scores of tile kt if it is mixed, move the base if needed and
  // return the exponent base c m for its P.  A tile this wavefront does not
  // see leaves the max alone and takes an infinite base, so its P is exactly
  // 0 and its scores need no rewrite.
  auto finish_scores = [&](int kt, f32x16 (&s)[2], bf16x8 (&pend)[4]) __attribute__((always_inline)) {
    const int cls = tile_class(kt);
    if (cls == 2) mask(kt, s);
    update_max(s, cls == 0, pend);
    float mb = (mrun == -kInf) ? 0.f : mrun * c;
    if (cls == 0) mb = kInf;
    asm volatile("" : "+v"(mb));                     // settled here, not inside the P V loop
    return mb;
  };

  // One pipeline step covers three tiles in schedule order, cur, nx, nx2:
  // P of cur is in pf (bf16) with V of cur in V buffer k%2, the raw scores
  // of nx are in s_nx, and K of nx2 is in K buffer k%2 (step k).  After the
  // mask, max and (rare) rescale of nx, one straight-line block runs the 16
  // score MFMAs of nx2 and the 16 O += V P MFMAs of cur with the
  // exponentials of nx between them: a wavefront's vector ALU work issues
  // while its own MFMAs execute.  K of the tile after nx2 goes to K buffer
  // (k+1)%2 and V of nx to V buffer (k+1)%2, both freed by the step before,
  // and are waited for at the step's end.  Steps run until cur is the last
  // tile; scores of tiles past the end come from whatever their K buffer
  // holds (always a loaded tile) and are discarded (P = 0).
  int t_cur = sc.next();
  if (t_cur >= 0) {
    int t_nx = sc.next();
    int t_nx2 = sc.next();
    issue_k(t_cur, 0);
    issue_v(t_cur, 0);
    issue_k(t_nx >= 0 ? t_nx : t_cur, 1);
    wait_bar<0>();
    bf16x8 pf[4];                                    // P of cur (bf16), not yet in O
#pragma unroll
    for (int cc = 0; cc < 4; ++cc) pf[cc] = __builtin_bit_cast(bf16x8, u32x4{0u, 0u, 0u, 0u});
    f32x16 s_nx[2];                                  // raw scores of nx
    {
      f32x16 s0[2];
      scores(std::integral_constant<int, 0>{}, s0);
      const float mb = finish_scores(t_cur, s0, pf);
      probs(s0, mb, t_cur == 0, pf);
      scores(std::integral_constant<int, 1>{}, s_nx);
    }
    wait_bar<0>();                                   // K buffer 0 no longer read
    if (t_nx2 >= 0) issue_k(t_nx2, 0);
    wait_bar<0>();

    // The block of step k (K buffer and V buffer ST = k%2): s_nn = scores of
    // nx2, O += V P of cur, pn = P of nx.  Slot x: score MFMA x (M-tile
    // x%2, k-step x/2), P V MFMA x (k-step x/4, dim tile x%4), exponentials
    // of elements 2x, 2x+1 of nx; K fragments read two slots ahead, V^T
    // fragments one slot ahead.
    auto block = [&](auto ST, f32x16 (&sn)[2], f32x16 (&sx)[2], float mb, bool first,
                     bf16x8 (&pn)[4]) __attribute__((always_inline)) {
      constexpr int st = decltype(ST)::value;
      const lds_char* kb = (const lds_char*)(kbuf[st]);
      const lds_char* vb = (const lds_char*)(vbuf[st]);
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int i = 0; i < 16; ++i) sn[mt][i] = 0.f;
      bf16x8 kf[3], vf[2];
      kf[0] = lds_frag(kb, koff[0]);
      kf[1] = lds_frag(kb, koff[0] + 8192);
      auto vfrag = [&](int x) __attribute__((always_inline)) {
        const int cc = x >> 2, dt = x & 3;
        const u32x2 lo = lds_tr(vb, voa[dt] + cc * 4096);
        const u32x2 hi = lds_tr(vb, vob[dt] + cc * 4096);
        return __builtin_bit_cast(bf16x8, u32x4{lo[0], lo[1], hi[0], hi[1]});
      };
      vf[0] = vfrag(0);
      float ls = 0.f;
#pragma unroll
      for (int x = 0; x < 16; ++x) {
        if (x + 2 < 16) kf[(x + 2) % 3] = lds_frag(kb, koff[(x + 2) >> 1] + ((x + 2) & 1) * 8192);
        if (x + 1 < 16) vf[(x + 1) & 1] = vfrag(x + 1);
        // each MFMA is followed by vector work that does not depend on it,
        // which issues while it executes
        auto expo = [&](int e) __attribute__((always_inline)) {
          const int mt = (2 * x + e) >> 4, i = (2 * x + e) & 15;
          const float ex = __builtin_amdgcn_exp2f(__builtin_fmaf(sx[mt][i], c, -mb));
          sx[mt][i] = ex;
          ls += ex;
          asm volatile("" : "+v"(ls));               // the row sum stays in its slot
        };
        sn[x & 1] = mfma32(kf[x % 3], qf[x >> 1], sn[x & 1]);
        __builtin_amdgcn_sched_barrier(0);
        expo(0);
        __builtin_amdgcn_sched_barrier(0);
        oacc[x & 3] = mfma32(vf[x & 1], pf[x >> 2], oacc[x & 3]);
        __builtin_amdgcn_sched_barrier(0);
        expo(1);
        if ((x & 3) == 3) pn[x >> 2] = pack_kstep(sx[x >> 3], (x >> 2) & 1);
        __builtin_amdgcn_sched_barrier(0);
      }
      lsum += ls;
      if constexpr (GATE) {
        if (first) l0 += gq == 0 ? sx[0][0] : 0.f;   // uniform branch
      }
    };
    auto step = [&](auto ST) __attribute__((always_inline)) {
      constexpr int st = decltype(ST)::value;
      const int t_nx3 = sc.next();
      if (t_nx3 >= 0) issue_k(t_nx3, st ^ 1);
      if (t_nx >= 0) issue_v(t_nx, st ^ 1);
      const float mb = finish_scores(t_nx, s_nx, pf);
      f32x16 s_nn[2];
      bf16x8 pn[4];
      block(ST, s_nn, s_nx, mb, t_nx == 0, pn);
#pragma unroll
      for (int cc = 0; cc < 4; ++cc) pf[cc] = pn[cc];
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) s_nx[mt] = s_nn[mt];
      // This step's loads landed and no read of the buffers they refill next
      // step is in flight.
      wait_bar<0>();
      t_cur = t_nx;
      t_nx = t_nx2;
      t_nx2 = t_nx3;
    };
    while (true) {                                   // t_cur is uniform over the workgroup
      step(std::integral_constant<int, 0>{});
      if (t_cur < 0) break;
      step(std::integral_constant<int, 1>{});
      if (t_cur < 0) break;
    }
  }

  // Epilogue: L_orig = alpha*m + ln l; s = sigma(L_orig - a_h); O = acc * s / l.
  const float lt = xhalf_sum(lsum);
  const float l0t = GATE ? xhalf_sum(l0) : 0.f;
  if (qi >= wq1 || qi < qs) return;
  const bool has_sink = p.sink != nullptr;
  float L_orig, s_val, mul;
  if (lt > 0.f) {
    L_orig = mrun * p.scale + __logf(lt);
    s_val = has_sink ? 1.f / (1.f + __expf(p.sink[h] - L_orig)) : 1.f;
    mul = s_val / lt;
  } else {
    L_orig = -kInf;
    s_val = has_sink ? 0.f : 1.f;
    mul = 0.f;
  }
  uint16_t* dst = O + (static_cast<size_t>(tq + qi) * p.hq + h) * D + 4 * gq;
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      u32x2 pk;
      pk[0] = pack_bf16x2(oacc[dt][4 * u] * mul, oacc[dt][4 * u + 1] * mul);
      pk[1] = pack_bf16x2(oacc[dt][4 * u + 2] * mul, oacc[dt][4 * u + 3] * mul);
      *reinterpret_cast<u32x2*>(dst + dt * 32 + 8 * u) = pk;
    }
  if (gq == 0) {
    const size_t r = static_cast<size_t>(tq + qi) * p.hq + h;
    lse_out[r] = L_orig;
    if (s_out) s_out[r] = s_val;
    if constexpr (GATE) gate_out[r] = lt > 0.f ? (lt - l0t) / lt : 0.f;
  }
}

// Test hook: the same geometry, schedule and classification as fwd_kernel,
// marking (query, key) pairs the forward visits and keeps.  One workgroup of
// 256 threads per forward workgroup; out[b][g][i][j] for sample-local i, j.
__global__ __launch_bounds__(256) void visit_map_kernel(Prefill p, Geo geo, uint8_t* out) {
  __shared__ uint32_t bitmap[BITMAP_LDS_WORDS];
  const WgCoord wc = wg_coord(geo, p.batch, blockIdx.x);
  if (wc.hg != 0) return;                        // the mask does not depend on the head group
  const int t0 = p.cu[wc.b];
  const int L = p.cu[wc.b + 1] - t0;
  const int p0 = wc.pt * geo.P;
  if (p0 >= L) return;
  const int p1 = min(L, p0 + geo.P);
  const int qoff = p.blocks ? q_block_offset(p.cu, wc.b) : 0;
  size_t base = 0;
  for (int b = 0; b < wc.b; ++b) {
    const size_t Lb = p.cu[b + 1] - p.cu[b];
    base += Lb * Lb * p.hkv;
  }
  uint8_t* m = out + base + static_cast<size_t>(wc.g) * L * L;
  Sched sc = make_sched(p, L, qoff, wc.g, p0, p1, bitmap);
  // The wavefronts of the first head of the workgroup: each covers FQW rows.
  for (int kt = sc.next(); kt >= 0; kt = sc.next()) {
    for (int wv = 0; wv < geo.wph; ++wv) {
      const int wq0 = p0 + wv * FQW;
      const int wq1 = min(L, wq0 + FQW);
      const int cls = wave_tile_class(p, sc, p0, wq0, wq1, kt);
      if (cls == 0) continue;
      for (int e = threadIdx.x; e < FQW * BN; e += blockDim.x) {
        const int qi = wq0 + e / BN;
        const int key = kt * BN + e % BN;
        if (qi >= wq1 || key >= L) continue;
        const bool ok = (cls == 1) || key_visible(qi, key, p.n_sink, p.window);
        if (ok) m[static_cast<size_t>(qi) * L + key] = 1;
      }
    }
  }
}

}  // namespace fwd128

bool fwd_mfma_supported(const Prefill& p) {
  if (p.dtype != SINK_ATTN_BF16 || p.d != qm::D) return false;
  if (p.blocks != nullptr && p.max_seqlen > qm::MAX_BITMAP_WORDS * 32 * qm::BN) return false;
  return true;
}

hipError_t launch_fwd_mfma(const Prefill& p, const void* q, const void* k, const void* v, void* o,
                           float* lse, float* s, float* gate0, hipStream_t st) {
  if (p.total == 0 || p.batch == 0) return hipSuccess;
  const qm::Geo geo = qm::make_geo(p, fwd128::FNW, fwd128::FQW);
  const long long grid = static_cast<long long>(geo.nptiles) * p.batch * geo.Z;
  if (grid <= 0) return hipSuccess;
  auto kern = gate0 ? fwd128::fwd_kernel<true, false> : fwd128::fwd_kernel<false, false>;
  hipLaunchKernelGGL(kern, dim3(static_cast<unsigned>(grid)), dim3(64 * fwd128::FNW), 0, st, p, geo,
                     static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                     static_cast<const uint16_t*>(v), static_cast<uint16_t*>(o), lse, s, gate0, CacheKv{});
  return hipGetLastError();
}

hipError_t launch_fwd_mfma_cache(const Prefill& p, const CacheKv& ckv, const void* q, void* o, float* lse,
                                 float* s, hipStream_t st) {
  if (p.total == 0 || p.batch == 0) return hipSuccess;
  const qm::Geo geo = qm::make_geo(p, fwd128::FNW, fwd128::FQW);
  const long long grid = static_cast<long long>(geo.nptiles) * p.batch * geo.Z;
  if (grid <= 0) return hipSuccess;
  hipLaunchKernelGGL((fwd128::fwd_kernel<false, true>), dim3(static_cast<unsigned>(grid)), dim3(64 * fwd128::FNW),
                     0, st, p, geo, static_cast<const uint16_t*>(q), nullptr, nullptr, static_cast<uint16_t*>(o),
                     lse, s, nullptr, ckv);
  return hipGetLastError();
}

hipError_t launch_visit_map(const Prefill& p, uint8_t* out, hipStream_t st) {
  if (p.total == 0 || p.batch == 0) return hipSuccess;
  const qm::Geo geo = qm::make_geo(p, fwd128::FNW, fwd128::FQW);
  const long long grid = static_cast<long long>(geo.nptiles) * p.batch * geo.Z;
  if (grid <= 0) return hipSuccess;
  hipLaunchKernelGGL(fwd128::visit_map_kernel, dim3(static_cast<unsigned>(grid)), dim3(256), 0, st,
                     p, geo, out);
  return hipGetLastError();
}

}  // namespace sa
