// Decode against a rolling KV cache: split-KV on matrix cores, then a merge of
// the splits by their log-sum-exp with the sink epilogue.
//
// The cache of each sequence is an unordered set of slots (a ring buffer keeps
// the first tokens and the recent window in any slot order: "Attention Sink"
// (lijianxiong.space), H2O circular cache; StreamingLLM's fixed first-token
// segment plus sliding window: "What is Attention Sink? ... StreamingLLM"
// (model.playoffer.cn)).  No mask applies beyond cache_seqlens.  The sink is
// the output scale s = sigma(L_orig - a_h) ("Attention Sink, Learnable Sink
// and dsink" s4), applied once after the merge.
//
// Split kernel (bf16, head_dim 128), one workgroup per (sequence b, KV head g,
// head group, split):
//   * 2 wavefronts stream disjoint 32-slot chunks of the split.  The query
//     heads of the group (up to 16) form the N side of
//     v_mfma_f32_16x16x32_bf16; S^T = K Q^T puts one head per lane column.
//   * K goes from HBM straight into the MFMA A-operand registers: lane
//     (slot, quarter) reads 16 bytes per k-step and the four quarters of a
//     slot read one contiguous 64-byte piece of its row.  The next chunk's K
//     is in flight while the current chunk computes.
//   * V is staged through a per-wavefront LDS buffer (rows XOR-swizzled in
//     16-byte chunks) and read back transposed with ds_read_b64_tr_b16, which
//     gives each lane one dim at 4 slots: the A operand of O^T += V^T P^T.
//   * The wavefronts merge (m, l, acc) in LDS; the workgroup writes one
//     partial per (b, head, split) to the workspace, or, with a single
//     split, applies the sink epilogue itself and writes O, LSE and s.
// Merge kernel (more than one split): M = max_k m_k, l = sum_k e^{m_k - M}
// l_k, L_orig = M + ln l, O = s * sum_k e^{m_k - M} acc_k / l.
//
// 8-bit cache (instantiation Q8): the first n_sink tokens are bfloat16 rows
// of one array and the ring of recent tokens e4m3 rows of another, with a
// float32 scale per (slot, KV head).  Slots are numbered sinks first (padded
// to a whole 32-slot chunk) then ring slots, so every chunk is all-bf16 or
// all-e4m3 and the choice is uniform per wavefront.  e4m3 codes convert to
// bfloat16 exactly (v_cvt_scalef32_pk_bf16_fp8 with scale 1); the K scale of
// a slot multiplies its scores, the V scale its probability in P V (not in
// the row sum l), so no row is rescaled element by element.
#include "common.cuh"

namespace sa {

hipError_t launch_decode_generic(const Decode& p, const void* q, const void* kc, const void* vc,
                                 void* o, float* lse, float* s, hipStream_t st);

namespace dec128 {

constexpr int D = 128;
constexpr int CH = 32;            // slots per chunk
// Wavefronts per workgroup.  Two (4 workgroups per CU at 2 wavefronts per
// SIMD) rather than four: 128 sequences x 8 KV heads then fill the chip in
// one round of workgroups instead of two, each wavefront streaming twice the
// chunks (measured, 128 x 4096 slots, Hq 64, Hkv 8: 8-bit cache 0.2245 ->
// 0.2163 ms, bf16 0.3655 -> 0.3618 ms).
constexpr int NW = 2;
constexpr int NT = 64 * NW;       // threads per workgroup
constexpr int HN = 16;            // query heads per workgroup (N of the MFMA)
constexpr int VBUF = CH * D;      // bf16 elements of one V chunk buffer (8 KB)
constexpr float kRescaleLog2 = 8.f;

typedef short i16x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// 16-byte chunk swizzle of a V row: spreads the 4 slots x 4 chunks that one
// transposed read touches over distinct banks.
__device__ __forceinline__ int vswz(int row) {
  const int r = row & 15;
  return ((r & 3) << 2) | ((r >> 2) & 3);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2 v = {static_cast<__bf16>(lo), static_cast<__bf16>(hi)};
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ i16x4 ds_read_tr(const uint16_t* lds_ptr) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) i16x4*)(const_cast<uint16_t*>(lds_ptr)));
}

// Two e4m3 codes (the 16-bit half `hi` of w) as two bfloat16, exactly.
__device__ __forceinline__ uint32_t fp8x2_to_bf16x2(uint32_t w, bool hi) {
  return __builtin_bit_cast(uint32_t, hi ? __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.f, true)
                                         : __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.f, false));
}
__device__ __forceinline__ u32x4 fp8x8_to_bf16x8(uint32_t w0, uint32_t w1) {
  return u32x4{fp8x2_to_bf16x2(w0, false), fp8x2_to_bf16x2(w0, true), fp8x2_to_bf16x2(w1, false),
               fp8x2_to_bf16x2(w1, true)};
}

// 16-byte cache load.  The bfloat16 cache streams through once per call:
// non-temporal loads keep it from displacing other data in the caches and
// measured faster; for the 8-bit ring, whose 128-byte rows each lane group
// reads in pieces, they measured slower, so Q8 keeps ordinary loads.
template <bool NT>
__device__ __forceinline__ u32x4 load16(const void* p) {
  if constexpr (NT) return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  else return *reinterpret_cast<const u32x4*>(p);
}

// First of the 8 dims that quarter gq holds at k-step ks.  bf16 cache: dims
// ks*32 + gq*8, so the four quarters of a slot read 64 contiguous bytes per
// k-step.  8-bit cache: (ks/2)*64 + gq*16 + (ks%2)*8, so one 16-byte load
// brings two k-steps of e4m3 codes and the four quarters read 64 contiguous
// bytes of the row per load.
template <bool Q8>
__device__ __forceinline__ int kdim(int ks, int gq) {
  return Q8 ? (ks >> 1) * 64 + gq * 16 + (ks & 1) * 8 : ks * 32 + gq * 8;
}

template <bool Q8>
__global__ __launch_bounds__(NT, 2) void split_kernel(Decode p, int nhg,
                                                       const uint16_t* __restrict__ Q,
                                                       const uint16_t* __restrict__ KC,
                                                       const uint16_t* __restrict__ VC,
                                                       float* __restrict__ ws,
                                                       uint16_t* __restrict__ O,
                                                       float* __restrict__ lse,
                                                       float* __restrict__ s_out, KvCache qc) {
  // Per-wavefront double-buffered V chunks; after the loop the same memory
  // holds the wavefronts' partial results for the merge.
  __shared__ __attribute__((aligned(16))) uint16_t vbuf[NW][2][VBUF];
  static_assert(sizeof(float) * NW * HN * (D + 2) <= sizeof(uint16_t) * NW * 2 * VBUF, "merge fits");
  float (*mbuf)[HN][D + 2] = reinterpret_cast<float (*)[HN][D + 2]>(&vbuf[0][0][0]);

  // grid: x = split (fastest), y = KV head * head groups, z = sequence
  const int split = blockIdx.x;
  const int g = blockIdx.y / nhg;
  const int hg = blockIdx.y % nhg;
  const int b = blockIdx.z;
  const int G = p.hq / p.hkv;
  const int h0 = g * G + hg * HN;                    // first query head of the group
  const int nh = min(HN, G - hg * HN);               // heads in this workgroup
  int n, per;
  int ns = 0, ns_pad = 0;                            // Q8: valid sinks, sink chunks' slots
  if constexpr (!Q8) {
    n = p.cache_seqlens ? min(p.cache_seqlens[b], p.slots) : p.slots;
    per = (p.slots + p.splits - 1) / p.splits;
  } else {
    const int tokens = p.cache_seqlens[b];           // appended so far, the current one included
    ns = min(tokens, qc.n_sink);
    const int nw = min(max(tokens - qc.n_sink, 0), qc.window);
    ns_pad = (ns + CH - 1) / CH * CH;
    n = ns_pad + nw;
    const int span = (qc.n_sink + CH - 1) / CH * CH + qc.window;   // the same for every sequence
    per = ((span + CH - 1) / CH + p.splits - 1) / p.splits * CH;   // whole chunks per split
  }
  const int s0 = split * per;
  const int s1 = min(n, s0 + per);

  const int tid = threadIdx.x;
  const int w = tid >> 6;
  const int lane = tid & 63;
  const int l16 = lane & 15;
  const int gq = lane >> 4;

  // Q^T as B operand: lane (head l16, quarter gq) holds at k-step ks the 8
  // dims kdim(ks, gq) (K uses the same order, so the sum over k-steps is the
  // full dot product whatever the order).
  bf16x8 qf[4];
  {
    const bool ok = l16 < nh;
    const uint16_t* src = Q + (static_cast<size_t>(b) * p.hq + h0 + (ok ? l16 : 0)) * D;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
      qf[ks] = ok ? __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(src + kdim<Q8>(ks, gq)))
                  : __builtin_bit_cast(bf16x8, u32x4{0u, 0u, 0u, 0u});
  }

  const size_t row_stride = static_cast<size_t>(p.hkv) * D;
  const int kv_slots = Q8 ? qc.n_sink : p.slots;     // rows per sequence of KC / VC
  const uint16_t* Kb = KC + (static_cast<size_t>(b) * kv_slots * p.hkv + g) * D;
  const uint16_t* Vb = VC + (static_cast<size_t>(b) * kv_slots * p.hkv + g) * D;
  // Q8 ring rows (bytes) and scales of this (sequence, KV head).
  const uint8_t* Kw = Q8 ? qc.win_k + (static_cast<size_t>(b) * qc.window * p.hkv + g) * D : nullptr;
  const uint8_t* Vw = Q8 ? qc.win_v + (static_cast<size_t>(b) * qc.window * p.hkv + g) * D : nullptr;
  const float* Ksc = Q8 ? qc.win_k_scale + (static_cast<size_t>(b) * p.hkv + g) * qc.window : nullptr;
  const float* Vsc = Q8 ? qc.win_v_scale + (static_cast<size_t>(b) * p.hkv + g) * qc.window : nullptr;
  const float c = p.scale * kLog2e;
  const float thr = kRescaleLog2 / c;

  f32x4 oacc[8];
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) oacc[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  float mrun = -kInf, lpart = 0.f;

  // Chunks of this wavefront: start at s0 + 32*(w + 4*i).
  const int nchunks_total = (s1 > s0) ? (s1 - s0 + CH - 1) / CH : 0;
  const int my_first = w;
  u32x4 kf[2][4], kn[2][4];     // current / next chunk K fragments [mt][ks]
  u32x4 vr[8];                  // next chunk V rows, 8 x 16 B per lane
  // Q8: whether the current / next chunk is ring (e4m3: K and V hold the raw
  // codes in words 0-1 until converted) and its slots' K / V scales.
  bool cur_win = false, nxt_win = false;
  float ksc[8], vsc[8], ksn[8], vsn[8];
  const int ring_last = Q8 ? max(qc.window - 1, 0) : 0;
  const int sink_last = Q8 ? max(ns - 1, 0) : 0;
  const bool sc_vec = Q8 && (qc.window & 3) == 0;   // scale rows in whole 16-byte groups

  auto load_k = [&](int cs, u32x4 (&dst)[2][4]) {
    if constexpr (Q8) {
      if (cs >= ns_pad) {                            // uniform: a ring chunk
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) {
          const int r = min(cs - ns_pad + mt * 16 + l16, ring_last);
          const uint8_t* src = Kw + static_cast<size_t>(r) * row_stride + gq * 16;
#pragma unroll
          for (int j = 0; j < 2; ++j) {              // k-steps 2j, 2j+1
            const u32x4 w = *reinterpret_cast<const u32x4*>(src + j * 64);
            dst[mt][2 * j] = u32x4{w[0], w[1], 0u, 0u};
            dst[mt][2 * j + 1] = u32x4{w[2], w[3], 0u, 0u};
          }
        }
        if (sc_vec) {
          // 4 consecutive slots per load; a start past the ring (only slots
          // that the mask drops) reads the ring's last 4 scales instead.
#pragma unroll
          for (int mt = 0; mt < 2; ++mt) {
            const int r = min(cs - ns_pad + 16 * mt + 4 * gq, qc.window - 4);
            const f32x4 a = *reinterpret_cast<const f32x4*>(Ksc + r);
            const f32x4 bb = *reinterpret_cast<const f32x4*>(Vsc + r);
#pragma unroll
            for (int i = 0; i < 4; ++i) { ksn[mt * 4 + i] = a[i]; vsn[mt * 4 + i] = bb[i]; }
          }
        } else {
#pragma unroll
          for (int mt = 0; mt < 2; ++mt)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const int r = min(cs - ns_pad + 16 * mt + 4 * gq + i, ring_last);
              ksn[mt * 4 + i] = Ksc[r];
              vsn[mt * 4 + i] = Vsc[r];
            }
        }
        return;
      }
    }
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      int slot = cs + mt * 16 + l16;
      if constexpr (Q8) slot = min(slot, sink_last);
      else slot = slot < p.slots ? slot : p.slots - 1;
      const uint16_t* src = Kb + static_cast<size_t>(slot) * row_stride;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) dst[mt][ks] = load16<!Q8>(src + kdim<Q8>(ks, gq));
    }
  };
  auto load_v = [&](int cs) {
    if constexpr (Q8) {
      if (cs >= ns_pad) {                            // 8 lanes per 128-byte row
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = min(cs - ns_pad + (lane >> 3) + 8 * i, ring_last);
          vr[i] = *reinterpret_cast<const u32x4*>(Vw + static_cast<size_t>(r) * row_stride + (lane & 7) * 16);
        }
        return;
      }
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      int slot = cs + (lane >> 4) + 4 * i;
      if constexpr (Q8) slot = min(slot, sink_last);
      else slot = slot < p.slots ? slot : p.slots - 1;
      vr[i] = load16<!Q8>(Vb + static_cast<size_t>(slot) * row_stride + l16 * 8);
    }
  };
  auto store_v = [&](uint16_t* buf, bool win) {
    if constexpr (Q8) {
      if (win) {                                     // e4m3 codes -> bf16, exactly
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int row = (lane >> 3) + 8 * i;
          const int c0 = (lane & 7) * 2;
          *reinterpret_cast<u32x4*>(buf + row * D + (c0 ^ vswz(row)) * 8) = fp8x8_to_bf16x8(vr[i][0], vr[i][1]);
          *reinterpret_cast<u32x4*>(buf + row * D + ((c0 + 1) ^ vswz(row)) * 8) =
              fp8x8_to_bf16x8(vr[i][2], vr[i][3]);
        }
        return;
      }
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int row = (lane >> 4) + 4 * i;
      const int pc = l16 ^ vswz(row);
      *reinterpret_cast<u32x4*>(buf + row * D + pc * 8) = vr[i];
    }
  };

  int ci = my_first;
  int cur = 0;
  if (ci < nchunks_total) {
    const int cs = s0 + CH * ci;
    load_k(cs, kf);
    load_v(cs);
    if constexpr (Q8) {
      cur_win = cs >= ns_pad;
#pragma unroll
      for (int e = 0; e < 8; ++e) { ksc[e] = ksn[e]; vsc[e] = vsn[e]; }
    }
    store_v(vbuf[w][0], cur_win);
  }
  while (ci < nchunks_total) {
    const int cs = s0 + CH * ci;
    const int cn = ci + NW;
    const bool has_next = cn < nchunks_total;
    if (has_next) {
      load_k(s0 + CH * cn, kn);
      load_v(s0 + CH * cn);
      if constexpr (Q8) nxt_win = s0 + CH * cn >= ns_pad;
    }
    if constexpr (Q8) {
      if (cur_win) {                                 // e4m3 codes -> bf16, exactly
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
          for (int ks = 0; ks < 4; ++ks) kf[mt][ks] = fp8x8_to_bf16x8(kf[mt][ks][0], kf[mt][ks][1]);
      }
    }
    // S^T = K Q^T for 32 slots (2 M-tiles of 16) x 16 heads.
    f32x4 sacc[2];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      sacc[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
        sacc[mt] = mfma16(__builtin_bit_cast(bf16x8, kf[mt][ks]), qf[ks], sacc[mt]);
    }
    if constexpr (Q8) {
      if (cur_win) {                                 // the slots' K scales
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
          for (int i = 0; i < 4; ++i) sacc[mt][i] *= ksc[mt * 4 + i];
      }
    }
    // Mask slots past the split or the valid length.  Element i of lane
    // (l16, gq) in M-tile mt is slot cs + 16mt + 4gq + i, head l16.  Q8: a
    // sink chunk's slots past the valid sinks too.
    const int lim = (Q8 && cs < ns_pad) ? min(s1, ns) : s1;
    if (cs + CH > lim) {
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (cs + 16 * mt + 4 * gq + i >= lim) {
            sacc[mt][i] = -kInf;
            if constexpr (Q8) vsc[mt * 4 + i] = 0.f;
          }
      // Unused slots may hold anything (NaN included) and 0 * NaN is NaN in
      // P V: zero their V rows in this wavefront's buffer (LDS operations of
      // one wavefront complete in order, so the reads below see the zeros).
      uint16_t* vz = vbuf[w][cur];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int row = (lane >> 4) + 4 * i;
        if (cs + row >= lim)
          *reinterpret_cast<u32x4*>(vz + row * D + (l16 ^ vswz(row)) * 8) = u32x4{0u, 0u, 0u, 0u};
      }
    }
    float mx = -kInf;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) mx = fmaxf(mx, sacc[mt][i]);
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    if (__ballot(mx > mrun + thr) != 0) {
      const float mnew = fmaxf(mrun, mx);
      const float f = (mrun == -kInf) ? 0.f : __builtin_amdgcn_exp2f((mrun - mnew) * c);
#pragma unroll
      for (int dt = 0; dt < 8; ++dt)
#pragma unroll
        for (int i = 0; i < 4; ++i) oacc[dt][i] *= f;
      lpart *= f;
      mrun = mnew;
    }
    const float mb = (mrun == -kInf) ? 0.f : mrun * c;
    float pv[8];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float e = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[mt][i], c, -mb));
        pv[mt * 4 + i] = e;
        lpart += e;
      }
    if constexpr (Q8) {
      if (cur_win) {                                 // the slots' V scales, in P V only
#pragma unroll
        for (int e = 0; e < 8; ++e) pv[e] *= vsc[e];
      }
    }
    // B operand: logical k slot t of quarter gq = slot 16*(t/4) + 4gq + t%4.
    const bf16x8 pf = __builtin_bit_cast(
        bf16x8, u32x4{pack_bf16x2(pv[0], pv[1]), pack_bf16x2(pv[2], pv[3]),
                      pack_bf16x2(pv[4], pv[5]), pack_bf16x2(pv[6], pv[7])});
    // O^T += V^T P^T: 8 dim tiles of 16.  Transposed reads: lane s = 4r + q of
    // quarter gq reads slot 4gq + r (and 16 + 4gq + r), dims dt*16 + 4q..+4.
    const uint16_t* vb = vbuf[w][cur];
    const int r = l16 >> 2, q4 = l16 & 3;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
      const int lc = dt * 2 + (q4 >> 1);
      const int off = (q4 & 1) * 4;
      const int r0 = 4 * gq + r, r1 = 16 + 4 * gq + r;
      const i16x4 a0 = ds_read_tr(vb + r0 * D + ((lc ^ vswz(r0)) * 8) + off);
      const i16x4 a1 = ds_read_tr(vb + r1 * D + ((lc ^ vswz(r1)) * 8) + off);
      const bf16x8 af = __builtin_bit_cast(
          bf16x8, u32x4{__builtin_bit_cast(u32x2, a0)[0], __builtin_bit_cast(u32x2, a0)[1],
                        __builtin_bit_cast(u32x2, a1)[0], __builtin_bit_cast(u32x2, a1)[1]});
      oacc[dt] = mfma16(af, pf, oacc[dt]);
    }
    if (has_next) {
      store_v(vbuf[w][cur ^ 1], nxt_win);
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) kf[mt][ks] = kn[mt][ks];
      if constexpr (Q8) {
        cur_win = nxt_win;
#pragma unroll
        for (int e = 0; e < 8; ++e) { ksc[e] = ksn[e]; vsc[e] = vsn[e]; }
      }
    }
    cur ^= 1;
    ci = cn;
  }

  // Merge the wavefronts.  Per head: m (same on the 4 quarters), l summed
  // over quarters, acc dims dt*16 + 4gq + i.
  lpart += __shfl_xor(lpart, 16);
  lpart += __shfl_xor(lpart, 32);
  __syncthreads();                 // every wavefront is done with its V buffers
#pragma unroll
  for (int dt = 0; dt < 8; ++dt)
#pragma unroll
    for (int i = 0; i < 4; ++i) mbuf[w][l16][dt * 16 + 4 * gq + i] = oacc[dt][i];
  if (gq == 0) {
    mbuf[w][l16][D] = mrun;
    mbuf[w][l16][D + 1] = lpart;
  }
  __syncthreads();
  // 16 threads per head, 8 dims each; NT / 16 heads per pass
  for (int hh = tid >> 4; hh < nh; hh += NT / 16) {
    const int d0 = (tid & 15) * 8;
    {
      float M = -kInf;
#pragma unroll
      for (int ww = 0; ww < NW; ++ww) M = fmaxf(M, mbuf[ww][hh][D]);
      float wgt[NW];
      float lt = 0.f;
#pragma unroll
      for (int ww = 0; ww < NW; ++ww) {
        const float mw = mbuf[ww][hh][D];
        wgt[ww] = (mw == -kInf) ? 0.f : __builtin_amdgcn_exp2f((mw - M) * c);
        lt += wgt[ww] * mbuf[ww][hh][D + 1];
      }
      float a[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        a[e] = 0.f;
#pragma unroll
        for (int ww = 0; ww < NW; ++ww) a[e] += wgt[ww] * mbuf[ww][hh][d0 + e];
      }
      const float Mn = (M == -kInf) ? -kInf : M * p.scale;   // natural-log units
      if (p.splits == 1) {
        // One split: this is the whole cache, so the sink epilogue of the
        // merge runs here and no partial goes through the workspace.
        const size_t r = static_cast<size_t>(b) * p.hq + h0 + hh;
        float L_orig, s_val, mul;
        if (lt > 0.f) {
          L_orig = Mn + __logf(lt);
          s_val = p.sink ? 1.f / (1.f + __expf(p.sink[h0 + hh] - L_orig)) : 1.f;
          mul = s_val / lt;
        } else {
          L_orig = -kInf;
          s_val = p.sink ? 0.f : 1.f;
          mul = 0.f;
        }
        u32x4 pk;
#pragma unroll
        for (int e = 0; e < 4; ++e) pk[e] = pack_bf16x2(a[2 * e] * mul, a[2 * e + 1] * mul);
        *reinterpret_cast<u32x4*>(O + r * D + d0) = pk;
        if ((tid & 15) == 0) {
          lse[r] = L_orig;
          if (s_out) s_out[r] = s_val;
        }
      } else {
        float* dst = ws + ((static_cast<size_t>(b) * p.hq + h0 + hh) * p.splits + split) * (D + 2);
#pragma unroll
        for (int e = 0; e < 8; ++e) dst[d0 + e] = a[e];
        if ((tid & 15) == 0) {
          dst[D] = Mn;
          dst[D + 1] = lt;
        }
      }
    }
  }
}

}  // namespace dec128

// Merge of the splits (any head_dim): one workgroup per (sequence, head).
template <typename T>
__global__ __launch_bounds__(128) void decode_merge_kernel(Decode p, const float* __restrict__ ws,
                                                           void* o, float* lse, float* s_out) {
  const int b = blockIdx.x / p.hq;
  const int h = blockIdx.x % p.hq;
  const int D = p.d;
  const float* base = ws + (static_cast<size_t>(b) * p.hq + h) * p.splits * (D + 2);
  float M = -kInf;
  for (int k = 0; k < p.splits; ++k) M = fmaxf(M, base[k * (D + 2) + D]);
  float l = 0.f;
  for (int k = 0; k < p.splits; ++k) {
    const float mk = base[k * (D + 2) + D];
    if (mk != -kInf) l += __expf(mk - M) * base[k * (D + 2) + D + 1];
  }
  const bool has_sink = p.sink != nullptr;
  float L_orig, s_val, mul;
  if (l > 0.f) {
    L_orig = M + __logf(l);
    s_val = has_sink ? 1.f / (1.f + __expf(p.sink[h] - L_orig)) : 1.f;
    mul = s_val / l;
  } else {
    L_orig = -kInf;
    s_val = has_sink ? 0.f : 1.f;
    mul = 0.f;
  }
  for (int d = threadIdx.x; d < D; d += blockDim.x) {
    float a = 0.f;
    for (int k = 0; k < p.splits; ++k) {
      const float mk = base[k * (D + 2) + D];
      if (mk != -kInf) a += __expf(mk - M) * base[k * (D + 2) + d];
    }
    Elem<T>::store(o, (static_cast<size_t>(b) * p.hq + h) * D + d, a * mul);
  }
  if (threadIdx.x == 0) {
    lse[static_cast<size_t>(b) * p.hq + h] = L_orig;
    if (s_out) s_out[static_cast<size_t>(b) * p.hq + h] = s_val;
  }
}

bool decode_mfma_supported(const Decode& p) {
  return p.dtype == SINK_ATTN_BF16 && p.d == dec128::D;
}

int decode_auto_splits(const Decode& p) {
  // One split (no merge pass) when the (sequence, KV head) units alone fill
  // every CU's 8 wavefront slots (2 per SIMD) once; otherwise enough splits
  // for about 4 rounds of workgroups, but no split shorter than 4 chunks per
  // wavefront.  Measured on 128 x 4096 slots, 8 KV heads (1024 units), with 4
  // wavefronts per workgroup: 1 split 0.391 ms, 2: 0.410, 4: 0.420, 16:
  // 0.436; with 2 (the 8-bit cache): 1 split 0.225 ms, 2: 0.248, 4: 0.284.
  // The thresholds count wavefronts, so they follow NW.
  const int G = p.hq / p.hkv;
  const long long units = static_cast<long long>(p.batch) * p.hkv * ((G + dec128::HN - 1) / dec128::HN);
  if (units <= 0) return 1;
  if (units * dec128::NW >= 2048) return 1;
  long long want = (8192 / dec128::NW + units - 1) / units;
  const long long max_by_len = p.slots / (dec128::CH * dec128::NW * 4);
  if (want > max_by_len) want = max_by_len;
  if (want < 1) want = 1;
  if (want > 64) want = 64;
  return static_cast<int>(want);
}

hipError_t launch_decode(const Decode& p, const void* q, const void* kc, const void* vc, void* o,
                         float* lse, float* s, float* ws, hipStream_t st) {
  if (!decode_mfma_supported(p)) return launch_decode_generic(p, q, kc, vc, o, lse, s, st);
  const int G = p.hq / p.hkv;
  const int nhg = (G + dec128::HN - 1) / dec128::HN;
  dim3 grid(p.splits, p.hkv * nhg, p.batch);
  hipLaunchKernelGGL(dec128::split_kernel<false>, grid, dim3(dec128::NT), 0, st, p, nhg,
                     static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(kc),
                     static_cast<const uint16_t*>(vc), ws, static_cast<uint16_t*>(o), lse, s,
                     KvCache{});
  if (p.splits > 1)
    hipLaunchKernelGGL(decode_merge_kernel<uint16_t>, dim3(p.batch * p.hq), dim3(128), 0, st, p, ws,
                       o, lse, s);
  return hipGetLastError();
}

int kvcache_q8_auto_splits(const Decode& p, const KvCache& c) {
  Decode d = p;
  d.slots = (c.n_sink + dec128::CH - 1) / dec128::CH * dec128::CH + c.window;
  return decode_auto_splits(d);
}

hipError_t launch_kvcache_decode_q8(const Decode& p, const KvCache& c, const void* q, void* o,
                                    float* lse, float* s, float* ws, hipStream_t st) {
  const int G = p.hq / p.hkv;
  const int nhg = (G + dec128::HN - 1) / dec128::HN;
  dim3 grid(p.splits, p.hkv * nhg, p.batch);
  hipLaunchKernelGGL(dec128::split_kernel<true>, grid, dim3(dec128::NT), 0, st, p, nhg,
                     static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(c.sink_k),
                     static_cast<const uint16_t*>(c.sink_v), ws, static_cast<uint16_t*>(o), lse, s, c);
  if (p.splits > 1)
    hipLaunchKernelGGL(decode_merge_kernel<uint16_t>, dim3(p.batch * p.hq), dim3(128), 0, st, p, ws,
                       o, lse, s);
  return hipGetLastError();
}

}  // namespace sa
