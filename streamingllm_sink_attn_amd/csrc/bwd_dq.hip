// dQ on gfx950 matrix cores (bfloat16, head_dim 128), query-major.
//
// dQ_i = alpha sum_j dS_ij K_j with dS = P (dO V^T - Delta) and P rebuilt
// from L_new, which already holds the sink's e^{a_h} ("Attention Sink,
// Learnable Sink and dsink" s8).  Computing dQ query-major, next to the
// key-major dK/dV pass, replaces per-tile float32 atomics by one
// deterministic store per element.
//
// Layout mirrors the forward: a wavefront owns 32 query rows of one head and
// walks the same key-tile schedule.  S^T = K Q^T and dP^T = V dO^T come out
// with one query per lane column, so L_new and Delta are per-lane scalars;
// dS^T in bf16 is directly the B operand of dQ^T += K^T dS^T, whose K^T
// operand comes from the staged K tile through ds_read_b64_tr_b16.
#include <type_traits>

#include "qmajor.cuh"

namespace sa {
namespace dq128 {

using namespace qm;

constexpr int NWQ = 8;      // wavefronts per workgroup (2 per SIMD)
constexpr int QWQ = 32;     // query rows per wavefront

__global__ __launch_bounds__(512, 1) void dq_kernel(Prefill p, Geo geo,
                                                    const uint16_t* __restrict__ Q,
                                                    const uint16_t* __restrict__ K,
                                                    const uint16_t* __restrict__ V,
                                                    const uint16_t* __restrict__ dO, BwdWork w,
                                                    uint16_t* __restrict__ dQ) {
  __shared__ __attribute__((aligned(16))) uint16_t kv[2][2][TILE];   // [stage][K, V]
  __shared__ uint32_t bitmap[BITMAP_LDS_WORDS];

  const WgCoord wc = wg_coord(geo, p.batch, blockIdx.x);
  const int t0 = p.cu[wc.b];
  const int L = p.cu[wc.b + 1] - t0;
  const int p0 = wc.pt * geo.P;
  if (p0 >= L) return;
  const int p1 = min(L, p0 + geo.P);

  const int tid = threadIdx.x;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);   // scalar: tile decisions branch uniformly
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int gq = lane >> 5;
  const int G = p.hq / p.hkv;
  const int g = wc.g;
  const int h = g * G + wc.hg * geo.hw + wv / geo.wph;
  const int wq0 = p0 + (wv % geo.wph) * QWQ;
  const int wq1 = min(L, wq0 + QWQ);
  const int qoff = p.blocks ? q_block_offset(p.cu, wc.b) : 0;

  // Q^T and dO^T as B operands (lane: query l32, dims gq*64 + ks*8), and the
  // per-query L_new, Delta (rows past the sample: P = 0 through L_new = +inf).
  const int qi = wq0 + l32;
  bf16x8 qf[8], dof[8];
  float Lq = kInf, Dq = 0.f;
  if (qi < L) {
    const size_t row = static_cast<size_t>(t0 + qi) * p.hq + h;
    const uint16_t* qs = Q + row * D + gq * 64;
    const uint16_t* ds = dO + row * D + gq * 64;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      qf[ks] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(qs + ks * 8));
      dof[ks] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(ds + ks * 8));
    }
    Lq = w.lnew[row];
    Dq = w.delta[row];
  } else {
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      qf[ks] = __builtin_bit_cast(bf16x8, u32x4{0u, 0u, 0u, 0u});
      dof[ks] = qf[ks];
    }
  }
  // Loaded before any tile DMA is in flight (the compiler counts only its own
  // loads): consuming them here makes it wait for them up front.
  asm volatile("" ::"v"(qf[0]), "v"(qf[1]), "v"(qf[2]), "v"(qf[3]), "v"(qf[4]), "v"(qf[5]),
               "v"(qf[6]), "v"(qf[7]));
  asm volatile("" ::"v"(dof[0]), "v"(dof[1]), "v"(dof[2]), "v"(dof[3]), "v"(dof[4]), "v"(dof[5]),
               "v"(dof[6]), "v"(dof[7]), "v"(Lq), "v"(Dq));
  const float lb = Lq;                               // L_new in log2 units

  Sched sc = make_sched(p, L, qoff, g, p0, p1, bitmap);

  const float c = p.scale * kLog2e;
  f32x16 dqacc[4];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int i = 0; i < 16; ++i) dqacc[dt][i] = 0.f;

  const int kvs = p.hkv * D;
  const uint16_t* Kg = K + static_cast<size_t>(t0) * kvs + g * D;
  const uint16_t* Vg = V + static_cast<size_t>(t0) * kvs + g * D;
  DmaTiles<NWQ> ld;
  ld.init(wv, lane, kvs);
  const uint32_t kv0 = lds_address(&kv[0][0][0]);
  auto issue = [&](int kt, int st) {
    const int k0 = kt * BN;
    ld.load(Kg + static_cast<size_t>(k0) * kvs, L - k0, kv0 + static_cast<uint32_t>((2 * st) * TILE * 2));
    ld.load(Vg + static_cast<size_t>(k0) * kvs, L - k0, kv0 + static_cast<uint32_t>((2 * st + 1) * TILE * 2));
  };

  // Per-lane LDS byte offsets of a staged tile, each family one base and an
  // XOR (the swizzle only permutes the bits the index moves), so the loop
  // holds three registers instead of twelve offsets: row fragment (row
  // 32mt + l32, logical chunk gq*8 + ks) at (rf ^ (ks << 4)) + 8192 mt;
  // transposed pair (rows 16cc + ra and +8, dims dt*32 + d) at
  // (ta | tb) ^ (dt << 6), plus 4096 cc.
  const int rf = l32 * 256 + (((gq * 8) ^ swz16(l32)) << 4);
  int ta, tb;
  {
    const int l16 = lane & 15, grp = lane >> 4;
    const int r = l16 >> 2, q4 = l16 & 3;
    const int c0 = 2 * (grp & 1) + (q4 >> 1), off = 8 * (q4 & 1);
    const int ra = 4 * (grp >> 1) + r;
    ta = ra * 256 + ((c0 ^ swz16(ra)) << 4) + off;
    tb = (ra + 8) * 256 + ((c0 ^ swz16(ra + 8)) << 4) + off;
  }
  typedef __attribute__((address_space(3))) char lds_char;
  auto frag = [&](const lds_char* t, int o) __attribute__((always_inline)) {
    return __builtin_bit_cast(bf16x8, *reinterpret_cast<const __attribute__((address_space(3))) u32x4*>(t + o));
  };
  auto tr_pair = [&](const lds_char* t, int oa, int ob) __attribute__((always_inline)) {
    const u32x2 a = __builtin_bit_cast(
        u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)(t + oa)));
    const u32x2 b = __builtin_bit_cast(
        u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)(t + ob)));
    return __builtin_bit_cast(bf16x8, u32x4{a[0], a[1], b[0], b[1]});
  };

  int kt = sc.next();
  if (kt >= 0) issue(kt, 0);
  wait_bar<0>();
  int stage = 0;
  while (kt >= 0) {
    const int kt_next = sc.next();
    if (kt_next >= 0) issue(kt_next, stage ^ 1);

    const int cls = wave_tile_class(p, sc, p0, wq0, wq1, kt);
    if (cls != 0) {
      const lds_char* Ks = (const lds_char*)(kv[stage][0]);
      const lds_char* Vs = (const lds_char*)(kv[stage][1]);
      const int k0 = kt * BN;
      // S^T = K Q^T and dP^T = V dO^T : M = keys (2 tiles), N = 32 queries.
      // Fragments are read two MFMA pairs ahead (order kept by the
      // scheduling barriers), so LDS latency overlaps the matrix core.
      f32x16 sacc[2], pacc[2];
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int i = 0; i < 16; ++i) { sacc[mt][i] = 0.f; pacc[mt][i] = 0.f; }
      {
        bf16x8 fk[3], fv[3];
        auto roff = [&](int y) { return (rf ^ ((y & 7) << 4)) + (y >> 3) * 8192; };
#pragma unroll
        for (int y = 0; y < 2; ++y) {
          fk[y] = frag(Ks, roff(y));
          fv[y] = frag(Vs, roff(y));
        }
#pragma unroll
        for (int x = 0; x < 16; ++x) {
          const int mt = x >> 3, ks = x & 7;
          if (x + 2 < 16) {
            fk[(x + 2) % 3] = frag(Ks, roff(x + 2));
            fv[(x + 2) % 3] = frag(Vs, roff(x + 2));
          }
          sacc[mt] = mfma32(fk[x % 3], qf[ks], sacc[mt]);
          pacc[mt] = mfma32(fv[x % 3], dof[ks], pacc[mt]);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      // dS^T = P^T (dP^T - Delta); element i of lane (l32, gq) in M-tile mt is
      // key k0 + 4gq + dk with dk = 32mt + 8(i/4) + i%4, query qi.  In a mixed
      // tile an invisible pair gets P = 0 (so dS = 0): visible iff dk <= a
      // (causal) and, with a window, wb < dk (inside it) or dk < cs (a kept
      // first token); a, wb, cs per lane, one or two compares and a select
      // per element, applied to P.
      auto exps = [&](auto MASK) {
        constexpr int mode = decltype(MASK)::value;  // 0: none, 1: range, 2: range or kept token
        int wb = 0, cs = 0;
        uint32_t span = 0u;
        if constexpr (mode > 0) {
          const int kb = k0 + 4 * gq;
          const int a = qi - kb;
          // a window longer than qi + 1 keys, or none, covers the same keys
          // as qi + 1 (all causal keys)
          const int wlen = p.window > 0 ? min(p.window, qi + 1) : qi + 1;
          wb = a - wlen;
          span = static_cast<uint32_t>(wlen);
          if constexpr (mode == 2) cs = min(p.n_sink - kb, a + 1);
        }
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            float pe = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[mt][i], c, -lb));
            if constexpr (mode > 0) {
              const int dk = 32 * mt + 8 * (i >> 2) + (i & 3);
              bool vis = static_cast<uint32_t>(dk - wb - 1) < span;
              if constexpr (mode == 2) vis = vis || dk < cs;
              pe = vis ? pe : 0.f;
            }
            pacc[mt][i] = pe * (pacc[mt][i] - Dq);
          }
      };
      if (cls != 2) exps(std::integral_constant<int, 0>{});
      else if (p.window <= 0 || k0 >= p.n_sink) exps(std::integral_constant<int, 1>{});   // uniform
      else exps(std::integral_constant<int, 2>{});
      // dQ^T += K^T dS^T : M = dims (4 tiles), N = 32 queries, K = 64 keys.
#pragma unroll
      for (int cc = 0; cc < 4; ++cc) {
        const bf16x8 dsb = pack_kstep(pacc[cc >> 1], cc & 1);
#pragma unroll
        for (int dt = 0; dt < 4; ++dt)
          dqacc[dt] = mfma32(tr_pair(Ks, (ta ^ (dt << 6)) + cc * 4096, (tb ^ (dt << 6)) + cc * 4096), dsb, dqacc[dt]);
      }
    }
    // The next tile landed and no read of this stage is in flight when it is
    // refilled.
    wait_bar<0>();
    stage ^= 1;
    kt = kt_next;
  }

  // dQ = alpha * acc: lane (query qi, gq) holds dims dt*32 + 8u + 4gq + 0..3.
  if (qi < wq1) {
    uint16_t* dst = dQ + (static_cast<size_t>(t0 + qi) * p.hq + h) * D + 4 * gq;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        u32x2 pk;
        pk[0] = pack_bf16x2(p.scale * dqacc[dt][4 * u], p.scale * dqacc[dt][4 * u + 1]);
        pk[1] = pack_bf16x2(p.scale * dqacc[dt][4 * u + 2], p.scale * dqacc[dt][4 * u + 3]);
        *reinterpret_cast<u32x2*>(dst + dt * 32 + 8 * u) = pk;
      }
  }
}

}  // namespace dq128

hipError_t launch_bwd_dq(const Prefill& p, const void* q, const void* k, const void* v,
                         const void* dout, const BwdWork& w, void* dq, hipStream_t st) {
  if (p.total == 0 || p.batch == 0) return hipSuccess;
  const qm::Geo geo = qm::make_geo(p, dq128::NWQ, dq128::QWQ);
  const long long grid = static_cast<long long>(geo.nptiles) * p.batch * geo.Z;
  if (grid <= 0) return hipSuccess;
  hipLaunchKernelGGL(dq128::dq_kernel, dim3(static_cast<unsigned>(grid)), dim3(512), 0, st, p, geo,
                     static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                     static_cast<const uint16_t*>(v), static_cast<const uint16_t*>(dout), w,
                     static_cast<uint16_t*>(dq));
  return hipGetLastError();
}

}  // namespace sa
