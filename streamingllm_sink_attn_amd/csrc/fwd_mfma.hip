// Forward for bfloat16, head_dim 128, on gfx950 matrix cores.
//
// What is computed is the forward of "Attention Sink, Learnable Sink and
// dsink" (notes.kuangjux.top): scores x = alpha <Q, K> (s1), softmax over the
// valid keys, O = sum P V (s1), with the sink applied as the output scale
// s = sigma(L_orig - a_h) and O_new = s O_orig (s4).  lse is L_orig.
//
// Work decomposition
//   * A workgroup is 4 wavefronts that share one KV head g: GQA packing puts
//     up to 4 query heads of the group in one workgroup, so every K/V tile
//     staged in LDS feeds 4 x 64 query rows.  Each wavefront owns 64 query
//     rows of one head.
//   * Keys are processed in tiles of 64.  The tiles visited are only the
//     ones the mask can reach: every causal tile, or (with a window) the
//     first-token tiles plus the window tiles, or (with block lists) the union
//     of the selected blocks.  Each wavefront then classifies each tile as
//     empty (skipped), full (no mask work) or mixed (element mask).
//   * Scores are computed transposed, S^T = K Q^T, with
//     v_mfma_f32_32x32x16_bf16: in the 32x32 result each lane holds 16 keys
//     of ONE query (its column), so the row max and row sum of the online
//     softmax stay in registers plus one exchange between the two lane
//     halves.  The same registers, converted to bf16, are the B operand of
//     O^T += V^T P^T; only V has to be transposed, which happens once per
//     tile while staging it into LDS.
//   * Online softmax with lazy rescaling: the running max used as the
//     exponent base only moves when a row's max grows by more than 2^8, which
//     keeps P <= 256 and the result exact (O and l share the same base).
//   * Heavy (late, more-keys) position tiles are dispatched first; KV heads
//     map onto XCDs so that all readers of one K/V slice share one L2.
#include "common.cuh"

namespace sa {
namespace fwd128 {

constexpr int D = 128;
constexpr int BN = 64;                 // keys per tile (= block size of block lists)
constexpr int NW = 4;                  // wavefronts per workgroup
constexpr int QW = 64;                 // query rows per wavefront
constexpr int KS = D + 8;              // LDS row stride of K (elements): 272 B
constexpr int VS = BN + 4;             // LDS row stride of V^T (elements): 136 B
constexpr int K_ELEMS = BN * KS;
constexpr int V_ELEMS = D * VS;
constexpr int STAGE = K_ELEMS + V_ELEMS;
constexpr int MAX_BITMAP_WORDS = 256;  // block lists: up to 8192 KV blocks per sample
constexpr float kRescaleLog2 = 8.f;    // lazy-rescale threshold (log2 units)

struct Geo {
  int hw;       // query heads per workgroup
  int wph;      // wavefronts per head
  int P;        // query positions per workgroup
  int nptiles;  // position tiles per sample (from max_seqlen)
  int nhg;      // head groups per KV head
  int Z;        // hkv * nhg
};

static Geo make_geo(const Prefill& p) {
  Geo g;
  const int G = p.hq / p.hkv;
  g.hw = (G % 4 == 0) ? 4 : (G % 2 == 0 ? 2 : 1);
  g.wph = NW / g.hw;
  g.P = QW * g.wph;
  g.nptiles = (p.max_seqlen + g.P - 1) / g.P;
  g.nhg = G / g.hw;
  g.Z = p.hkv * g.nhg;
  return g;
}

// Workgroup coordinates from the flat block id: position tiles slowest and
// heaviest first, then sample, then (KV head, head group).
struct WgCoord {
  int pt, b, g, hg;
};
__device__ __forceinline__ WgCoord wg_coord(const Geo& geo, int batch, int bid) {
  WgCoord c;
  const int per_pt = batch * geo.Z;
  c.pt = geo.nptiles - 1 - bid / per_pt;
  const int rem = bid % per_pt;
  c.b = rem / geo.Z;
  const int z = rem % geo.Z;
  c.g = z / geo.nhg;
  c.hg = z % geo.nhg;
  return c;
}

// The workgroup's key-tile schedule: ranges without block lists, else the
// union bitmap of the selected blocks (built in LDS by the caller).
struct Sched {
  bool blk;
  TileRanges tr;
  int n;
  int word, nwords;
  uint32_t bits;
  const uint32_t* bm;
  __device__ __forceinline__ int next() {
    if (!blk) return n < tr.count() ? tr.at(n++) : -1;
    while (bits == 0) {
      if (++word >= nwords) return -1;
      bits = bm[word];
    }
    const int kb = word * 32 + __builtin_ctz(bits);
    bits &= bits - 1;
    return kb;
  }
};

// Builds the bitmap of KV blocks selected by any query block in [p0, p1)
// (causal blocks only).  Every thread of the workgroup must call it.
__device__ __forceinline__ void build_block_bitmap(const Prefill& p, int L, int qoff, int g,
                                                   int p0, int p1, uint32_t* bm, int* nwords_out) {
  const int nkb = (L + BN - 1) / BN;
  const int nwords = min((nkb + 31) / 32, MAX_BITMAP_WORDS);
  for (int i = threadIdx.x; i < nwords; i += blockDim.x) bm[i] = 0u;
  __syncthreads();
  const int qb0 = p0 / BN, qb1 = (p1 - 1) / BN;
  const int total = (qb1 - qb0 + 1) * p.max_blocks;
  for (int idx = threadIdx.x; idx < total; idx += blockDim.x) {
    const int qb = qb0 + idx / p.max_blocks;
    const int e = idx % p.max_blocks;
    const int kb = p.blocks[(static_cast<size_t>(qoff + qb) * p.hkv + g) * p.max_blocks + e];
    if (kb >= 0 && kb <= qb && (kb >> 5) < nwords) atomicOr(&bm[kb >> 5], 1u << (kb & 31));
  }
  __syncthreads();
  *nwords_out = nwords;
}

// Class of key tile kt for a wavefront's rows [wq0, wq1): 0 empty, 1 full,
// 2 mixed.  With block lists the wavefront's own query block must select it.
__device__ __forceinline__ int wave_tile_class(const Prefill& p, int qoff, int g, int wq0, int wq1,
                                               int kt) {
  if (wq0 >= wq1) return 0;
  int cls = classify_tile(wq0, wq1, kt * BN, BN, p.n_sink, p.window);
  if (cls != 0 && p.blocks != nullptr) {
    const int32_t* row =
        p.blocks + (static_cast<size_t>(qoff + wq0 / BN) * p.hkv + g) * p.max_blocks;
    if (!row_selects(row, p.max_blocks, kt)) cls = 0;
  }
  return cls;
}

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2 v = {static_cast<__bf16>(lo), static_cast<__bf16>(hi)};
  return __builtin_bit_cast(uint32_t, v);
}

__global__ __launch_bounds__(256, 1) void fwd_kernel(Prefill p, Geo geo,
                                                     const uint16_t* __restrict__ Q,
                                                     const uint16_t* __restrict__ K,
                                                     const uint16_t* __restrict__ V,
                                                     uint16_t* __restrict__ O,
                                                     float* __restrict__ lse_out,
                                                     float* __restrict__ s_out) {
  __shared__ __attribute__((aligned(16))) uint16_t smem[2 * STAGE];
  __shared__ uint32_t bitmap[MAX_BITMAP_WORDS];

  const WgCoord wc = wg_coord(geo, p.batch, blockIdx.x);
  const int t0 = p.cu[wc.b];
  const int L = p.cu[wc.b + 1] - t0;
  const int p0 = wc.pt * geo.P;
  if (p0 >= L) return;                               // uniform over the workgroup
  const int p1 = min(L, p0 + geo.P);

  const int tid = threadIdx.x;
  const int w = tid >> 6;
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int gq = lane >> 5;
  const int G = p.hq / p.hkv;
  const int g = wc.g;
  const int h = g * G + wc.hg * geo.hw + w / geo.wph;
  const int wq0 = p0 + (w % geo.wph) * QW;
  const int wq1 = min(L, wq0 + QW);
  const bool wave_rows = wq0 < wq1;
  const int qoff = p.blocks ? q_block_offset(p.cu, wc.b) : 0;

  // Q^T as the B operand: lane (query l32 of N-tile nt, half gq) holds dims
  // gq*64 + ks*8 .. +8 for k-step ks (a fixed permutation of the contraction
  // index shared with the K reads below).
  bf16x8 qf[2][8];
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
    const int qi = wq0 + nt * 32 + l32;
    if (qi < L) {
      const uint16_t* src = Q + (static_cast<size_t>(t0 + qi) * p.hq + h) * D + gq * 64;
#pragma unroll
      for (int ks = 0; ks < 8; ++ks)
        qf[nt][ks] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(src + ks * 8));
    } else {
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) qf[nt][ks] = __builtin_bit_cast(bf16x8, u32x4{0u, 0u, 0u, 0u});
    }
  }

  Sched sc;
  sc.blk = p.blocks != nullptr;
  sc.n = 0;
  sc.word = -1;
  sc.bits = 0u;
  sc.bm = bitmap;
  sc.nwords = 0;
  if (sc.blk) {
    build_block_bitmap(p, L, qoff, g, p0, p1, bitmap, &sc.nwords);
  } else {
    sc.tr = window_tiles(p0, p1, p.n_sink, p.window, BN);
  }

  const float c = p.scale * kLog2e;                  // exp(scale*x) = exp2(c*x)
  const float thr = kRescaleLog2 / c;                // raw-score rescale threshold
  f32x16 oacc[4][2];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int nt = 0; nt < 2; ++nt)
#pragma unroll
      for (int i = 0; i < 16; ++i) oacc[dt][nt][i] = 0.f;
  float mrun[2] = {-kInf, -kInf};
  float lsum[2] = {0.f, 0.f};

  // Global -> register staging of one key tile; each thread moves 4 x 16 B of
  // K (rows tid/16 + 16r, chunk tid%16) and 4 x 16 B of V (keys 4*(tid/16)+r,
  // dims 8*(tid%16)..+8) so that V can be written transposed.
  u32x4 kreg[4], vreg[4];
  const uint16_t* Kbase = K + (static_cast<size_t>(t0) * p.hkv + g) * D;
  const uint16_t* Vbase = V + (static_cast<size_t>(t0) * p.hkv + g) * D;
  const size_t kv_stride = static_cast<size_t>(p.hkv) * D;
  auto load_tile = [&](int kt) {
    const int k0 = kt * BN;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int ci = tid + 256 * r;
      const int key = k0 + (ci >> 4);
      kreg[r] = key < L ? *reinterpret_cast<const u32x4*>(Kbase + key * kv_stride + (ci & 15) * 8)
                        : u32x4{0u, 0u, 0u, 0u};
      const int vkey = k0 + (tid >> 4) * 4 + r;
      vreg[r] = vkey < L ? *reinterpret_cast<const u32x4*>(Vbase + vkey * kv_stride + (tid & 15) * 8)
                         : u32x4{0u, 0u, 0u, 0u};
    }
  };
  auto store_tile = [&](int stage) {
    uint16_t* Ks = smem + stage * STAGE;
    uint16_t* Vt = Ks + K_ELEMS;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int ci = tid + 256 * r;
      *reinterpret_cast<u32x4*>(Ks + (ci >> 4) * KS + (ci & 15) * 8) = kreg[r];
    }
    const int dim0 = (tid & 15) * 8;
    const int key0 = (tid >> 4) * 4;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int sh = (e & 1) * 16;
      const uint32_t a0 = (vreg[0][e >> 1] >> sh) & 0xffffu;
      const uint32_t a1 = (vreg[1][e >> 1] >> sh) & 0xffffu;
      const uint32_t a2 = (vreg[2][e >> 1] >> sh) & 0xffffu;
      const uint32_t a3 = (vreg[3][e >> 1] >> sh) & 0xffffu;
      *reinterpret_cast<u32x2*>(Vt + (dim0 + e) * VS + key0) = u32x2{a0 | (a1 << 16), a2 | (a3 << 16)};
    }
  };

  int kt = sc.next();
  if (kt >= 0) {
    load_tile(kt);
    store_tile(0);
  }
  __syncthreads();
  int stage = 0;
  while (kt >= 0) {
    const int kt_next = sc.next();
    if (kt_next >= 0) load_tile(kt_next);

    const int cls = wave_tile_class(p, qoff, g, wq0, wq1, kt);
    if (cls != 0) {
      const uint16_t* Ks = smem + stage * STAGE;
      const uint16_t* Vt = Ks + K_ELEMS;
      const int k0 = kt * BN;
      // S^T = K Q^T : M = keys (2 tiles of 32), N = queries (2 tiles), K = 128
      f32x16 sacc[2][2];
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int nt = 0; nt < 2; ++nt)
#pragma unroll
          for (int i = 0; i < 16; ++i) sacc[mt][nt][i] = 0.f;
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) {
        const uint16_t* krow = Ks + (mt * 32 + l32) * KS + gq * 64;
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) {
          const bf16x8 kf = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(krow + ks * 8));
#pragma unroll
          for (int nt = 0; nt < 2; ++nt) sacc[mt][nt] = mfma32(kf, qf[nt][ks], sacc[mt][nt]);
        }
      }
      // Element mask on mixed tiles.  Result element i of lane (l32, gq) in
      // M-tile mt is key 8*(i/4) + 4*gq + i%4 of that M-tile, query l32.
      if (cls == 2) {
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
          const int qi = wq0 + nt * 32 + l32;
#pragma unroll
          for (int mt = 0; mt < 2; ++mt)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
              const int key = k0 + mt * 32 + 8 * (i >> 2) + 4 * gq + (i & 3);
              if (!key_visible(qi, key, p.n_sink, p.window)) sacc[mt][nt][i] = -kInf;
            }
        }
      }
      // Online softmax (per lane = per query column).
      float mx[2];
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
        float m0 = -kInf;
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
          for (int i = 0; i < 16; ++i) m0 = fmaxf(m0, sacc[mt][nt][i]);
        mx[nt] = fmaxf(m0, __shfl_xor(m0, 32));
      }
      const bool need = (mx[0] > mrun[0] + thr) || (mx[1] > mrun[1] + thr);
      if (__ballot(need) != 0) {
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
          const float mnew = fmaxf(mrun[nt], mx[nt]);
          const float f = (mrun[nt] == -kInf) ? 0.f : __builtin_amdgcn_exp2f((mrun[nt] - mnew) * c);
#pragma unroll
          for (int dt = 0; dt < 4; ++dt)
#pragma unroll
            for (int i = 0; i < 16; ++i) oacc[dt][nt][i] *= f;
          lsum[nt] *= f;
          mrun[nt] = mnew;
        }
      }
      bf16x8 pf[2][4];
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
        const float mb = (mrun[nt] == -kInf) ? 0.f : mrun[nt] * c;
        float ls = 0.f;
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const float e = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[mt][nt][i], c, -mb));
            sacc[mt][nt][i] = e;
            ls += e;
          }
        lsum[nt] += ls;
        // k-step cc of the PV product takes elements (cc%2)*8 .. +8 of M-tile cc/2
#pragma unroll
        for (int cc = 0; cc < 4; ++cc) {
          u32x4 u;
#pragma unroll
          for (int t = 0; t < 4; ++t)
            u[t] = pack_bf16x2(sacc[cc >> 1][nt][(cc & 1) * 8 + 2 * t],
                               sacc[cc >> 1][nt][(cc & 1) * 8 + 2 * t + 1]);
          pf[nt][cc] = __builtin_bit_cast(bf16x8, u);
        }
      }
      // O^T += V^T P^T : M = dims (4 tiles), N = queries (2), K = 64 keys (4
      // steps).  Logical k slot t of half gq in step cc is key
      // 16cc + 8(t/4) + 4gq + t%4, matching the P^T registers above.
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) {
        const uint16_t* vrow = Vt + (dt * 32 + l32) * VS + 4 * gq;
#pragma unroll
        for (int cc = 0; cc < 4; ++cc) {
          const u32x2 lo = *reinterpret_cast<const u32x2*>(vrow + 16 * cc);
          const u32x2 hi = *reinterpret_cast<const u32x2*>(vrow + 16 * cc + 8);
          const bf16x8 vf = __builtin_bit_cast(bf16x8, u32x4{lo[0], lo[1], hi[0], hi[1]});
#pragma unroll
          for (int nt = 0; nt < 2; ++nt) oacc[dt][nt] = mfma32(vf, pf[nt][cc], oacc[dt][nt]);
        }
      }
    }

    if (kt_next >= 0) store_tile(stage ^ 1);
    __syncthreads();
    stage ^= 1;
    kt = kt_next;
  }

  // Epilogue: L_orig = alpha*m + ln l; s = sigma(L_orig - a_h); O = acc * s / l.
  if (!wave_rows) return;
  const bool has_sink = p.sink != nullptr;
  const float a = has_sink ? p.sink[h] : 0.f;
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
    const float lt = lsum[nt] + __shfl_xor(lsum[nt], 32);
    const int qi = wq0 + nt * 32 + l32;
    if (qi >= wq1) continue;
    float L_orig, s_val, mul;
    if (lt > 0.f) {
      L_orig = mrun[nt] * p.scale + __logf(lt);
      s_val = has_sink ? 1.f / (1.f + __expf(a - L_orig)) : 1.f;
      mul = s_val / lt;
    } else {
      L_orig = -kInf;
      s_val = has_sink ? 0.f : 1.f;
      mul = 0.f;
    }
    uint16_t* dst = O + (static_cast<size_t>(t0 + qi) * p.hq + h) * D + 4 * gq;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        u32x2 pk;
        pk[0] = pack_bf16x2(oacc[dt][nt][4 * u] * mul, oacc[dt][nt][4 * u + 1] * mul);
        pk[1] = pack_bf16x2(oacc[dt][nt][4 * u + 2] * mul, oacc[dt][nt][4 * u + 3] * mul);
        *reinterpret_cast<u32x2*>(dst + dt * 32 + 8 * u) = pk;
      }
    if (gq == 0) {
      const size_t r = static_cast<size_t>(t0 + qi) * p.hq + h;
      lse_out[r] = L_orig;
      if (s_out) s_out[r] = s_val;
    }
  }
}

// Test hook: the same geometry, schedule and classification as fwd_kernel,
// marking (query, key) pairs the forward visits and keeps.  One workgroup of
// 256 threads per forward workgroup; out[b][g][i][j] for sample-local i, j.
__global__ __launch_bounds__(256) void visit_map_kernel(Prefill p, Geo geo, uint8_t* out) {
  __shared__ uint32_t bitmap[MAX_BITMAP_WORDS];
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

  Sched sc;
  sc.blk = p.blocks != nullptr;
  sc.n = 0;
  sc.word = -1;
  sc.bits = 0u;
  sc.bm = bitmap;
  sc.nwords = 0;
  if (sc.blk) build_block_bitmap(p, L, qoff, wc.g, p0, p1, bitmap, &sc.nwords);
  else sc.tr = window_tiles(p0, p1, p.n_sink, p.window, BN);

  // Only the wavefronts of the first head of the workgroup: each covers QW rows.
  for (int kt = sc.next(); kt >= 0; kt = sc.next()) {
    for (int wv = 0; wv < geo.wph; ++wv) {
      const int wq0 = p0 + wv * QW;
      const int wq1 = min(L, wq0 + QW);
      const int cls = wave_tile_class(p, qoff, wc.g, wq0, wq1, kt);
      if (cls == 0) continue;
      for (int e = threadIdx.x; e < QW * BN; e += blockDim.x) {
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
  if (p.dtype != SINK_ATTN_BF16 || p.d != fwd128::D) return false;
  if (p.blocks != nullptr) {
    if (p.max_seqlen > fwd128::MAX_BITMAP_WORDS * 32 * fwd128::BN) return false;
  }
  return true;
}

hipError_t launch_fwd_mfma(const Prefill& p, const void* q, const void* k, const void* v, void* o,
                           float* lse, float* s, hipStream_t st) {
  if (p.total == 0 || p.batch == 0) return hipSuccess;
  const fwd128::Geo geo = fwd128::make_geo(p);
  const long long grid = static_cast<long long>(geo.nptiles) * p.batch * geo.Z;
  if (grid <= 0) return hipSuccess;
  hipLaunchKernelGGL(fwd128::fwd_kernel, dim3(static_cast<unsigned>(grid)), dim3(256), 0, st, p, geo,
                     static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                     static_cast<const uint16_t*>(v), static_cast<uint16_t*>(o), lse, s);
  return hipGetLastError();
}

hipError_t launch_visit_map(const Prefill& p, uint8_t* out, hipStream_t st) {
  if (p.total == 0 || p.batch == 0) return hipSuccess;
  const fwd128::Geo geo = fwd128::make_geo(p);
  const long long grid = static_cast<long long>(geo.nptiles) * p.batch * geo.Z;
  if (grid <= 0) return hipSuccess;
  hipLaunchKernelGGL(fwd128::visit_map_kernel, dim3(static_cast<unsigned>(grid)), dim3(256), 0, st,
                     p, geo, out);
  return hipGetLastError();
}

}  // namespace sa
