// Forward for bfloat16, head_dim 128, on gfx950 matrix cores.
//
// What is computed is the forward of "Attention Sink, Learnable Sink and
// dsink" (notes.kuangjux.top): scores x = alpha <Q, K> (s1), softmax over the
// valid keys, O = sum P V (s1), with the sink applied as the output scale
// s = sigma(L_orig - a_h) and O_new = s O_orig (s4).  lse is L_orig.
//
// Work decomposition (geometry and schedule in qmajor.cuh):
//   * A workgroup is 4 wavefronts of one KV head; each wavefront owns 64
//     query rows of one query head.  Keys come in 64-key tiles loaded straight
//     into LDS (global_load_lds_dwordx4, double-buffered), and only the tiles
//     the mask can reach are visited: every causal tile, or the first-token
//     tiles plus the window tiles, or the union of the selected blocks.  Each
//     wavefront classifies a tile as empty (skipped), full, or mixed (element
//     mask).
//   * Scores are computed transposed, S^T = K Q^T, with
//     v_mfma_f32_32x32x16_bf16: in the 32x32 result each lane holds 16 keys
//     of ONE query (its column), so the online-softmax max and sum stay in
//     registers plus one exchange between the two lane halves.  The same
//     registers, converted to bf16, are the B operand of O^T += V^T P^T; the
//     V^T operand comes from the staged V tile by ds_read_b64_tr_b16.
//   * Online softmax with lazy rescaling: the exponent base only moves when a
//     row's max grows by more than 2^8 (P <= 256), which is exact because O
//     and l always share the same base.
#include "qmajor.cuh"

namespace sa {
namespace fwd128 {

using namespace qm;

constexpr float kRescaleLog2 = 8.f;    // lazy-rescale threshold (log2 units)

__global__ __launch_bounds__(256, 1) void fwd_kernel(Prefill p, Geo geo,
                                                     const uint16_t* __restrict__ Q,
                                                     const uint16_t* __restrict__ K,
                                                     const uint16_t* __restrict__ V,
                                                     uint16_t* __restrict__ O,
                                                     float* __restrict__ lse_out,
                                                     float* __restrict__ s_out) {
  __shared__ __attribute__((aligned(16))) uint16_t kv[2][2][TILE];   // [stage][K, V]
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
  // gq*64 + ks*8 .. +8 for k-step ks (the K fragments use the same order).
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

  Sched sc = make_sched(p, L, qoff, g, p0, p1, bitmap);

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

  const size_t kvs = static_cast<size_t>(p.hkv) * D;
  const uint16_t* Kg = K + static_cast<size_t>(t0) * kvs + g * D;
  const uint16_t* Vg = V + static_cast<size_t>(t0) * kvs + g * D;
  auto issue = [&](int kt, int st) {
    const int k0 = kt * BN;
    const int nvalid = min(BN, L - k0);
    load_tile_lds(Kg + static_cast<size_t>(k0) * kvs, kvs, nvalid, kv[st][0], w, NW, lane);
    load_tile_lds(Vg + static_cast<size_t>(k0) * kvs, kvs, nvalid, kv[st][1], w, NW, lane);
  };

  int kt = sc.next();
  if (kt >= 0) issue(kt, 0);
  __syncthreads();
  int stage = 0;
  while (kt >= 0) {
    const int kt_next = sc.next();
    if (kt_next >= 0) issue(kt_next, stage ^ 1);

    const int cls = wave_tile_class(p, qoff, g, wq0, wq1, kt);
    if (cls != 0) {
      const uint16_t* Ks = kv[stage][0];
      const uint16_t* Vs = kv[stage][1];
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
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) {
          const bf16x8 kf = row_frag(Ks, mt * 32 + l32, gq * 8 + ks);
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
#pragma unroll
        for (int cc = 0; cc < 4; ++cc) pf[nt][cc] = pack_kstep(sacc[cc >> 1][nt], cc & 1);
      }
      // O^T += V^T P^T : M = dims (4 tiles), N = queries (2), K = 64 keys (4 steps).
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) {
#pragma unroll
        for (int cc = 0; cc < 4; ++cc) {
          const bf16x8 vf = tr_frag(Vs, 16 * cc, dt * 32, lane);
#pragma unroll
          for (int nt = 0; nt < 2; ++nt) oacc[dt][nt] = mfma32(vf, pf[nt][cc], oacc[dt][nt]);
        }
      }
    }
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
  Sched sc = make_sched(p, L, qoff, wc.g, p0, p1, bitmap);
  // The wavefronts of the first head of the workgroup: each covers QW rows.
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
  if (p.dtype != SINK_ATTN_BF16 || p.d != qm::D) return false;
  if (p.blocks != nullptr && p.max_seqlen > qm::MAX_BITMAP_WORDS * 32 * qm::BN) return false;
  return true;
}

hipError_t launch_fwd_mfma(const Prefill& p, const void* q, const void* k, const void* v, void* o,
                           float* lse, float* s, hipStream_t st) {
  if (p.total == 0 || p.batch == 0) return hipSuccess;
  const qm::Geo geo = qm::make_geo(p);
  const long long grid = static_cast<long long>(geo.nptiles) * p.batch * geo.Z;
  if (grid <= 0) return hipSuccess;
  hipLaunchKernelGGL(fwd128::fwd_kernel, dim3(static_cast<unsigned>(grid)), dim3(256), 0, st, p, geo,
                     static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                     static_cast<const uint16_t*>(v), static_cast<uint16_t*>(o), lse, s);
  return hipGetLastError();
}

hipError_t launch_visit_map(const Prefill& p, uint8_t* out, hipStream_t st) {
  if (p.total == 0 || p.batch == 0) return hipSuccess;
  const qm::Geo geo = qm::make_geo(p);
  const long long grid = static_cast<long long>(geo.nptiles) * p.batch * geo.Z;
  if (grid <= 0) return hipSuccess;
  hipLaunchKernelGGL(fwd128::visit_map_kernel, dim3(static_cast<unsigned>(grid)), dim3(256), 0, st,
                     p, geo, out);
  return hipGetLastError();
}

}  // namespace sa
