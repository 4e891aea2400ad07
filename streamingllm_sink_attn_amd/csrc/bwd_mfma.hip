// dK and dV on gfx950 matrix cores (bfloat16, head_dim 128), key-major.
//
// What is computed ("Attention Sink, Learnable Sink and dsink", s8): with P
// rebuilt from L_new = log(Z + e^{a_h}) (the sink's normalisation is already
// in it) and Delta = rowsum(dO * O_new) from the preprocess,
//   dS = P * (dO V^T - Delta),  dV = sum_h P^T dO,  dK = alpha sum_h dS^T Q.
// dQ is computed query-major by the dQ kernel.  dsink needs no per-visit work
// here: it was reduced per query row in the preprocess, so a key tile never
// adds it again (s10's double-count warning).
//
// Work decomposition:
//   * One workgroup of 2 wavefronts owns a 64-key tile of one KV head (one
//     block of the block lists); wavefront w owns keys 32w..32w+31.  It walks
//     every (query head of the group, 64-row query tile) that can see the
//     tile: the causal tiles, the window tiles (every tile for a tile holding
//     first tokens), or the reverse block list of the tile.  dK and dV stay in
//     registers across all of them and are written once.
//   * Per (head, query tile): S = Q K^T and dP = dO V^T with
//     v_mfma_f32_32x32x16_bf16 (lane column = key), so the P^T and dS^T
//     registers are directly the A operands of dV += P^T dO and
//     dK += dS^T Q; dO^T and Q^T come from LDS through ds_read_b64_tr_b16.
//   * Q and dO tiles go straight into LDS (global_load_lds_dwordx4),
//     double-buffered; L_new and Delta of the 64 rows through registers.
#include "qmajor.cuh"

namespace sa {
namespace bwd128 {

using namespace qm;

constexpr int BM = 64;            // query rows per iteration
constexpr int NWK = 2;            // wavefronts per workgroup

__global__ __launch_bounds__(128, 2) void dkdv_kernel(Prefill p, int nkt,
                                                      const uint16_t* __restrict__ Q,
                                                      const uint16_t* __restrict__ K,
                                                      const uint16_t* __restrict__ V,
                                                      const uint16_t* __restrict__ dO, BwdWork w,
                                                      uint16_t* __restrict__ dK,
                                                      uint16_t* __restrict__ dV) {
  __shared__ __attribute__((aligned(16))) uint16_t qbuf[2][TILE];
  __shared__ __attribute__((aligned(16))) uint16_t dobuf[2][TILE];
  __shared__ __attribute__((aligned(16))) float lbuf[2][BM];
  __shared__ __attribute__((aligned(16))) float dbuf[2][BM];

  // Flat block id -> (key tile, sample, KV head), key tiles ascending: the
  // tiles with the most query rows (early causal tiles, first-token tiles)
  // start first.
  const int per_kt = p.batch * p.hkv;
  const int kt = blockIdx.x / per_kt;
  const int b = (blockIdx.x % per_kt) / p.hkv;
  const int g = blockIdx.x % p.hkv;
  (void)nkt;
  const int t0 = p.cu[b];
  const int L = p.cu[b + 1] - t0;
  const int k0 = kt * BN;
  if (k0 >= L) return;

  const int tid = threadIdx.x;
  const int wv = tid >> 6;
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int gq = lane >> 5;
  const int G = p.hq / p.hkv;
  const int kw0 = k0 + 32 * wv;         // this wavefront's first key
  const size_t kvs = static_cast<size_t>(p.hkv) * D;
  const size_t qst = static_cast<size_t>(p.hq) * D;

  // ---- query tiles that can see this key tile ----
  const int nqt = (L + BM - 1) / BM;
  int qt_begin = kt, qt_end = nqt;                  // causal
  const int32_t* list = nullptr;
  int list_n = 0;
  if (p.blocks != nullptr) {
    const int idx = (q_block_offset(p.cu, b) + kt) * p.hkv + g;
    list = w.csr_idx + w.csr_off[idx];
    list_n = w.csr_off[idx + 1] - w.csr_off[idx];
  } else if (p.window > 0 && k0 >= p.n_sink) {
    // no first token here: only queries with q - key < window see the tile
    const int last_q = min(L - 1, k0 + BN - 1 + p.window - 1);
    qt_end = last_q / BM + 1;
  }
  const int per_head = p.blocks ? list_n : (qt_end - qt_begin);
  const int n_iter = G * per_head;

  // ---- K, V as B operands (lane: key kw0 + l32, dims gq*64 + ks*8) ----
  bf16x8 kB[8], vB[8];
  {
    const int key = kw0 + l32;
    const bool ok = key < L;
    const uint16_t* ks_ = K + static_cast<size_t>(t0 + (ok ? key : 0)) * kvs + g * D + gq * 64;
    const uint16_t* vs_ = V + static_cast<size_t>(t0 + (ok ? key : 0)) * kvs + g * D + gq * 64;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      kB[ks] = ok ? __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(ks_ + ks * 8))
                  : __builtin_bit_cast(bf16x8, u32x4{0u, 0u, 0u, 0u});
      vB[ks] = ok ? __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(vs_ + ks * 8))
                  : __builtin_bit_cast(bf16x8, u32x4{0u, 0u, 0u, 0u});
    }
  }

  f32x16 dKacc[4], dVacc[4];
#pragma unroll
  for (int nt = 0; nt < 4; ++nt)
#pragma unroll
    for (int i = 0; i < 16; ++i) { dKacc[nt][i] = 0.f; dVacc[nt][i] = 0.f; }

  const float c_l2 = p.scale * kLog2e;

  auto coord = [&](int it, int* h, int* qt) {
    const int hh = it / per_head;
    const int n = it % per_head;
    *h = g * G + hh;
    *qt = p.blocks ? list[n] : qt_begin + n;
  };
  // L_new (wavefront 0) or Delta (wavefront 1) of row `lane` of the tile:
  // Hq floats apart in memory, so they go through a register into LDS.
  auto load_ld = [&](int it) -> float {
    int h, qt;
    coord(it, &h, &qt);
    const int q0 = qt * BM;
    const int row = min(lane, min(BM, L - q0) - 1);
    const size_t idx = static_cast<size_t>(t0 + q0 + row) * p.hq + h;
    return wv == 0 ? w.lnew[idx] : w.delta[idx];
  };
  auto store_ld = [&](int buf, float x) {
    if (wv == 0) lbuf[buf][lane] = x;
    else dbuf[buf][lane] = x;
  };
  auto issue = [&](int it, int buf) {
    int h, qt;
    coord(it, &h, &qt);
    const int q0 = qt * BM;
    const int nvalid = min(BM, L - q0);
    load_tile_lds(Q + static_cast<size_t>(t0 + q0) * qst + h * D, qst, nvalid, qbuf[buf], wv, NWK, lane);
    load_tile_lds(dO + static_cast<size_t>(t0 + q0) * qst + h * D, qst, nvalid, dobuf[buf], wv, NWK, lane);
  };

  if (n_iter > 0) {
    const float x = load_ld(0);
    issue(0, 0);
    store_ld(0, x);
  }
  __syncthreads();

  for (int it = 0; it < n_iter; ++it) {
    const int buf = it & 1;
    const bool has_next = it + 1 < n_iter;
    float ld_next = 0.f;
    if (has_next) {
      ld_next = load_ld(it + 1);
      issue(it + 1, buf ^ 1);
    }
    int h, qt;
    coord(it, &h, &qt);
    const int q0 = qt * BM;
    const int q1 = min(L, q0 + BM);
    int cls = classify_tile(q0, q1, kw0, 32, p.n_sink, p.window);
    if (cls == 1 && q1 - q0 < BM) cls = 2;          // rows past the sample must be masked
    if (cls != 0) {
      const uint16_t* qs = qbuf[buf];
      const uint16_t* dos = dobuf[buf];
      // S = Q K^T, dP = dO V^T : M = query rows (2 tiles), N = this wave's 32 keys
      f32x16 sacc[2], pacc[2];
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) {
#pragma unroll
        for (int i = 0; i < 16; ++i) { sacc[mt][i] = 0.f; pacc[mt][i] = 0.f; }
        const int row = 32 * mt + l32;
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) {
          sacc[mt] = mfma32(row_frag(qs, row, gq * 8 + ks), kB[ks], sacc[mt]);
          pacc[mt] = mfma32(row_frag(dos, row, gq * 8 + ks), vB[ks], pacc[mt]);
        }
      }
      // P = e^{x - L_new}; dS = P (dP - Delta).  Element i of lane (l32, gq)
      // in M-tile mt: query row 32mt + 8(i/4) + 4gq + i%4, key kw0 + l32.
      const int key = kw0 + l32;
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) {
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int r0 = 32 * mt + 8 * u + 4 * gq;
          const f32x4 lv = *reinterpret_cast<const f32x4*>(&lbuf[buf][r0]);
          const f32x4 dv = *reinterpret_cast<const f32x4*>(&dbuf[buf][r0]);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int i = 4 * u + e;
            float pe = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[mt][i], c_l2, -lv[e] * kLog2e));
            if (cls == 2) {
              const int qi = q0 + r0 + e;
              if (!(qi < L && key_visible(qi, key, p.n_sink, p.window))) pe = 0.f;
            }
            sacc[mt][i] = pe;
            pacc[mt][i] = pe * (pacc[mt][i] - dv[e]);
          }
        }
      }
      // dV += P^T dO and dK += dS^T Q: N = dims (4 tiles), K = 64 query rows.
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const bf16x8 pa = pack_kstep(sacc[c >> 1], c & 1);
        const bf16x8 da = pack_kstep(pacc[c >> 1], c & 1);
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) {
          dVacc[nt] = mfma32(pa, tr_frag(dos, 16 * c, nt * 32, lane), dVacc[nt]);
          dKacc[nt] = mfma32(da, tr_frag(qs, 16 * c, nt * 32, lane), dKacc[nt]);
        }
      }
    }
    if (has_next) store_ld(buf ^ 1, ld_next);
    __syncthreads();
  }

  // ---- write dK (alpha-scaled) and dV: lane (dim nt*32 + l32, gq) holds
  //      keys kw0 + 8(i/4) + 4gq + i%4 of C tile nt.
#pragma unroll
  for (int nt = 0; nt < 4; ++nt) {
    const int dim = nt * 32 + l32;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int key = kw0 + 8 * (i >> 2) + 4 * gq + (i & 3);
      if (key < L) {
        const size_t o = static_cast<size_t>(t0 + key) * kvs + g * D + dim;
        dK[o] = f32_to_bf16(p.scale * dKacc[nt][i]);
        dV[o] = f32_to_bf16(dVacc[nt][i]);
      }
    }
  }
}

}  // namespace bwd128

bool bwd_mfma_supported(const Prefill& p) {
  return p.dtype == SINK_ATTN_BF16 && p.d == qm::D &&
         (p.blocks == nullptr || p.max_seqlen <= qm::MAX_BITMAP_WORDS * 32 * qm::BN);
}

hipError_t launch_bwd_dq(const Prefill& p, const void* q, const void* k, const void* v,
                         const void* dout, const BwdWork& w, void* dq, hipStream_t st);

hipError_t launch_bwd_mfma(const Prefill& p, const void* q, const void* k, const void* v,
                           const void* dout, const BwdWork& w, void* dq, void* dk, void* dv,
                           hipStream_t st) {
  if (p.total == 0 || p.batch == 0) return hipSuccess;
  const int nkt = (p.max_seqlen + qm::BN - 1) / qm::BN;
  const long long grid = static_cast<long long>(nkt) * p.batch * p.hkv;
  if (grid <= 0) return hipSuccess;
  hipLaunchKernelGGL(bwd128::dkdv_kernel, dim3(static_cast<unsigned>(grid)), dim3(128), 0, st, p,
                     nkt, static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                     static_cast<const uint16_t*>(v), static_cast<const uint16_t*>(dout), w,
                     static_cast<uint16_t*>(dk), static_cast<uint16_t*>(dv));
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_bwd_dq(p, q, k, v, dout, w, dq, st);
}

}  // namespace sa
