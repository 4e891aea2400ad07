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
//   * A key tile is 64 keys of one KV head (one block of the block lists).
//     Its iterations are the (query head of the group, 64-row query tile)
//     pairs that can see it: the causal tiles, the window tiles (every tile
//     for a tile holding first tokens), or the reverse block list of the tile
//     ("Attention Sink, Learnable Sink and dsink" s10: work split by KV-block
//     reverse lists).
//   * Tiles differ a lot in work (a first-token tile, or block 0 that every
//     block list selects, is seen by every query tile), so a planning kernel
//     cuts every tile's iterations into chunks of at most item_iters(p) and a
//     persistent kernel pulls chunks from work queues (one per XCD, keyed by
//     KV head, so one XCD's L2 streams one head group's Q/dO).  A tile done in
//     one chunk writes bf16 dK/dV directly; a split tile adds its chunks'
//     float32 partials atomically (once per chunk) and a convert kernel
//     finishes it.
//   * A chunk runs on a workgroup of 2 wavefronts, wavefront w owning keys
//     32w..32w+31.  Per iteration: S = Q K^T and dP = dO V^T with
//     v_mfma_f32_32x32x16_bf16 (lane column = key), so the P^T and dS^T
//     registers are directly the A operands of dV += P^T dO and
//     dK += dS^T Q; dO^T and Q^T come from LDS through ds_read_b64_tr_b16.
//     Q and dO tiles (and the L_new and Delta of their 64 rows) go straight
//     into swizzled LDS, double-buffered: the next tile's loads are issued
//     from asm blocks and waited for explicitly at the end of the iteration,
//     so they overlap the whole current iteration.
//     Per-lane LDS offsets are computed once and the loop is unrolled by two
//     so buffer offsets are immediates.
#include <algorithm>
#include <type_traits>

#include "qmajor.cuh"

namespace sa {
namespace bwd128 {

using namespace qm;

constexpr int BM = 64;            // query rows per iteration
constexpr int NWK = 2;            // wavefronts per workgroup
constexpr int kChunkMax = 256;    // most iterations per work item

// Iterations per work item.  Window and causal key tiles have few iterations
// each (at most (W + 62) / 64 + 1 query tiles times G), and finer items
// balance the queues' tails better; a key tile of the block lists is seen by
// G x (about 17 on average) iterations, so the longer item keeps most tiles
// whole instead of splitting them into float32 partials.  (Measured: window
// 1024, G = 4: dK/dV 1,255 us at 128, 1,369 us at 192; 17 blocks, G = 8:
// 6,174 us at 128, 6,072 us at 256, and half the split-tile passes.)
constexpr int kItemDense = 128, kItemBlocks = 256;
static_assert(kItemDense <= kChunkMax && kItemBlocks <= kChunkMax, "item fits the LDS iteration table");
__host__ __device__ inline int item_iters(const Prefill& p) {
  return p.blocks != nullptr ? kItemBlocks : kItemDense;
}
constexpr int kMaxQueues = 8;

typedef __attribute__((address_space(3))) char lds_char;

// Number of work queues: one per XCD when KV heads spread evenly over 8.
inline int num_queues(const Prefill& p) { return (p.hkv % kMaxQueues == 0) ? kMaxQueues : 1; }

// Key tile ti <-> (b, kt, g): queue-major so each queue's tiles are
// contiguous, then sample, key tile, and the KV heads of the queue.
struct TileId {
  int b, kt, g;
};
__device__ __forceinline__ TileId tile_of(const Prefill& p, int nkt, int nq, int ti) {
  const int hq_per = p.hkv / nq;                   // KV heads per queue
  const int per_q = p.batch * nkt * hq_per;
  const int q = ti / per_q;
  int r = ti % per_q;
  TileId t;
  t.b = r / (nkt * hq_per);
  r %= nkt * hq_per;
  t.kt = r / hq_per;
  t.g = (r % hq_per) * nq + q;
  return t;
}

// Iterations of key tile (b, kt, g): the query tiles [qt_begin, qt_end) or
// the reverse block list, times the G query heads of the group.
struct TileWork {
  int per_head, qt_begin;
  const int32_t* list;
};
__device__ __forceinline__ TileWork tile_work(const Prefill& p, const BwdWork& w, int b, int kt, int g,
                                              int L) {
  TileWork tw;
  tw.list = nullptr;
  tw.qt_begin = kt;
  const int k0 = kt * BN;
  if (k0 >= L) {
    tw.per_head = 0;
    return tw;
  }
  const int nqt = (L + BM - 1) / BM;
  if (p.blocks != nullptr) {
    const int idx = (q_block_offset(p.cu, b) + kt) * p.hkv + g;
    tw.list = w.csr_idx + w.csr_off[idx];
    tw.per_head = w.csr_off[idx + 1] - w.csr_off[idx];
  } else {
    int qt_end = nqt;
    if (p.window > 0 && k0 >= p.n_sink) {
      // no first token here: only queries with q - key < window see the tile
      const int last_q = min(L - 1, k0 + BN - 1 + p.window - 1);
      qt_end = last_q / BM + 1;
    }
    tw.per_head = qt_end - kt;
  }
  return tw;
}

// Chunks per key tile (an empty tile still gets one, which writes zeros),
// and whether the tile is split over several chunks.
__global__ __launch_bounds__(256) void plan_kernel(Prefill p, BwdWork w, int nkt, int nq) {
  const int ntiles = p.batch * nkt * p.hkv;
  const int ti = blockIdx.x * blockDim.x + threadIdx.x;
  if (ti < kMaxQueues && blockIdx.x == 0) w.queues[ti] = 0;
  if (ti >= ntiles) return;
  const TileId t = tile_of(p, nkt, nq, ti);
  const int L = p.cu[t.b + 1] - p.cu[t.b];
  int chunks = 0;
  if (t.kt * BN < L) {
    const TileWork tw = tile_work(p, w, t.b, t.kt, t.g, L);
    const int n = tw.per_head * (p.hq / p.hkv);
    const int per_item = item_iters(p);
    chunks = max(1, (n + per_item - 1) / per_item);
  }
  w.plan[ti + 1] = chunks;
  w.split_slot[ti + 1] = chunks > 1 ? 1 : 0;
}

// After the split tiles are numbered (a scan of the flags): a split tile
// without an accumulator slot runs as one chunk.
__global__ __launch_bounds__(256) void plan_clamp_kernel(Prefill p, BwdWork w, int ntiles) {
  const int ti = blockIdx.x * blockDim.x + threadIdx.x;
  if (ti >= ntiles) return;
  if (w.plan[ti + 1] > 1 && w.split_slot[ti] >= w.max_split) w.plan[ti + 1] = 1;
}

// Zero (before) and convert (after) the float32 accumulators of split tiles.
template <bool kConvert>
__global__ __launch_bounds__(256) void split_tiles_kernel(Prefill p, BwdWork w, int nkt, int nq,
                                                          uint16_t* __restrict__ dK,
                                                          uint16_t* __restrict__ dV) {
  const int ti = blockIdx.x;
  if (w.plan[ti + 1] - w.plan[ti] <= 1) return;
  const TileId t = tile_of(p, nkt, nq, ti);
  const int t0 = p.cu[t.b];
  const int L = p.cu[t.b + 1] - t0;
  const int rows = min(BN, L - t.kt * BN);
  const float* dka = w.dk_acc + static_cast<size_t>(w.split_slot[ti]) * BN * D;
  const float* dva = w.dv_acc + static_cast<size_t>(w.split_slot[ti]) * BN * D;
  // 8 consecutive dims per thread and step: two 16-byte float32 accesses and
  // one 16-byte bf16 store per tensor.
  for (int c = threadIdx.x; c < rows * (D / 8); c += blockDim.x) {
    const int r = c / (D / 8), d0 = (c % (D / 8)) * 8;
    const size_t o = (static_cast<size_t>(t0 + t.kt * BN + r) * p.hkv + t.g) * D + d0;
    const size_t a = static_cast<size_t>(r) * D + d0;       // slot row r
    if (kConvert) {
      const f32x4 k0 = *reinterpret_cast<const f32x4*>(dka + a);
      const f32x4 k1 = *reinterpret_cast<const f32x4*>(dka + a + 4);
      const f32x4 v0 = *reinterpret_cast<const f32x4*>(dva + a);
      const f32x4 v1 = *reinterpret_cast<const f32x4*>(dva + a + 4);
      *reinterpret_cast<u32x4*>(dK + o) = u32x4{pack_bf16x2(k0[0], k0[1]), pack_bf16x2(k0[2], k0[3]),
                                                pack_bf16x2(k1[0], k1[1]), pack_bf16x2(k1[2], k1[3])};
      *reinterpret_cast<u32x4*>(dV + o) = u32x4{pack_bf16x2(v0[0], v0[1]), pack_bf16x2(v0[2], v0[3]),
                                                pack_bf16x2(v1[0], v1[1]), pack_bf16x2(v1[2], v1[3])};
    } else {
      const f32x4 z = {0.f, 0.f, 0.f, 0.f};
      *reinterpret_cast<f32x4*>(const_cast<float*>(dka) + a) = z;
      *reinterpret_cast<f32x4*>(const_cast<float*>(dka) + a + 4) = z;
      *reinterpret_cast<f32x4*>(const_cast<float*>(dva) + a) = z;
      *reinterpret_cast<f32x4*>(const_cast<float*>(dva) + a + 4) = z;
    }
  }
}

__device__ __forceinline__ bf16x8 lds_frag(const lds_char* base, int byte_off) {
  return __builtin_bit_cast(bf16x8, *reinterpret_cast<const __attribute__((address_space(3))) u32x4*>(base + byte_off));
}
__device__ __forceinline__ bf16x8 lds_tr_pair(const lds_char* base, int off_a, int off_b) {
  const u32x2 a = __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                                                (__attribute__((address_space(3))) i16x4*)(base + off_a)));
  const u32x2 b = __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                                                (__attribute__((address_space(3))) i16x4*)(base + off_b)));
  return __builtin_bit_cast(bf16x8, u32x4{a[0], a[1], b[0], b[1]});
}

__global__ __launch_bounds__(128, 2) void dkdv_kernel(Prefill p, int nkt, int nq,
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
  __shared__ int qt_tab[kChunkMax];  // query head and tile of each iteration of the item
  __shared__ int item_sh;

  const int tid = threadIdx.x;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int gq = lane >> 5;
  const int G = p.hq / p.hkv;
  const size_t kvs = static_cast<size_t>(p.hkv) * D;
  const int qst = p.hq * D;
  const float c_l2 = p.scale * kLog2e;

  // Per-lane swizzled LDS byte offsets: row fragments (rows 32mt + l32,
  // logical chunk gq*8 + ks) and transposed fragments (rows 16c + ra0 and
  // +8, dims nt*32 + d4) of a staged 64 x 256-byte tile.
  int roff[8], toa[4], tob[4];
  {
    const int sk = swz16(l32);
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) roff[ks] = l32 * 256 + (((gq * 8 + ks) ^ sk) << 4);
    const int l16 = lane & 15, grp = lane >> 4;
    const int ra0 = 4 * (grp >> 1) + (l16 >> 2);
    const int d4 = 16 * (grp & 1) + 4 * (l16 & 3);
    const int c4 = d4 >> 3, off = (d4 & 7) * 2;
    const int sa_ = swz16(ra0), sb_ = swz16(ra0 + 8);
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
      toa[nt] = ra0 * 256 + (((nt * 4 + c4) ^ sa_) << 4) + off;
      tob[nt] = (ra0 + 8) * 256 + (((nt * 4 + c4) ^ sb_) << 4) + off;
    }
  }

  // This wavefront's share of a 64-row tile: 4-row blocks 8wv .. 8wv + 7.
  uint32_t toff[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int row = 4 * (wv * 8 + j) + (lane >> 4);
    const int lc = (lane & 15) ^ swz16(row);
    toff[j] = static_cast<uint32_t>(row * qst + lc * 8) * 2u;
  }
  const uint32_t qbuf0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(
      (__attribute__((address_space(3))) uint16_t*)(&qbuf[0][0])));
  const uint32_t dobuf0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(
      (__attribute__((address_space(3))) uint16_t*)(&dobuf[0][0])));
  const uint32_t lbuf0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(
      (__attribute__((address_space(3))) float*)(&lbuf[0][0])));
  const uint32_t dbuf0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(
      (__attribute__((address_space(3))) float*)(&dbuf[0][0])));

  const int queue = blockIdx.x % nq;
  const int tiles_per_q = p.batch * nkt * (p.hkv / nq);
  const int item_lo = w.plan[queue * tiles_per_q];
  const int item_hi = w.plan[(queue + 1) * tiles_per_q];

  for (;;) {
    if (tid == 0) item_sh = item_lo + atomicAdd(&w.queues[queue], 1);
    __syncthreads();
    const int item = item_sh;
    __syncthreads();
    if (item >= item_hi) break;

    // item -> (tile, chunk): the tile whose plan range holds it
    int lo = queue * tiles_per_q, hi = (queue + 1) * tiles_per_q - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (w.plan[mid] <= item) lo = mid; else hi = mid - 1;
    }
    const int ti = lo;
    const int chunk = item - w.plan[ti];
    const bool split = (w.plan[ti + 1] - w.plan[ti]) > 1;
    // a split tile's float32 accumulators: slot rows 0..63 = keys k0..k0+63
    const size_t slot_base = split ? static_cast<size_t>(w.split_slot[ti]) * BN * D : 0;
    const TileId t = tile_of(p, nkt, nq, ti);
    const int b = t.b, kt = t.kt, g = t.g;
    const int t0 = p.cu[b];
    const int L = p.cu[b + 1] - t0;
    const int k0 = kt * BN;
    const int kw0 = k0 + 32 * wv;                 // this wavefront's first key
    const TileWork tw = tile_work(p, w, b, kt, g, L);
    const int n_all = G * tw.per_head;
    const int it_begin = chunk * item_iters(p);
    const int it_end = min(n_all, it_begin + item_iters(p));

    // K, V as B operands (lane: key kw0 + l32, dims gq*64 + ks*8)
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
    // The operands must be in registers before any DMA of this item is in
    // flight (the compiler counts only its own loads): consuming them here
    // makes it wait for them before the loop rather than inside it.
    asm volatile("" ::"v"(kB[0]), "v"(kB[1]), "v"(kB[2]), "v"(kB[3]), "v"(kB[4]), "v"(kB[5]),
                 "v"(kB[6]), "v"(kB[7]));
    asm volatile("" ::"v"(vB[0]), "v"(vB[1]), "v"(vB[2]), "v"(vB[3]), "v"(vB[4]), "v"(vB[5]),
                 "v"(vB[6]), "v"(vB[7]));
    // Query tiles of the item's iterations, read from the reverse list once
    // (the loop then issues no vector memory operation besides the DMA).
    // Entry: (query head within the group) << 16 | query tile.
    for (int j = tid; j < it_end - it_begin; j += 64 * NWK) {
      const int it = it_begin + j;
      const int n = it % tw.per_head;
      qt_tab[j] = ((it / tw.per_head) << 16) | (tw.list ? tw.list[n] : tw.qt_begin + n);
    }
    __syncthreads();
    f32x16 dKacc[4], dVacc[4];
#pragma unroll
    for (int nt = 0; nt < 4; ++nt)
#pragma unroll
      for (int i = 0; i < 16; ++i) { dKacc[nt][i] = 0.f; dVacc[nt][i] = 0.f; }

    auto coord = [&](int it, int* h, int* qt) {
      const int e = __builtin_amdgcn_readfirstlane(qt_tab[it - it_begin]);   // scalar from here on
      *h = g * G + (e >> 16);
      *qt = e & 0xffff;
    };
    // Stage the Q / dO tile and the L_new (wavefront 0) or Delta (wavefront
    // 1) rows of iteration it in buffer buf: direct-to-LDS buffer loads from
    // asm blocks (the compiler, which cannot see which LDS bytes they fill,
    // would otherwise wait for them before the current tile's reads).  A
    // ragged tile reads its last row in place of the missing ones.
    auto issue = [&](int it, int buf) {
      int h, qt;
      coord(it, &h, &qt);
      const int q0 = qt * BM;
      const int rows = min(BM, L - q0);
      const size_t r0 = static_cast<size_t>(t0 + q0);
      const u32x4 rq = make_rsrc(Q + r0 * qst + h * D, static_cast<uint32_t>(rows * qst * 2));
      const u32x4 rd = make_rsrc(dO + r0 * qst + h * D, static_cast<uint32_t>(rows * qst * 2));
      if (rows == BM) {                             // uniform: a full tile
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const uint32_t blk = static_cast<uint32_t>(buf * TILE + 4 * (wv * 8 + j) * D) * 2u;
          dma16(rq, toff[j], qbuf0 + blk);
          dma16(rd, toff[j], dobuf0 + blk);
        }
      } else {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int row = 4 * (wv * 8 + j) + (lane >> 4);
          const int lc = (lane & 15) ^ swz16(row);
          const uint32_t o = static_cast<uint32_t>(min(row, rows - 1) * qst + lc * 8) * 2u;
          const uint32_t blk = static_cast<uint32_t>(buf * TILE + 4 * (wv * 8 + j) * D) * 2u;
          dma16(rq, o, qbuf0 + blk);
          dma16(rd, o, dobuf0 + blk);
        }
      }
      const float* src = (wv == 0 ? w.lnew : w.delta) + r0 * p.hq + h;
      const u32x4 rs = make_rsrc(src, static_cast<uint32_t>(rows * p.hq * 4));
      dma4(rs, static_cast<uint32_t>(min(lane, rows - 1) * p.hq) * 4u,
           (wv == 0 ? lbuf0 : dbuf0) + static_cast<uint32_t>(buf * BM * 4));
    };

    // One iteration on LDS buffer BUF: S, dP, P, dS, dV += P^T dO, dK += dS^T Q.
    auto body = [&](auto BUF, int it) {
      constexpr int buf = decltype(BUF)::value;
      int h, qt;
      coord(it, &h, &qt);
      const int q0 = qt * BM;
      const int q1 = min(L, q0 + BM);
      int cls = classify_tile(q0, q1, kw0, 32, p.n_sink, p.window);
      if (cls == 1 && q1 - q0 < BM) cls = 2;        // rows past the sample must be masked
      f32x16 sacc[2], pacc[2];
      if (cls != 0) {
        const lds_char* qs = (const lds_char*)(qbuf[buf]);
        const lds_char* dos = (const lds_char*)(dobuf[buf]);
        // S = Q K^T, dP = dO V^T : M = query rows (2 tiles), N = this wave's 32 keys
        // Fragments are read one step ahead of their MFMAs (order fixed by
        // the scheduling barriers), so LDS latency overlaps the matrix core.
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
          for (int i = 0; i < 16; ++i) { sacc[mt][i] = 0.f; pacc[mt][i] = 0.f; }
        {
          bf16x8 fq[2], fd[2];
          fq[0] = lds_frag(qs, roff[0]);
          fd[0] = lds_frag(dos, roff[0]);
#pragma unroll
          for (int x = 0; x < 16; ++x) {
            const int mt = x >> 3, ks = x & 7;
            if (x + 1 < 16) {
              const int mt1 = (x + 1) >> 3, ks1 = (x + 1) & 7;
              fq[(x + 1) & 1] = lds_frag(qs, roff[ks1] + mt1 * 8192);
              fd[(x + 1) & 1] = lds_frag(dos, roff[ks1] + mt1 * 8192);
            }
            sacc[mt] = mfma32(fq[x & 1], kB[ks], sacc[mt]);
            pacc[mt] = mfma32(fd[x & 1], vB[ks], pacc[mt]);
            __builtin_amdgcn_sched_barrier(0);
          }
        }
      }
      // The next tile's loads are issued behind this tile's first MFMAs.
      if (it + 1 < it_end) issue(it + 1, buf ^ 1);
      if (cls != 0) {
        const lds_char* qs = (const lds_char*)(qbuf[buf]);
        const lds_char* dos = (const lds_char*)(dobuf[buf]);
        // P = e^{x - L_new} (L_new staged in log2 units); dS = P (dP - Delta).
        // Element i of lane (l32, gq) in M-tile mt: query row q0 + 32mt +
        // 8(i/4) + 4gq + i%4, key kw0 + l32.  In a mixed tile an invisible pair gets P = 0 (so dS =
        // 0): with d = row - key, the pair is visible iff 0 <= d < hi, where
        // hi folds the window (unless the key is a kept first token) and the
        // sample end; one unsigned compare and a select per element.
        auto exps = [&](auto MASKED) {
          constexpr bool masked = decltype(MASKED)::value;
          int dbase = 0;
          uint32_t hi = 0u;
          if constexpr (masked) {
            const int key = kw0 + l32;
            dbase = q0 + 4 * gq - key;
            const int lo = (p.window <= 0 || key < p.n_sink) ? 0x7fffffff : p.window;
            hi = static_cast<uint32_t>(max(0, min(lo, L - key)));
          }
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
                float pe = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[mt][i], c_l2, -lv[e]));
                if constexpr (masked)
                  pe = static_cast<uint32_t>(dbase + 32 * mt + 8 * u + e) < hi ? pe : 0.f;
                sacc[mt][i] = pe;
                pacc[mt][i] = pe * (pacc[mt][i] - dv[e]);
              }
            }
          }
        };
        if (cls == 2) exps(std::true_type{});
        else exps(std::false_type{});
        // dV += P^T dO and dK += dS^T Q: N = dims (4 tiles), K = 64 query rows.
        bf16x8 pa[4], da[4];
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          pa[c] = pack_kstep(sacc[c >> 1], c & 1);
          da[c] = pack_kstep(pacc[c >> 1], c & 1);
        }
        {
          bf16x8 fv[2], fk[2];
          fv[0] = lds_tr_pair(dos, toa[0], tob[0]);
          fk[0] = lds_tr_pair(qs, toa[0], tob[0]);
#pragma unroll
          for (int x = 0; x < 16; ++x) {
            const int c = x >> 2, nt = x & 3;
            if (x + 1 < 16) {
              const int c1 = (x + 1) >> 2, nt1 = (x + 1) & 3;
              fv[(x + 1) & 1] = lds_tr_pair(dos, toa[nt1] + c1 * 4096, tob[nt1] + c1 * 4096);
              fk[(x + 1) & 1] = lds_tr_pair(qs, toa[nt1] + c1 * 4096, tob[nt1] + c1 * 4096);
            }
            dVacc[nt] = mfma32(pa[c], fv[x & 1], dVacc[nt]);
            dKacc[nt] = mfma32(da[c], fk[x & 1], dKacc[nt]);
            __builtin_amdgcn_sched_barrier(0);
          }
        }
      }
      // Next tile landed (each wavefront waits for its own loads) and no
      // read of this buffer is in flight when it is refilled.
      wait_bar<0>();
    };

    if (it_begin < it_end) issue(it_begin, 0);
    wait_bar<0>();
    for (int it = it_begin; it < it_end; it += 2) {
      body(std::integral_constant<int, 0>{}, it);
      if (it + 1 < it_end) body(std::integral_constant<int, 1>{}, it + 1);
    }

    // Results: lane (dim nt*32 + l32, gq) holds keys kw0 + 8(i/4) + 4gq + i%4
    // of C tile nt.  dK is alpha-scaled.
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
      const int dim = nt * 32 + l32;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int key = kw0 + 8 * (i >> 2) + 4 * gq + (i & 3);
        if (key < L) {
          const size_t o = static_cast<size_t>(t0 + key) * kvs + g * D + dim;
          if (split) {
            const size_t a = slot_base + static_cast<size_t>(key - k0) * D + dim;
            __hip_atomic_fetch_add(w.dk_acc + a, p.scale * dKacc[nt][i], __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_fetch_add(w.dv_acc + a, dVacc[nt][i], __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
          } else {
            dK[o] = f32_to_bf16(p.scale * dKacc[nt][i]);
            dV[o] = f32_to_bf16(dVacc[nt][i]);
          }
        }
      }
    }
  }
}


}  // namespace bwd128

bool bwd_mfma_supported(const Prefill& p) {
  return p.dtype == SINK_ATTN_BF16 && p.d == qm::D &&
         (p.blocks == nullptr || p.max_seqlen <= qm::MAX_BITMAP_WORDS * 32 * qm::BN);
}

int bwd_num_tiles(const Prefill& p) {
  const int nkt = (p.max_seqlen + qm::BN - 1) / qm::BN;
  return p.batch * nkt * p.hkv;
}

// A key tile splits when its iterations (query tiles or reverse-list entries
// seeing it, times the G query heads of its group) exceed item_iters(p), i.e.
// when more than cap = item_iters(p) / G query tiles see it.
int bwd_max_split_tiles(const Prefill& p) {
  const long long ntiles = bwd_num_tiles(p);
  const int nkt = (p.max_seqlen + qm::BN - 1) / qm::BN;
  const int G = p.hq / p.hkv;
  const long long cap = bwd128::item_iters(p) / G;
  long long bound = ntiles;
  if (p.blocks != nullptr) {
    // every reverse-list entry comes from one block_indices entry
    bound = static_cast<long long>(p.nqb) * p.hkv * p.max_blocks / (cap + 1);
  } else if (p.window > 0) {
    // a tile holding no kept first token is seen by at most (62 + W) / 64 + 1
    // query tiles; tiles holding kept tokens may split
    const long long per_head = (62LL + p.window) / qm::BN + 1;
    if (per_head <= cap) {
      const long long sink_tiles = std::min<long long>(nkt, (p.n_sink + qm::BN - 1) / qm::BN);
      bound = static_cast<long long>(p.batch) * p.hkv * sink_tiles;
    }
  } else {
    // causal: tile kt of a sample is seen by nqt - kt <= nkt - kt query tiles
    bound = static_cast<long long>(p.batch) * p.hkv * std::max<long long>(0, nkt - cap);
  }
  return static_cast<int>(std::min(ntiles, std::max(0LL, bound)));
}

hipError_t launch_scan(int32_t* off, int n, hipStream_t st);

hipError_t launch_bwd_dkdv_plan(const Prefill& p, const BwdWork& w, void* dk, void* dv, hipStream_t st) {
  if (p.total == 0 || p.batch == 0) return hipSuccess;
  const int nkt = (p.max_seqlen + qm::BN - 1) / qm::BN;
  const int ntiles = p.batch * nkt * p.hkv;
  if (ntiles <= 0) return hipSuccess;
  const int nq = bwd128::num_queues(p);
  uint16_t* dK = static_cast<uint16_t*>(dk);
  uint16_t* dV = static_cast<uint16_t*>(dv);
  hipLaunchKernelGGL(bwd128::plan_kernel, dim3((ntiles + 255) / 256), dim3(256), 0, st, p, w, nkt, nq);
  hipError_t e = launch_scan(w.split_slot, ntiles, st);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(bwd128::plan_clamp_kernel, dim3((ntiles + 255) / 256), dim3(256), 0, st, p, w, ntiles);
  e = launch_scan(w.plan, ntiles, st);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(bwd128::split_tiles_kernel<false>, dim3(ntiles), dim3(256), 0, st, p, w, nkt, nq,
                     dK, dV);
  return hipGetLastError();
}

hipError_t launch_bwd_dkdv(const Prefill& p, const void* q, const void* k, const void* v,
                           const void* dout, const BwdWork& w, void* dk, void* dv, hipStream_t st) {
  if (p.total == 0 || p.batch == 0) return hipSuccess;
  const int nkt = (p.max_seqlen + qm::BN - 1) / qm::BN;
  const int ntiles = p.batch * nkt * p.hkv;
  if (ntiles <= 0) return hipSuccess;
  const int nq = bwd128::num_queues(p);
  uint16_t* dK = static_cast<uint16_t*>(dk);
  uint16_t* dV = static_cast<uint16_t*>(dv);
  // Persistent: two 2-wavefront workgroups per CU, a multiple of the queues.
  hipLaunchKernelGGL(bwd128::dkdv_kernel, dim3(512), dim3(128), 0, st, p, nkt, nq,
                     static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                     static_cast<const uint16_t*>(v), static_cast<const uint16_t*>(dout), w, dK, dV);
  hipLaunchKernelGGL(bwd128::split_tiles_kernel<true>, dim3(ntiles), dim3(256), 0, st, p, w, nkt, nq,
                     dK, dV);
  return hipGetLastError();
}

}  // namespace sa
