// Query-major machinery shared by the forward and the dQ kernels (bf16,
// head_dim 128): workgroup geometry, the key-tile schedule of a group of
// query rows, per-wavefront tile classification, direct-to-LDS tile loads and
// the MFMA fragment readers.
#pragma once

#include "common.cuh"

namespace sa {
namespace qm {

constexpr int D = 128;
constexpr int BN = 64;                 // keys per tile (= block size of block lists)
constexpr int TILE = BN * D;           // bf16 elements of one staged K or V tile (16 KB)
constexpr int MAX_BITMAP_WORDS = 256;  // block lists: up to 8192 KV blocks per sample

typedef short i16x4 __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------------------
// Geometry: a workgroup holds nw wavefronts of qw query rows each, all of one
// KV head g.  With G = Hq/Hkv query heads per KV head, up to nw of them share
// the workgroup (GQA packing: every staged K/V tile feeds nw x qw query
// rows); when G has fewer factors of two, the wavefronts of a head take
// consecutive qw-row slabs.  The forward and dQ kernels use nw = 8, qw = 32.
// ---------------------------------------------------------------------------
struct Geo {
  int hw;       // query heads per workgroup
  int wph;      // wavefronts per head
  int P;        // query positions per workgroup
  int nptiles;  // position tiles per sample (from max_seqlen)
  int nhg;      // head groups per KV head
  int Z;        // hkv * nhg
};

// nw wavefronts of qw rows each (nw a power of two, qw dividing 64).
inline Geo make_geo(const Prefill& p, int nw, int qw) {
  Geo g;
  const int G = p.hq / p.hkv;
  g.hw = 1;
  while (g.hw * 2 <= nw && G % (g.hw * 2) == 0) g.hw *= 2;
  g.wph = nw / g.hw;
  g.P = qw * g.wph;
  g.nptiles = (p.max_seqlen + g.P - 1) / g.P;
  g.nhg = G / g.hw;
  g.Z = p.hkv * g.nhg;
  return g;
}

// Flat block id -> coordinates: sample slowest, then position tiles heaviest
// (latest) first, then (head group, KV head) fastest, KV head fastest of all.
// Consecutive ids go to the XCDs round-robin, so with Hkv a multiple of 8
// every XCD serves fixed KV heads, all head groups of a KV head on the same
// XCD, and working one sample at a time keeps that sample's K/V slice of each
// KV head resident in the XCD's L2.
struct WgCoord {
  int pt, b, g, hg;
};
__device__ __forceinline__ WgCoord wg_coord(const Geo& geo, int batch, int bid) {
  WgCoord c;
  const int per_b = geo.nptiles * geo.Z;
  c.b = bid / per_b;
  const int rem = bid % per_b;
  c.pt = geo.nptiles - 1 - rem / geo.Z;
  const int z = rem % geo.Z;
  const int hkv = geo.Z / geo.nhg;
  c.g = z % hkv;
  c.hg = z / hkv;
  (void)batch;
  return c;
}

// Block lists: one bitmap per query block of the workgroup (at most
// MAX_QB_PER_WG; a workgroup's rows start on a block boundary), bit kb of row
// j set when query block qb0 + j selects KV block kb (kb <= qb only).  Built
// in LDS once, so classifying a tile inside the loop reads no global memory.
constexpr int MAX_QB_PER_WG = 4;
constexpr int BITMAP_LDS_WORDS = MAX_QB_PER_WG * MAX_BITMAP_WORDS;

// The workgroup's key-tile schedule: ranges without block lists, else the
// union of the query blocks' bitmaps.
struct Sched {
  bool blk;
  TileRanges tr;
  int n;
  int word, nwords, nrows;
  uint32_t bits;
  const uint32_t* bm;
  __device__ __forceinline__ int next() {
    if (!blk) return n < tr.count() ? tr.at(n++) : -1;
    while (bits == 0) {
      if (++word >= nwords) return -1;
      uint32_t u = 0u;
      for (int j = 0; j < nrows; ++j) u |= bm[j * MAX_BITMAP_WORDS + word];
      bits = u;
    }
    const int kb = word * 32 + __builtin_ctz(bits);
    bits &= bits - 1;
    return kb;
  }
};

// Bitmaps of the query blocks in [p0, p1) (p0 a multiple of BN).  Every
// thread of the workgroup must call it.
__device__ __forceinline__ void build_block_bitmaps(const Prefill& p, int L, int qoff, int g, int p0,
                                                    int p1, uint32_t* bm, int* nwords_out,
                                                    int* nrows_out) {
  const int nkb = (L + BN - 1) / BN;
  const int nwords = min((nkb + 31) / 32, MAX_BITMAP_WORDS);
  const int qb0 = p0 / BN, qb1 = (p1 - 1) / BN;
  const int nrows = min(qb1 - qb0 + 1, MAX_QB_PER_WG);
  for (int i = threadIdx.x; i < nrows * nwords; i += blockDim.x)
    bm[(i / nwords) * MAX_BITMAP_WORDS + i % nwords] = 0u;
  __syncthreads();
  const int total = nrows * p.max_blocks;
  for (int idx = threadIdx.x; idx < total; idx += blockDim.x) {
    const int j = idx / p.max_blocks;
    const int e = idx % p.max_blocks;
    const int qb = qb0 + j;
    const int kb = p.blocks[(static_cast<size_t>(qoff + qb) * p.hkv + g) * p.max_blocks + e];
    if (kb >= 0 && kb <= qb && (kb >> 5) < nwords)
      atomicOr(&bm[j * MAX_BITMAP_WORDS + (kb >> 5)], 1u << (kb & 31));
  }
  __syncthreads();
  *nwords_out = nwords;
  *nrows_out = nrows;
}

// bm holds BITMAP_LDS_WORDS words of LDS.
__device__ __forceinline__ Sched make_sched(const Prefill& p, int L, int qoff, int g, int p0, int p1,
                                            uint32_t* bm) {
  Sched sc;
  sc.blk = p.blocks != nullptr;
  sc.n = 0;
  sc.word = -1;
  sc.bits = 0u;
  sc.bm = bm;
  sc.nwords = 0;
  sc.nrows = 0;
  if (sc.blk) build_block_bitmaps(p, L, qoff, g, p0, p1, bm, &sc.nwords, &sc.nrows);
  else sc.tr = window_tiles(p0, p1, p.n_sink, p.window, BN);
  return sc;
}

// Class of key tile kt for a wavefront's rows [wq0, wq1) (inside one query
// block; p0 the workgroup's first row): 0 empty, 1 full, 2 mixed.  With block
// lists the wavefront's own query block must select the tile.
__device__ __forceinline__ int wave_tile_class(const Prefill& p, const Sched& sc, int p0, int wq0,
                                               int wq1, int kt) {
  if (wq0 >= wq1) return 0;
  int cls = classify_tile(wq0, wq1, kt * BN, BN, p.n_sink, p.window);
  if (cls != 0 && sc.blk) {
    const int j = wq0 / BN - p0 / BN;
    if (((sc.bm[j * MAX_BITMAP_WORDS + (kt >> 5)] >> (kt & 31)) & 1u) == 0u) cls = 0;
  }
  return cls;
}

// ---------------------------------------------------------------------------
// Staged tiles: 64 rows of 256 bytes, 16-byte chunks XOR-swizzled per row so
// that (a) 8 consecutive rows at one logical chunk hit distinct banks (the
// MFMA row-fragment reads) and (b) the 4 rows x 4 chunks of one transposed
// read spread over distinct banks.
// ---------------------------------------------------------------------------
__device__ __forceinline__ int swz16(int row) {
  const int r = row & 15;
  return ((r & 3) << 2) | ((r >> 2) & 3);
}
// Element offset of (row, logical chunk lc).
__device__ __forceinline__ int at16(int row, int lc) { return row * D + ((lc ^ swz16(row)) << 3); }

// ---------------------------------------------------------------------------
// Direct-to-LDS buffer loads issued from asm blocks.  With the compiler's own
// LDS-DMA intrinsics it cannot tell which LDS bytes a load fills, so it waits
// for every such load before the wavefront's next LDS read; a tile prefetched
// for the next iteration would then be waited for before the current one is
// computed.  Issued from asm the loads stay in flight until the caller waits
// for them (s_waitcnt vmcnt) and passes a barrier (wait_bar, which also waits
// for the wavefront's own LDS reads so no read of a buffer is in flight when
// it is refilled).  The compiler counts only its own vector memory
// operations: loops that use these loads must issue no other vector memory
// operation between issue and wait, and operands loaded before them are
// consumed (or waited for) before the first one is issued.
// ---------------------------------------------------------------------------
constexpr uint32_t kBufferWord3 = 0x00020000u;   // raw buffer, 32-bit data format

__device__ __forceinline__ u32x4 make_rsrc(const void* base, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  u32x4 r;
  r[0] = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(a));
  r[1] = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(a >> 32) & 0xffffu);   // stride 0
  r[2] = __builtin_amdgcn_readfirstlane(bytes);
  r[3] = kBufferWord3;
  return r;
}
// One direct-to-LDS load: lane bytes (16 or 4) go to LDS m0 + lane * size.
// An M0 write needs one wait state before an LDS DMA reads it.
__device__ __forceinline__ void dma16(const u32x4& rsrc, uint32_t voff, uint32_t lds_addr) {
  lds_addr = __builtin_amdgcn_readfirstlane(lds_addr);    // wave-uniform
  uint32_t keep;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %1\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %2, %3, 0 offen lds\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(keep)
      : "s"(lds_addr), "v"(voff), "s"(rsrc)
      : "memory");
}
__device__ __forceinline__ void dma4(const u32x4& rsrc, uint32_t voff, uint32_t lds_addr) {
  lds_addr = __builtin_amdgcn_readfirstlane(lds_addr);    // wave-uniform
  uint32_t keep;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %1\n\t"
      "s_nop 0\n\t"
      "buffer_load_dword %2, %3, 0 offen lds\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(keep)
      : "s"(lds_addr), "v"(voff), "s"(rsrc)
      : "memory");
}
// Waits until at most N of this wavefront's vector memory operations are in
// flight, then for its LDS reads, then passes the workgroup barrier.
template <int N>
__device__ __forceinline__ void wait_bar() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(N) : "memory");
}

// LDS byte address of a __shared__ object.
__device__ __forceinline__ uint32_t lds_address(const void* p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>(
      (__attribute__((address_space(3))) const char*)(p)));
}

// 64-row tiles into swizzled LDS with dma16: wavefront wv of NWV owns the
// 4-row blocks PER*wv .. PER*wv + PER - 1; per-lane offsets inside a full tile
// are computed once, a ragged tile reads its last row in place of the
// missing ones (finite data that the mask discards).
template <int NWV>
struct DmaTiles {
  static constexpr int PER = 16 / NWV;
  uint32_t off[PER];
  int wv, lane, stride;
  __device__ __forceinline__ void init(int wv_, int lane_, int row_stride) {
    wv = wv_;
    lane = lane_;
    stride = row_stride;
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      const int row = 4 * (wv * PER + j) + (lane >> 4);
      const int lc = (lane & 15) ^ swz16(row);
      off[j] = static_cast<uint32_t>(row * row_stride + lc * 8) * 2u;
    }
  }
  __device__ __forceinline__ void load(const uint16_t* base, int nvalid, uint32_t lds_tile) const {
    const int rows = nvalid < BN ? nvalid : BN;
    const u32x4 rsrc = make_rsrc(base, static_cast<uint32_t>(rows * stride * 2));
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      uint32_t o = off[j];
      if (rows < BN) {
        const int row = 4 * (wv * PER + j) + (lane >> 4);
        const int lc = (lane & 15) ^ swz16(row);
        o = static_cast<uint32_t>(min(row, rows - 1) * stride + lc * 8) * 2u;
      }
      dma16(rsrc, o, lds_tile + static_cast<uint32_t>(4 * (wv * PER + j) * D) * 2u);
    }
  }
};

// 16-byte row fragment (8 consecutive dims of one row) of a staged tile.
__device__ __forceinline__ bf16x8 row_frag(const uint16_t* tile, int row, int lc) {
  return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(tile + at16(row, lc)));
}

__device__ __forceinline__ u32x2 ds_read_tr(const uint16_t* lds_ptr) {
  i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) i16x4*)(const_cast<uint16_t*>(lds_ptr)));
  return __builtin_bit_cast(u32x2, v);
}

// Transposed 32x32x16 operand fragment of a staged tile: lane (column
// 16*(grp%2) + i of a 32-wide dim block starting at dim0, k-half grp/2) gets
// dims dim0 + 16*(grp%2) + i of rows rbase + 4*(grp/2) + {0..3} and
// rbase + 8 + 4*(grp/2) + {0..3}.  With ds_read_b64_tr_b16, source lane
// 4r + q of each 16-lane group reads 4 dims of row r, and the hardware hands
// lane i the value of dim i in each of the 4 rows.
__device__ __forceinline__ bf16x8 tr_frag(const uint16_t* tile, int rbase, int dim0, int lane) {
  const int l16 = lane & 15, grp = lane >> 4;
  const int r = l16 >> 2, q4 = l16 & 3;
  const int d = dim0 + 16 * (grp & 1) + 4 * q4;
  const int lc = d >> 3, off = d & 7;
  const int ra = rbase + 4 * (grp >> 1) + r;
  const int rb = ra + 8;
  const u32x2 a = ds_read_tr(tile + at16(ra, lc) + off);
  const u32x2 b = ds_read_tr(tile + at16(rb, lc) + off);
  return __builtin_bit_cast(bf16x8, u32x4{a[0], a[1], b[0], b[1]});
}

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2 v = {static_cast<__bf16>(lo), static_cast<__bf16>(hi)};
  return __builtin_bit_cast(uint32_t, v);
}

// k-step cc (16 keys) of a 64-key contraction as a B (or A) operand from two
// 32x32 result tiles: elements (cc%2)*8 .. +8 of tile cc/2.  Logical k slot t
// of lane half gq is key 16cc + 8(t/4) + 4gq + t%4, which matches tr_frag
// with rbase = 16cc.
__device__ __forceinline__ bf16x8 pack_kstep(const f32x16& t, int half) {
  u32x4 u;
#pragma unroll
  for (int e = 0; e < 4; ++e) u[e] = pack_bf16x2(t[half * 8 + 2 * e], t[half * 8 + 2 * e + 1]);
  return __builtin_bit_cast(bf16x8, u);
}

}  // namespace qm
}  // namespace sa
