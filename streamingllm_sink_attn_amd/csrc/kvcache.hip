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

namespace sa {
namespace kvc {

constexpr float kE4m3Max = 448.f;

// One wavefront per (sequence b, chunk token c, KV head g): writes the K and
// V rows of the token to its slot, or nothing when a later token of the same
// chunk takes that slot (only the last `window` non-first tokens survive, so
// no slot gets two writers).
template <bool QUANT>
__global__ __launch_bounds__(64) void append_kernel(KvCache c, const uint16_t* __restrict__ k_new,
                                                    const uint16_t* __restrict__ v_new, int chunk,
                                                    const int32_t* __restrict__ n_seen) {
  const int g = blockIdx.x % c.hkv;
  const int tok = blockIdx.x / c.hkv;
  const int cc = tok % chunk;
  const int b = tok / chunk;
  const int lane = threadIdx.x;
  const int D = c.d;
  const long long p = static_cast<long long>(n_seen[b]) + cc;
  const long long total = static_cast<long long>(n_seen[b]) + chunk;
  if (p >= c.n_sink && p < total - c.window) return;      // evicted within this chunk
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
    for (int d = lane; d < D; d += 64) {
      dk[d] = k_new[src + d];
      dv[d] = v_new[src + d];
    }
    return;
  }

  // 8-bit ring row: amax over the row, then the codes.
  const size_t dst = ((static_cast<size_t>(b) * c.window + ring) * c.hkv + g) * D;
  const size_t sidx = (static_cast<size_t>(b) * c.hkv + g) * c.window + ring;
#pragma unroll
  for (int which = 0; which < 2; ++which) {
    const uint16_t* x = (which == 0 ? k_new : v_new) + src;
    float xv[4];
    float amax = 0.f;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int d = lane + 64 * r;
      xv[r] = d < D ? bf16_to_f32(x[d]) : 0.f;
      amax = fmaxf(amax, fabsf(xv[r]));
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off));
    const float scale = amax > 0.f ? amax / kE4m3Max : 0.f;
    const float inv = amax > 0.f ? kE4m3Max / amax : 0.f;
    uint8_t* out = (which == 0 ? c.win_k : c.win_v) + dst;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int d = lane + 64 * r;
      if (d < D) {
        const float v = xv[r] * inv;
        const int code = __builtin_amdgcn_cvt_pk_fp8_f32(v, 0.f, 0, false);
        out[d] = static_cast<uint8_t>(amax > 0.f ? (code & 0xff) : 0);
      }
    }
    if (lane == 0) (which == 0 ? c.win_k_scale : c.win_v_scale)[sidx] = scale;
  }
}

}  // namespace kvc

hipError_t launch_kvcache_append(const KvCache& c, const void* k_new, const void* v_new, int chunk,
                                 const int32_t* n_seen, hipStream_t st) {
  const long long rows = static_cast<long long>(c.batch) * chunk * c.hkv;
  if (rows <= 0) return hipSuccess;
  auto kern = c.quantized ? kvc::append_kernel<true> : kvc::append_kernel<false>;
  hipLaunchKernelGGL(kern, dim3(static_cast<unsigned>(rows)), dim3(64), 0, st, c,
                     static_cast<const uint16_t*>(k_new), static_cast<const uint16_t*>(v_new), chunk,
                     n_seen);
  return hipGetLastError();
}

}  // namespace sa
