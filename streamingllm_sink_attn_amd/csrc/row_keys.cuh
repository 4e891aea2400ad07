// Enumerates the valid keys of one query row (generic kernels).
#pragma once

#include "common.cuh"

namespace sa {

// Calls f(j) for every sample-local key j valid for query row i of sample b
// and KV head g: causal order, the kept first tokens plus the recent window,
// and the selected blocks (each distinct block id once).  Wave-uniform.
template <typename F>
__device__ __forceinline__ void for_each_valid_key(const Prefill& p, int b, int i, int g, F&& f) {
  if (p.blocks == nullptr) {
    if (p.window <= 0) {
      for (int j = 0; j <= i; ++j) f(j);
    } else {
      const int s_end = min(p.n_sink, i + 1);
      for (int j = 0; j < s_end; ++j) f(j);
      const int w0 = max(s_end, i - p.window + 1);
      for (int j = w0; j <= i; ++j) f(j);
    }
    return;
  }
  const int qb = i / kBlock;
  const int32_t* row =
      p.blocks + (static_cast<size_t>(q_block_offset(p.cu, b) + qb) * p.hkv + g) * p.max_blocks;
  for (int e = 0; e < p.max_blocks; ++e) {
    const int kb = row[e];
    if (kb < 0 || kb > qb || !first_occurrence(row, e)) continue;
    const int j1 = min(kb * kBlock + kBlock, i + 1);
    for (int j = kb * kBlock; j < j1; ++j)
      if (key_visible(i, j, p.n_sink, p.window)) f(j);
  }
}

}  // namespace sa
