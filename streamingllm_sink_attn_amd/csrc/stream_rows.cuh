// Key rows of a chunked prefill against a rolling cache, read in place.
//
// StreamingLLM keeps a stream's first tokens and a rolling window of its
// most recent ones ("What is Attention Sink? ... StreamingLLM", core idea).
// Stream b's keys in position order are
//   [kept first tokens | ring tokens, oldest first | new chunk]
// and key row r of the stream lives in:
//   r < ns               cache slot r (a kept first token);
//   ns <= r < ns + nw    cache slot n_sink + (rf + r - ns) mod window (ring);
//   r >= ns + nw         chunk row r - ns - nw.
// A 64-row key tile inside one contiguous run (first tokens, ring rows on
// one side of the wrap, chunk rows) is read where it lies, from a per-tile
// base.  A tile holding a seam (where first tokens meet the ring or the
// chunk, the ring's wrap, where the ring meets the chunk) is copied
// beforehand into a staging tile of the stream: seam kind i (0 first tokens
// end, 1 ring wrap, 2 chunk start) owns staging slot i, and a tile holding
// several seams uses the lowest slot among them.
#pragma once

#include "internal.h"   // kSeamSlots, kSeamRows

namespace sa {

struct StreamRows {
  int ns, nw, rf, L;           // first tokens, ring tokens, oldest ring slot, key rows
  int n_sink, window;

  __device__ __forceinline__ void init(int n_seen, int n_sink_, int window_, int chunk) {
    n_sink = n_sink_;
    window = window_;
    const int p0 = n_seen > 0 ? n_seen : 0;          // a negative count reads as an empty stream
    ns = min(p0, n_sink);
    nw = min(max(p0 - n_sink, 0), window);
    rf = nw > 0 ? (p0 - nw - n_sink) % window : 0;
    L = ns + nw + chunk;
  }

  // Row r's source: true and the cache slot, or false and the chunk row.
  __device__ __forceinline__ bool source(int r, int* row) const {
    if (r < ns) {
      *row = r;
      return true;
    }
    if (r < ns + nw) {
      int x = rf + (r - ns);
      if (x >= window) x -= window;
      *row = n_sink + x;
      return true;
    }
    *row = r - ns - nw;
    return false;
  }

  // Tile kt, rows [64 kt, min(64 kt + 64, L)): 0 chunk rows from chunk row
  // *row on, 1 cache rows from slot *row on, or 2 a seam.
  __device__ __forceinline__ int tile_kind(int kt, int* row) const {
    const int k0 = kt * kSeamRows;
    const int last = min(k0 + kSeamRows, L) - 1;
    const int wend = ns + nw;
    *row = 0;
    if (k0 >= wend) {
      *row = k0 - wend;
      return 0;
    }
    if (last < ns) {
      *row = k0;
      return 1;
    }
    if (k0 >= ns && last < wend) {
      const int x0 = rf + (k0 - ns), x1 = rf + (last - ns);   // both below 2 window
      if (x1 < window) {
        *row = n_sink + x0;
        return 1;
      }
      if (x0 >= window) {
        *row = n_sink + x0 - window;
        return 1;
      }
    }
    return 2;
  }

  // The tile of seam kind i, or -1 where the stream has no such seam.
  __device__ __forceinline__ int seam_tile(int i) const {
    int r = -1;
    if (i == 0 && ns > 0 && ns < L) r = ns;
    if (i == 1 && rf > 0 && window - rf < nw) r = ns + window - rf;
    if (i == 2 && ns + nw > 0 && ns + nw < L) r = ns + nw;
    return r < 0 ? -1 : r / kSeamRows;
  }

  // Staging slot of a seam tile (tile_kind 2): the lowest seam kind in it.
  __device__ __forceinline__ int seam_slot(int kt) const {
    if (seam_tile(0) == kt) return 0;
    if (seam_tile(1) == kt) return 1;
    return 2;
  }
};

}  // namespace sa
