// Host check of the key-row mapping of a chunked prefill read in place
// (streamingllm_sink_attn_amd/csrc/stream_rows.cuh), built with g++ against
// the HIP headers' host definitions.  For every (n_sink, window, chunk,
// n_seen) case below and every 64-row key tile of the stream:
//   * a tile read from one base (a run of the cache or of the chunk) yields,
//     row by row, the source the StreamingLLM cache layout defines (kept
//     first tokens in slots 0..n_sink-1; the token at position t >= n_sink in
//     ring slot n_sink + (t - n_sink) mod window; chunk row c after them) and
//     stays inside its array;
//   * a tile spanning a seam has a staging slot that the staging pass fills.
// Prints "cases N seam tiles M bad 0" and exits 0 when every check holds.
#include <algorithm>
#include <cstdio>
using std::max;
using std::min;
#include "stream_rows.cuh"

int main() {
  long bad = 0, cases = 0, seams = 0;
  for (int n_sink : {0, 1, 4, 64, 70})
    for (int window : {0, 1, 5, 63, 64, 65, 200, 1024})
      for (int chunk : {1, 7, 64, 150, 1024})
        for (int n_seen = -3; n_seen < n_sink + 3 * window + 130; n_seen += (n_seen < 300 ? 1 : 37)) {
          sa::StreamRows sr;
          sr.init(n_seen, n_sink, window, chunk);
          ++cases;
          // the tiles the staging pass copies, by slot
          int staged[sa::kSeamSlots];
          for (int i = 0; i < sa::kSeamSlots; ++i) {
            const int kt = sr.seam_tile(i);
            int unused;
            staged[i] = (kt >= 0 && sr.tile_kind(kt, &unused) == 2 && sr.seam_slot(kt) == i) ? kt : -1;
          }
          // the layout's own definition of each key row's source
          const int p0 = max(n_seen, 0);
          const int ns = min(p0, n_sink), nw = min(max(p0 - n_sink, 0), window);
          auto want = [&](int r, bool* cache) {
            if (r < ns) { *cache = true; return r; }
            if (r < ns + nw) {
              const int t = p0 - nw + (r - ns);          // the token's position
              *cache = true;
              return n_sink + (t - n_sink) % window;
            }
            *cache = false;
            return r - ns - nw;
          };
          if (sr.L != ns + nw + chunk) ++bad;
          for (int kt = 0; kt * sa::kSeamRows < sr.L; ++kt) {
            int row;
            const int kind = sr.tile_kind(kt, &row);
            if (kind == 2) {
              ++seams;
              if (staged[sr.seam_slot(kt)] != kt) ++bad;
              continue;
            }
            for (int r = kt * sa::kSeamRows; r < min(kt * sa::kSeamRows + sa::kSeamRows, sr.L); ++r) {
              bool wc;
              const int w = want(r, &wc);
              const int got = row + (r - kt * sa::kSeamRows);
              const bool gc = kind == 1;
              const int lim = gc ? n_sink + window : chunk;
              if (wc != gc || w != got || got < 0 || got >= lim) ++bad;
              int via;
              const bool vc = sr.source(r, &via);
              if (vc != wc || via != w) ++bad;
            }
          }
        }
  std::printf("cases %ld seam tiles %ld bad %ld\n", cases, seams, bad);
  return bad != 0;
}
