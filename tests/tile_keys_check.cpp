// Host check of the score kernel's tile sizes (tests/test_tile_keys_host.py builds
// and runs it on the CPU).  For every n_max (a multiple of 16 up to the longest row
// the score kernel takes) and every query-head group size:
//   * each tile size is a multiple of 256 keys (a wave takes a quarter of a tile in
//     64-key stages) and at most its cap;
//   * the single-buffer mode's tiles (tria_score picks them at run time) are never
//     more per row than the tiles the workspace is sized for (score_tile_keys): the
//     tile moments of that mode must fit in the workspace's moment array.
#include "tria_kernels.h"

#include <cstdio>

namespace {

int fails = 0;

void expect(bool ok, const char* what, int n, int g, int tile) {
  if (!ok && fails++ < 20) std::printf("FAIL %s: n_max %d, G %d, tile %d\n", what, n, g, tile);
}

void check_tile(int tile, int cap, int n, int g, const char* what) {
  expect(tile % 256 == 0, what, n, g, tile);
  expect(tile > 0 && tile <= cap, what, n, g, tile);
}

}  // namespace

int main() {
  const int n_hi = 1 << 20;
  long cases = 0;
  for (int n = 16; n <= n_hi; n += 16) {
    for (int g = 1; g <= tria::kMaxGroup; ++g) {
      for (int omax = 0; omax < 2; ++omax) {
        const int t = tria::score_tile_keys(g, omax, n);
        check_tile(t, g <= 4 && !omax ? TRIA_SCORE_TILE_SMALL_G : TRIA_SCORE_TILE_LARGE_G, n, g, "score_tile_keys");
        ++cases;
      }
      const int t = tria::score_tile_keys(g, 0, n);
      const int t1 = tria::single_tile_keys(n);
      check_tile(t1, TRIA_SCORE_TILE_SMALL_G, n, g, "single_tile_keys");
      expect((n + t1 - 1) / t1 <= (n + t - 1) / t, "single-buffer tiles within the workspace's count", n, g, t1);
    }
  }
  std::printf("%ld cases, %d failures\n", cases, fails);
  if (fails) return 1;
  std::printf("ok\n");
  return 0;
}
