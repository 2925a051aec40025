// Host check of the decode scan's tile bounds (scan_tiles.h): for every
// stream chunk count nc up to the host's bound cap, the launch gives every
// tile a workgroup and the workspace holds a total for every tile.
// Built with g++ by tests/test_scan_tiles.py; the header's __host__ /
// __device__ markers are defined away for the host compiler.
#define __host__
#define __device__
#include <cstdio>
#include <cstdint>
#include <vector>

#include "scan_tiles.h"

using namespace gpulz;

static int bad = 0;
static void check(uint64_t nc, uint64_t cap) {
  const uint32_t t = scan_tiles(nc), g = scan_groups(cap), w = workspace_tiles(cap);
  const uint32_t T = scan_tile_chunks(nc);
  const bool tiles_cover = (uint64_t)t * T >= nc && (t == 0 || (uint64_t)(t - 1) * T < nc);
  if (t > g || t > w || g == 0 || !tiles_cover || T % kTileMin != 0 || T < kTileMin || T > kTileMax ||
      (T & (T - 1u)) != 0 || (T < kTileMax && (uint64_t)T * kMaxTiles < nc)) {
    if (bad < 20) std::printf("nc=%llu cap=%llu tiles=%u groups=%u slots=%u T=%u\n", (unsigned long long)nc,
                              (unsigned long long)cap, t, g, w, T);
    ++bad;
  }
}

int main() {
  // exhaustive over small bounds
  for (uint64_t cap = 0; cap <= 70000; cap += (cap < 5000 ? 1 : 37))
    for (uint64_t nc = 0; nc <= cap; nc += (cap < 3000 ? 1 : 1 + nc / 64)) check(nc, cap);
  // around the tile-size boundaries: 64 tiles of 1024, tiles reaching 2^20
  // chunks, and the largest 32-bit chunk count
  std::vector<uint64_t> edges = {65535, 65536, 65537, 1ull << 26, (1ull << 26) - 1, (1ull << 26) + 1,
                                 (1ull << 26) + 1024, 0xFFFFFFFFull, 0xFFFFFFFEull, 1ull << 31, (1ull << 31) + 7};
  for (uint64_t cap : edges) {
    for (uint64_t nc : edges)
      if (nc <= cap) check(nc, cap);
    for (uint64_t d = 0; d < 5000; ++d) {
      if (d <= cap) check(cap - d, cap);
      check(d, cap);
      check(cap / 2 + d < cap ? cap / 2 + d : cap, cap);
    }
    for (uint64_t nc = 0; nc <= cap; nc += 1 + cap / 100000) check(nc, cap);
  }
  std::printf("%s (%d failures)\n", bad ? "FAIL" : "ok", bad);
  return bad ? 1 : 0;
}
