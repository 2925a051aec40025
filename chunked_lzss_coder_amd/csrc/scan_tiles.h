// scan_tiles.h -- tile geometry of the decode-side size-table scan.
//
// The scan kernel cuts a stream's size table into tiles of T chunks (one
// workgroup per tile) and sizes T on the device from the header's chunk count
// nc; the host only knows a bound chunks_cap >= nc (from the stream and
// output sizes).  Memory safety rests on two facts for every nc <= chunks_cap:
//   tiles(nc) <= scan_groups(chunks_cap)   (every tile gets a workgroup), and
//   tiles(nc) <= workspace_tiles(chunks_cap)  (every tile has a total slot).
// Plain integer functions, shared by the host launcher and the kernels.
#pragma once

#include <stdint.h>

namespace gpulz {

constexpr uint32_t kTileMin = 1024;      // chunks per scan tile: at least,
constexpr uint32_t kTileMax = 1u << 20;  // at most (offsets within a tile < 2^32)
constexpr uint32_t kMaxTiles = 64;       // tiles wanted (one tile total per lane)
constexpr uint32_t kWorkspaceTilesMin = 256;

// Chunks per scan tile for a stream of nc chunks: the smallest power of two
// from kTileMin up to kTileMax with nc <= kMaxTiles * T (kTileMax if none), so
// a chunk's tile is its index shifted right.
__host__ __device__ inline uint32_t scan_tile_chunks(uint64_t nc) {
  uint64_t T = kTileMin;
  while (T < kTileMax && T * kMaxTiles < nc) T <<= 1;
  return (uint32_t)T;
}

// Tiles of a stream of nc chunks (0 for an empty stream).
__host__ __device__ inline uint32_t scan_tiles(uint64_t nc) {
  const uint32_t T = scan_tile_chunks(nc);
  return (uint32_t)((nc + T - 1u) / T);
}

// Scan workgroups launched for any stream of at most chunks_cap chunks.  For
// nc <= chunks_cap: either nc's tiles hold kTileMax chunks, and then so do
// chunks_cap's, which are as many or more; or nc has at most kMaxTiles tiles
// and at most one per kTileMin chunks.  At least one workgroup (it writes the
// header status).
__host__ __device__ inline uint32_t scan_groups(uint64_t chunks_cap) {
  const uint64_t by_min = (chunks_cap + kTileMin - 1u) / kTileMin;
  const uint32_t small = by_min < kMaxTiles ? (uint32_t)by_min : kMaxTiles;
  const uint32_t nt = scan_tiles(chunks_cap);
  const uint32_t g = nt > small ? nt : small;
  return g ? g : 1u;
}

// Tile-total and tile-error slots the decode workspace holds for chunks_cap.
__host__ __device__ inline uint32_t workspace_tiles(uint64_t chunks_cap) {
  const uint32_t nt = scan_tiles(chunks_cap);
  return nt > kWorkspaceTilesMin ? nt : kWorkspaceTilesMin;
}

}  // namespace gpulz
