// compact.hip -- chunk-size scan and stream assembly for gfx950.
//
// The encode kernel leaves every chunk's payload in a fixed-stride staging
// slot and its 8-byte size-table entry in a workspace array.  Chunk offsets
// are the exclusive scan of the payload sizes (GPULZStage page, CUDA-graph
// paragraph: the inverse derives them from the size table, so they are not
// stored).  Three passes over the sizes and one over the payload bytes:
//   tile_sums:     per tile of kTile chunks, the sum of payload sizes;
//   scan_tiles:    one workgroup, exclusive scan of the tile sums; writes the
//                  32-byte header and the stream length;
//   chunk_offsets: per tile, offsets of its chunks + the size-table rows;
//   copy_payloads: one wave per chunk, staging -> stream at any byte offset
//                  (interior dwords aligned by a funnel shift, edges as bytes).
// Launch shapes depend only on the chunk count.
#include "common.h"

namespace gpulz {
namespace {

__device__ __forceinline__ void put_bytes_le(uint8_t* p, uint64_t v, int nbytes) {
  for (int i = 0; i < nbytes; ++i) p[i] = (uint8_t)(v >> (8 * i));
}

__global__ __launch_bounds__(kBlock) void tile_sums_kernel(const uint2* __restrict__ entries,
                                                           uint32_t num_chunks,
                                                           uint64_t* __restrict__ tile_sums) {
  __shared__ uint64_t sh[kWaves];
  const uint64_t t = blockIdx.x;
  uint64_t s = 0;
  for (uint32_t i = threadIdx.x; i < kTile; i += kBlock) {
    const uint64_t c = t * kTile + i;
    if (c < num_chunks) {
      const uint2 e = entries[c];
      s += entry_payload(e.x, e.y);
    }
  }
  s = block_sum(s, sh);
  if (threadIdx.x == 0) tile_sums[t] = s;
}

// Exclusive scan of the tile sums in place (one workgroup); header + length.
__global__ __launch_bounds__(kBlock) void scan_tiles_kernel(uint64_t* __restrict__ tile_sums,
                                                            uint32_t num_tiles, uint8_t* __restrict__ out,
                                                            uint64_t* __restrict__ out_bytes, uint64_t n,
                                                            uint32_t cs, uint32_t ws, uint32_t num_chunks) {
  __shared__ uint64_t sh[kWaves];
  uint64_t carry = 0;
  for (uint32_t b = 0; b < num_tiles; b += kBlock) {
    const uint32_t i = b + threadIdx.x;
    const uint64_t v = i < num_tiles ? tile_sums[i] : 0;
    uint64_t tot;
    const uint64_t ex = block_exclusive_scan(v, &tot, sh);
    if (i < num_tiles) tile_sums[i] = carry + ex;
    carry += tot;
  }
  if (threadIdx.x == 0) {
    put_bytes_le(out + 0, kMagic, 4);
    out[4] = (uint8_t)kVersion;
    out[5] = (uint8_t)ws;
    out[6] = 0;
    out[7] = 0;
    put_bytes_le(out + 8, cs, 4);
    put_bytes_le(out + 12, num_chunks, 4);
    put_bytes_le(out + 16, n, 8);
    put_bytes_le(out + 24, carry, 8);
    *out_bytes = (uint64_t)kHeaderBytes + (uint64_t)kEntryBytes * num_chunks + carry;
  }
}

__global__ __launch_bounds__(kBlock) void chunk_offsets_kernel(const uint2* __restrict__ entries,
                                                               uint32_t num_chunks,
                                                               const uint64_t* __restrict__ tile_prefix,
                                                               uint64_t* __restrict__ offsets,
                                                               uint8_t* __restrict__ out) {
  __shared__ uint64_t sh[kWaves];
  constexpr uint32_t PER = kTile / kBlock;
  const uint64_t t = blockIdx.x;
  const uint64_t c0 = t * kTile + (uint64_t)threadIdx.x * PER;
  uint2 e[PER];
  uint64_t local = 0;
#pragma unroll
  for (uint32_t j = 0; j < PER; ++j) {
    e[j] = (c0 + j < num_chunks) ? entries[c0 + j] : make_uint2(0u, 0u);
    local += entry_payload(e[j].x, e[j].y);
  }
  uint64_t tot;
  uint64_t off = tile_prefix[t] + block_exclusive_scan(local, &tot, sh);
  uint8_t* table = out + kHeaderBytes;
  const bool al8 = (((uintptr_t)table) & 7u) == 0;
#pragma unroll
  for (uint32_t j = 0; j < PER; ++j) {
    const uint64_t c = c0 + j;
    if (c >= num_chunks) break;
    offsets[c] = off;
    off += entry_payload(e[j].x, e[j].y);
    uint8_t* row = table + kEntryBytes * c;
    if (al8) {
      *(uint2*)row = e[j];
    } else {
      put_bytes_le(row, e[j].x, 4);
      put_bytes_le(row + 4, e[j].y, 4);
    }
  }
}

// One wave copies one chunk's payload from its 4-aligned staging slot to an
// arbitrary byte offset of the stream.
__global__ __launch_bounds__(kBlock) void copy_payloads_kernel(const uint8_t* __restrict__ staging,
                                                               const uint2* __restrict__ entries,
                                                               const uint64_t* __restrict__ offsets,
                                                               uint32_t num_chunks, uint32_t cs,
                                                               uint8_t* __restrict__ payload_base) {
  const uint32_t lane = threadIdx.x & 63u;
  const uint64_t c = (uint64_t)blockIdx.x * kWaves + (threadIdx.x >> 6);
  if (c >= num_chunks) return;
  const uint2 e = entries[c];
  const uint32_t sz = entry_payload(e.x, e.y);
  if (sz == 0) return;
  const uint32_t* sw = (const uint32_t*)(staging + c * cs);
  const uint8_t* sb = (const uint8_t*)sw;
  uint8_t* dst = payload_base + offsets[c];
  uint32_t head = (uint32_t)((4u - ((uintptr_t)dst & 3u)) & 3u);
  if (head > sz) head = sz;
  if (lane < head) dst[lane] = sb[lane];
  const uint32_t nbody = (sz - head) / 4u;
  uint32_t* dw = (uint32_t*)(dst + head);
  const uint32_t sh = head & 3u;
  for (uint32_t j = lane; j < nbody; j += 64u) {
    const uint32_t s = head + 4u * j;  // source byte of this destination word
    const uint32_t lo = sw[s >> 2];
    const uint32_t hi = sh ? sw[(s >> 2) + 1u] : 0u;
    dw[j] = __builtin_amdgcn_alignbyte(hi, lo, sh);
  }
  const uint32_t tail0 = head + 4u * nbody;
  if (tail0 + lane < sz) dst[tail0 + lane] = sb[tail0 + lane];
}

}  // namespace

hipError_t launch_compact(const CompactArgs& a, hipStream_t stream) {
  if (a.num_chunks > 0) {
    hipLaunchKernelGGL(tile_sums_kernel, dim3(a.num_tiles), dim3(kBlock), 0, stream, a.entries, a.num_chunks,
                       a.tile_sums);
  }
  hipLaunchKernelGGL(scan_tiles_kernel, dim3(1), dim3(kBlock), 0, stream, a.tile_sums, a.num_tiles, a.out,
                     a.out_bytes, a.n, a.cs, a.ws, a.num_chunks);
  if (a.num_chunks > 0) {
    hipLaunchKernelGGL(chunk_offsets_kernel, dim3(a.num_tiles), dim3(kBlock), 0, stream, a.entries,
                       a.num_chunks, (const uint64_t*)a.tile_sums, a.offsets, a.out);
    const uint32_t grid = (a.num_chunks + kWaves - 1) / kWaves;
    hipLaunchKernelGGL(copy_payloads_kernel, dim3(grid), dim3(kBlock), 0, stream, a.staging, a.entries,
                       (const uint64_t*)a.offsets, a.num_chunks, a.cs,
                       a.out + kHeaderBytes + (uint64_t)kEntryBytes * a.num_chunks);
  }
  return hipGetLastError();
}

}  // namespace gpulz
