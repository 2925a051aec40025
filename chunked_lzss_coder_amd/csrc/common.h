// common.h -- internal constants, device helpers and launcher declarations of
// the gfx950 chunked LZSS coder.  Stream format: see include/gpulz.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gpulz {

// ---- stream format ------------------------------------------------------
constexpr uint32_t kMagic = 0x315A4C47u;  // "GLZ1"
constexpr uint32_t kVersion = 1u;
constexpr uint32_t kSplitVersion = 2u;  // split mode: four ports, meta carries the header
constexpr uint32_t kHeaderBytes = 32u;
constexpr uint32_t kEntryBytes = 8u;
constexpr uint32_t kRawBit = 0x80000000u;

// ---- method constants (GPULZStage page) ---------------------------------
constexpr uint32_t kWindow = 32u;     // near window: offsets 1..32 (window paragraph)
constexpr uint32_t kMaxLen = 255u;    // one-byte length field (long-match paragraph)
constexpr uint32_t kMaxFar = 255u;    // one-byte offset field: level-1 reach (level table)
constexpr uint32_t kSubBlocks = 8u;   // level-1 sub-block walk (hashed-table paragraph)
constexpr uint32_t kHashBits = 11u;   // table size: not on the pages; 2048 buckets
constexpr uint32_t kHashSize = 1u << kHashBits;

// ---- launch geometry ----------------------------------------------------
constexpr int kBlock = 256;           // threads per workgroup (4 wave64)
constexpr int kWaves = kBlock / 64;

// Status codes mirrored from the public header.
constexpr uint32_t kStatusOk = 0u;
constexpr uint32_t kStatusCapacity = 2u;
constexpr uint32_t kStatusCorrupt = 3u;

__host__ __device__ inline bool chunk_size_ok(uint32_t cs) {
  return cs == 1024u || cs == 2048u || cs == 4096u;
}
__host__ __device__ inline bool word_size_ok(uint32_t ws) {
  return ws == 1u || ws == 2u || ws == 4u;
}

// Payload bytes a size-table entry stands for.
__host__ __device__ inline uint32_t entry_payload(uint32_t f, uint32_t d) {
  return f != 0u ? f + d : ((d & kRawBit) ? (d & ~kRawBit) : 0u);
}

// Level-1 bucket of the two-word key (w0, w1): Fibonacci multiplicative hash
// of the 64-bit key w0 | w1<<32, top kHashBits bits.  The pages give no hash
// function; this choice only affects which candidates the encoder sees.
__device__ __forceinline__ uint32_t bucket_of(uint32_t w0, uint32_t w1) {
  uint64_t key = (uint64_t)w0 | ((uint64_t)w1 << 32);
  return (uint32_t)((key * 0x9E3779B97F4A7C15ull) >> (64u - kHashBits));
}

// ---- block-wide helpers (blockDim.x == kBlock) ---------------------------
// Exclusive scan of one value per thread.  `sh` needs kWaves elements of T.
template <typename T>
__device__ __forceinline__ T block_exclusive_scan(T v, T* total, T* sh) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  T inc = v;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    T nb = __shfl_up(inc, d, 64);
    if (lane >= d) inc += nb;
  }
  if (lane == 63) sh[wid] = inc;
  __syncthreads();
  T pre = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    T t = sh[w];
    pre += (w < wid) ? t : T(0);
    tot += t;
  }
  __syncthreads();
  *total = tot;
  return pre + inc - v;
}

template <typename T>
__device__ __forceinline__ T block_sum(T v, T* sh) {
  T tot;
  block_exclusive_scan(v, &tot, sh);
  return tot;
}

// ---- wave primitives on DPP lane moves (no lane-address registers) ------------------
// Controls of the GFX9 DPP encoding: row_shr:n, row_bcast:15, row_bcast:31,
// wave_shl:1 (lane i takes lane i+1), wave_shr:1 (lane i takes lane i-1).  A lane whose source is out of its row, or whose row is masked
// off, receives 0.
constexpr int kRowShr1 = 0x111, kRowShr2 = 0x112, kRowShr4 = 0x114, kRowShr8 = 0x118;
constexpr int kRowBcast15 = 0x142, kRowBcast31 = 0x143, kWaveShl1 = 0x130, kWaveShr1 = 0x138;

template <int CTRL, int ROWS = 0xF>
__device__ __forceinline__ uint32_t dpp0(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, ROWS, 0xF, false);
}
template <int CTRL, int ROWS = 0xF>
__device__ __forceinline__ uint64_t dpp0_64(uint64_t v) {
  return (uint64_t)dpp0<CTRL, ROWS>((uint32_t)v) | ((uint64_t)dpp0<CTRL, ROWS>((uint32_t)(v >> 32)) << 32);
}

// Inclusive prefix sum over the 64 lanes: four shifts within each 16-lane
// row, then row 0's total into row 1 (and row 2's into row 3), then lane 31
// into rows 2 and 3.
__device__ __forceinline__ uint32_t wave_incl_add(uint32_t v) {
  v += dpp0<kRowShr1>(v);
  v += dpp0<kRowShr2>(v);
  v += dpp0<kRowShr4>(v);
  v += dpp0<kRowShr8>(v);
  v += dpp0<kRowBcast15, 0xA>(v);
  v += dpp0<kRowBcast31, 0xC>(v);
  return v;
}
__device__ __forceinline__ uint64_t wave_incl_add64(uint64_t v) {
  v += dpp0_64<kRowShr1>(v);
  v += dpp0_64<kRowShr2>(v);
  v += dpp0_64<kRowShr4>(v);
  v += dpp0_64<kRowShr8>(v);
  v += dpp0_64<kRowBcast15, 0xA>(v);
  v += dpp0_64<kRowBcast31, 0xC>(v);
  return v;
}
__device__ __forceinline__ uint32_t umax(uint32_t a, uint32_t b) { return a > b ? a : b; }
__device__ __forceinline__ uint32_t wave_incl_max(uint32_t v) {
  v = umax(v, dpp0<kRowShr1>(v));
  v = umax(v, dpp0<kRowShr2>(v));
  v = umax(v, dpp0<kRowShr4>(v));
  v = umax(v, dpp0<kRowShr8>(v));
  v = umax(v, dpp0<kRowBcast15, 0xA>(v));
  v = umax(v, dpp0<kRowBcast31, 0xC>(v));
  return v;
}
__device__ __forceinline__ uint32_t lane63(uint32_t v) { return (uint32_t)__builtin_amdgcn_readlane((int)v, 63); }
__device__ __forceinline__ uint64_t lane63_64(uint64_t v) {
  return (uint64_t)lane63((uint32_t)v) | ((uint64_t)lane63((uint32_t)(v >> 32)) << 32);
}

// 4 bytes starting at p (any alignment) from a buffer whose readable bytes
// end at lim; bytes at or past lim read as 0.  Only aligned dwords holding at
// least one readable byte are loaded: such a dword lies in a page the buffer
// occupies, so nothing outside it can fault.
__device__ __forceinline__ uint32_t load4_unaligned(const uint8_t* p, const uint8_t* lim) {
  const uintptr_t a = (uintptr_t)p, a0 = a & ~(uintptr_t)3, e = (uintptr_t)lim;
  const uint32_t sh = (uint32_t)(a & 3u);
  const uint32_t* w = (const uint32_t*)a0;
  const uint32_t lo = a0 < e ? w[0] : 0u;
  const uint32_t hi = (sh != 0u && a0 + 4u < e) ? w[1] : 0u;
  uint32_t v = __builtin_amdgcn_alignbyte(hi, lo, sh);
  if (a + 4u > e) v = a >= e ? 0u : (v & ((1u << (8u * (uint32_t)(e - a))) - 1u));
  return v;
}

// ---- 16-byte copies ---------------------------------------------------------
// Bytes 4q + r .. 4q + r + 15 of the 32 bytes a | b (q < 4, r < 4, the same
// in every lane).  Plain variables, no array: a select between two array
// elements would keep the array in memory.
__device__ __forceinline__ uint4 funnel16(uint4 a, uint4 b, uint32_t q, uint32_t r) {
  const bool q2 = (q & 2u) != 0u, q1 = (q & 1u) != 0u;
  // shift by two dwords, then by one
  const uint32_t v0 = q2 ? a.z : a.x, v1 = q2 ? a.w : a.y, v2 = q2 ? b.x : a.z, v3 = q2 ? b.y : a.w,
                 v4 = q2 ? b.z : b.x, v5 = q2 ? b.w : b.y;
  const uint32_t u0 = q1 ? v1 : v0, u1 = q1 ? v2 : v1, u2 = q1 ? v3 : v2, u3 = q1 ? v4 : v3, u4 = q1 ? v5 : v4;
  return make_uint4(__builtin_amdgcn_alignbyte(u1, u0, r), __builtin_amdgcn_alignbyte(u2, u1, r),
                    __builtin_amdgcn_alignbyte(u3, u2, r), __builtin_amdgcn_alignbyte(u4, u3, r));
}

// Copy n bytes from src to dst (any alignments) with one wave (this is lane
// l): single bytes before dst's first 16-byte boundary and after its last,
// 16-byte stores in between.  The source is read as aligned 16-byte blocks
// that each hold at least one of the n bytes, so no read leaves the pages the
// source bytes lie in.  Each lane loads four blocks before it stores; the
// block after a lane's comes from the next lane by a wave shift (lane 63
// takes lane 0's next block, or loads the block after the round).  Named
// registers rather than an array keep the blocks out of memory.
__device__ __forceinline__ void copy_bytes16(uint8_t* dst, const uint8_t* src, uint32_t n, uint32_t l) {
  const uint32_t h0 = (uint32_t)((16u - ((uintptr_t)dst & 15u)) & 15u);
  const uint32_t h = h0 < n ? h0 : n;
  if (l < h) dst[l] = src[l];
  const uint32_t nb = (n - h) >> 4;         // 16-byte stores
  const uintptr_t s = (uintptr_t)(src + h);
  const uint32_t sh = (uint32_t)(s & 15u);
  const uint32_t ns = nb + (sh ? 1u : 0u);  // source blocks holding the stored bytes
  const uint4* sb = (const uint4*)(s - sh);
  uint4* db = (uint4*)(dst + h);
  const uint32_t q = sh >> 2, r = sh & 3u;
  const uint4 z = make_uint4(0u, 0u, 0u, 0u);
  auto next_of = [&](uint4 a, uint4 nx) {  // the block after this lane's
    uint4 b;
    b.x = dpp0<kWaveShl1>(a.x);
    b.y = dpp0<kWaveShl1>(a.y);
    b.z = dpp0<kWaveShl1>(a.z);
    b.w = dpp0<kWaveShl1>(a.w);
    return l == 63u ? nx : b;
  };
  auto lane0 = [&](uint4 a) {
    return make_uint4((uint32_t)__builtin_amdgcn_readlane((int)a.x, 0), (uint32_t)__builtin_amdgcn_readlane((int)a.y, 0),
                      (uint32_t)__builtin_amdgcn_readlane((int)a.z, 0), (uint32_t)__builtin_amdgcn_readlane((int)a.w, 0));
  };
  auto put = [&](uint32_t k, uint4 a, uint4 b) {
    if (k < nb) db[k] = sh ? funnel16(a, b, q, r) : a;
  };
#pragma unroll 1
  for (uint32_t k0 = 0; k0 < nb; k0 += 256u) {
    const uint32_t k = k0 + l;
    const uint4 a0 = k < ns ? sb[k] : z;
    const uint4 a1 = k + 64u < ns ? sb[k + 64u] : z;
    const uint4 a2 = k + 128u < ns ? sb[k + 128u] : z;
    const uint4 a3 = k + 192u < ns ? sb[k + 192u] : z;
    const uint32_t kx = k0 + 256u;  // first block of the next round
    const uint4 x = (l == 63u && sh && kx < ns) ? sb[kx] : z;
    put(k, a0, next_of(a0, lane0(a1)));
    put(k + 64u, a1, next_of(a1, lane0(a2)));
    put(k + 128u, a2, next_of(a2, lane0(a3)));
    put(k + 192u, a3, next_of(a3, x));
  }
  const uint32_t t = h + 16u * nb + l;  // fewer than 16 tail bytes
  if (t < n) dst[t] = src[t];
}

// copy_bytes16 with one block per lane per round (fewer registers, for
// callers under register pressure).
__device__ __forceinline__ void copy_bytes16_r1(uint8_t* dst, const uint8_t* src, uint32_t n, uint32_t l) {
  const uint32_t h0 = (uint32_t)((16u - ((uintptr_t)dst & 15u)) & 15u);
  const uint32_t h = h0 < n ? h0 : n;
  if (l < h) dst[l] = src[l];
  const uint32_t nb = (n - h) >> 4;
  const uintptr_t s = (uintptr_t)(src + h);
  const uint32_t sh = (uint32_t)(s & 15u);
  const uint32_t ns = nb + (sh ? 1u : 0u);
  const uint4* sb = (const uint4*)(s - sh);
  uint4* db = (uint4*)(dst + h);
  const uint32_t q = sh >> 2, r = sh & 3u;
  const uint4 z = make_uint4(0u, 0u, 0u, 0u);
#pragma unroll 1
  for (uint32_t k0 = 0; k0 < nb; k0 += 64u) {
    const uint32_t k = k0 + l;
    const uint4 a = k < ns ? sb[k] : z;
    const uint4 x = (l == 63u && sh && k0 + 64u < ns) ? sb[k0 + 64u] : z;  // lane 63's next block
    uint4 b;
    b.x = dpp0<kWaveShl1>(a.x);
    b.y = dpp0<kWaveShl1>(a.y);
    b.z = dpp0<kWaveShl1>(a.z);
    b.w = dpp0<kWaveShl1>(a.w);
    if (l == 63u) b = x;
    if (k < nb) db[k] = sh ? funnel16(a, b, q, r) : a;
  }
  const uint32_t t = h + 16u * nb + l;
  if (t < n) dst[t] = src[t];
}

// copy_bytes16 with two blocks per lane per round.
__device__ __forceinline__ void copy_bytes16_r2(uint8_t* dst, const uint8_t* src, uint32_t n, uint32_t l) {
  const uint32_t h0 = (uint32_t)((16u - ((uintptr_t)dst & 15u)) & 15u);
  const uint32_t h = h0 < n ? h0 : n;
  if (l < h) dst[l] = src[l];
  const uint32_t nb = (n - h) >> 4;
  const uintptr_t s = (uintptr_t)(src + h);
  const uint32_t sh = (uint32_t)(s & 15u);
  const uint32_t ns = nb + (sh ? 1u : 0u);
  const uint4* sb = (const uint4*)(s - sh);
  uint4* db = (uint4*)(dst + h);
  const uint32_t q = sh >> 2, r = sh & 3u;
  const uint4 z = make_uint4(0u, 0u, 0u, 0u);
  auto next_of = [&](uint4 a, uint4 nx) {
    uint4 b;
    b.x = dpp0<kWaveShl1>(a.x);
    b.y = dpp0<kWaveShl1>(a.y);
    b.z = dpp0<kWaveShl1>(a.z);
    b.w = dpp0<kWaveShl1>(a.w);
    return l == 63u ? nx : b;
  };
  auto lane0 = [&](uint4 a) {
    return make_uint4((uint32_t)__builtin_amdgcn_readlane((int)a.x, 0), (uint32_t)__builtin_amdgcn_readlane((int)a.y, 0),
                      (uint32_t)__builtin_amdgcn_readlane((int)a.z, 0), (uint32_t)__builtin_amdgcn_readlane((int)a.w, 0));
  };
  auto put = [&](uint32_t k, uint4 a, uint4 b) {
    if (k < nb) db[k] = sh ? funnel16(a, b, q, r) : a;
  };
#pragma unroll 1
  for (uint32_t k0 = 0; k0 < nb; k0 += 128u) {
    const uint32_t k = k0 + l;
    const uint4 a0 = k < ns ? sb[k] : z;
    const uint4 a1 = k + 64u < ns ? sb[k + 64u] : z;
    const uint32_t kx = k0 + 128u;  // first block of the next round
    const uint4 x = (l == 63u && sh && kx < ns) ? sb[kx] : z;
    put(k, a0, next_of(a0, lane0(a1)));
    put(k + 64u, a1, next_of(a1, x));
  }
  const uint32_t t = h + 16u * nb + l;  // fewer than 16 tail bytes
  if (t < n) dst[t] = src[t];
}

// Zero n bytes at dst (any alignment) with one wave (this is lane l).
__device__ __forceinline__ void zero_bytes16(uint8_t* dst, uint32_t n, uint32_t l) {
  const uint32_t h0 = (uint32_t)((16u - ((uintptr_t)dst & 15u)) & 15u);
  const uint32_t h = h0 < n ? h0 : n;
  if (l < h) dst[l] = 0u;
  const uint32_t nb = (n - h) >> 4;
  uint4* db = (uint4*)(dst + h);
  for (uint32_t k = l; k < nb; k += 64u) db[k] = make_uint4(0u, 0u, 0u, 0u);
  const uint32_t t = h + 16u * nb + l;
  if (t < n) dst[t] = 0u;
}

// Fill n bytes at dst with the 32-bit pattern rep (byte k of the run is
// byte (k mod 4) of rep), one 16-byte block per lane of the wave per round.
__device__ __forceinline__ void fill_bytes16(uint8_t* dst, uint32_t n, uint32_t l, uint32_t rep) {
  const uint32_t h0 = (uint32_t)((16u - ((uintptr_t)dst & 15u)) & 15u);
  const uint32_t h = h0 < n ? h0 : n;
  if (l < h) dst[l] = (uint8_t)(rep >> (8u * (l & 3u)));
  const uint32_t nb = (n - h) >> 4;
  const uint32_t rot = __builtin_amdgcn_alignbyte(rep, rep, h & 3u);  // the pattern from byte h on
  uint4* db = (uint4*)(dst + h);
  for (uint32_t k = l; k < nb; k += 64u) db[k] = make_uint4(rot, rot, rot, rot);
  const uint32_t t = h + 16u * nb + l;
  if (t < n) dst[t] = (uint8_t)(rep >> (8u * (t & 3u)));
}

// ---- launchers (host side, one per kernel family) -------------------------
struct EncodeArgs {
  const uint8_t* in;
  uint64_t n;
  uint32_t cs, ws, level;
  uint32_t num_chunks;
  uint8_t* out;          // the stream
  uint64_t* out_bytes;
  uint8_t* staging;      // num_chunks * cs bytes (+ slack): one payload slot per chunk
  uint64_t* tile_flags;  // one look-back word per compaction tile (three sets in split mode)
  void* ctl;             // error flag
  // split mode only (km == nullptr otherwise): per-chunk {items, matches}
  // and the ports; out is then the meta port
  uint2* km = nullptr;
  uint8_t* lit = nullptr;
  uint8_t* lens = nullptr;
  uint8_t* offs = nullptr;
  uint64_t* port_bytes = nullptr;  // [4]: literals, lengths, offsets, meta
  uint32_t window = kWindow;        // near-window offsets: 32, 48 or 64
};
uint64_t encode_ctl_bytes();
uint64_t encode_tiles(uint32_t num_chunks);
hipError_t launch_encode_chunks(const EncodeArgs& a, hipStream_t stream);
hipError_t launch_encode_advancing(const EncodeArgs& a, hipStream_t stream);
hipError_t launch_compact(const EncodeArgs& a, hipStream_t stream);
hipError_t launch_split_compact(const EncodeArgs& a, hipStream_t stream);

struct DecodeArgs {
  const uint8_t* in;
  uint64_t in_bytes;
  uint8_t* out;
  uint64_t out_capacity;
  uint64_t* out_bytes;
  uint32_t* status;
  void* params;         // device-resident stream parameters
  uint32_t* loc;        // chunks_cap payload offsets within their scan tile
  uint64_t* tile_sums;  // one per scan tile (workspace_tiles slots)
  uint32_t* tile_err;   // one per scan tile
  uint32_t chunks_cap;  // host bound on num_chunks
  hipEvent_t ev_start;  // optional, recorded around the chunk decode kernel
  hipEvent_t ev_stop;
};
uint64_t decode_params_bytes();
hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream);
hipError_t launch_decode_serial(const DecodeArgs& a, hipStream_t stream);

// Split mode: the meta port plays the stream's part (header, size table, flag
// bitmaps); the item bytes come from the other three ports.
struct SplitDecodeArgs {
  const uint8_t* meta;
  uint64_t meta_bytes;
  const uint8_t* lit;
  uint64_t lit_bytes;
  const uint8_t* lens;
  const uint8_t* offs;
  uint64_t tok_bytes;   // bytes of each of lengths and offsets
  uint8_t* out;
  uint64_t out_capacity;
  uint64_t* out_bytes;
  uint32_t* status;
  void* params;
  uint32_t* loc;        // 3 x chunks_cap offsets within the scan tile: flags, literals, matches
  uint64_t* tile_sums;  // 3 x tiles
  uint32_t* tile_err;   // tiles
  uint32_t chunks_cap;
};
hipError_t launch_decode_split(const SplitDecodeArgs& a, hipStream_t stream);

}  // namespace gpulz
