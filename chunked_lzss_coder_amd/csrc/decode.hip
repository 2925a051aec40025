// decode.hip -- stream decode for gfx950 (two kernels, no host round trip).
//
// The header and size table are read on the device, so nothing waits on the
// host (the GPULZStage page's own inverse reads the header with blocking
// copies before it can launch; this one can be captured).
//
// scan_kernel (<= 256 workgroups, one per tile of T chunks): checks the
//   header, writes the parameters, the initial status and length; validates
//   every size-table row against its chunk's real bytes, writes each chunk's
//   payload offset within its tile, the tile's total and an error flag.
//   No workgroup waits on another.
// chunks_kernel (one wave per chunk; four waves per chunk when a chunk has
//   more than 1024 elements): the chunk's payload offset is its tile's offset
//   (sum of earlier tile totals) plus its offset in the tile; then
//     zero row -> zero fill; raw row -> copy; otherwise, per the
//     block-parallel decode paragraph of the GPULZStage page:
//     a. items 64 at a time: an item's token position follows from the
//        number of matches before it (flag popcounts), its output length is
//        1 or the token's length; a wave scan of the lengths gives every
//        item's output position; every token rule is checked;
//     b. each element of a match item points into the data before the item,
//        start - O + (q - start) mod O, always < start; pointer jumping
//        resolves chains in at most log2(items)+1 rounds with early exit;
//     c. the chunk's real bytes are stored; the zero padding must have
//        decoded to zeros.
//   Errors only ever raise the status (and zero the length), so the kernel
//   order makes the first write of the status the header kernel's.
#include "common.h"

namespace gpulz {
namespace {

constexpr uint32_t kTileMin = 4096;   // chunks per scan tile (at least)
constexpr uint32_t kMaxTiles = 256;
constexpr uint32_t kScanPer = 16;     // chunks per thread per scan round
constexpr uint32_t kScanRound = kScanPer * kBlock;

__device__ __forceinline__ uint32_t ld_u32_bytes(const uint8_t* p) {
  return (uint32_t)p[0] | ((uint32_t)p[1] << 8) | ((uint32_t)p[2] << 16) | ((uint32_t)p[3] << 24);
}
__device__ __forceinline__ uint64_t ld_u64_bytes(const uint8_t* p) {
  return (uint64_t)ld_u32_bytes(p) | ((uint64_t)ld_u32_bytes(p + 4) << 32);
}
__device__ __forceinline__ uint32_t lane_id() { return threadIdx.x & 63u; }

__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__device__ __forceinline__ uint2 read_row(const uint8_t* in, uint64_t c) {
  const uint8_t* e = in + kHeaderBytes + kEntryBytes * c;
  return make_uint2(ld_u32_bytes(e), ld_u32_bytes(e + 4));
}

__device__ __forceinline__ bool row_ok(uint2 e, uint32_t bc) {
  if (e.x == 0u) return e.y == 0u || ((e.y & kRawBit) && (e.y & ~kRawBit) == bc);
  return !(e.y & kRawBit) && (uint64_t)e.x + e.y < bc;
}

__device__ __forceinline__ void raise_status(uint32_t* status, uint64_t* out_bytes, uint32_t code) {
  atomicMax(status, code);
  *out_bytes = 0u;
}

struct DecP {
  uint64_t n;            // original size
  uint64_t pb;           // payload bytes
  uint64_t base;         // stream offset of the first payload
  uint32_t cs, ws, nc;   // chunk size, word size, chunks
  uint32_t status;       // header status
  uint32_t T, ntiles;    // chunks per scan tile, tiles
};

__global__ __launch_bounds__(kBlock) void scan_kernel(const uint8_t* __restrict__ in, uint64_t in_bytes,
                                                      uint64_t out_capacity, uint32_t chunks_cap, uint32_t T,
                                                      DecP* __restrict__ P, uint32_t* __restrict__ loc,
                                                      uint64_t* __restrict__ tile_sum,
                                                      uint32_t* __restrict__ tile_err, uint32_t* __restrict__ status,
                                                      uint64_t* __restrict__ out_bytes) {
  __shared__ uint64_t sh[kWaves];
  const uint32_t magic = ld_u32_bytes(in);
  const uint32_t ver = in[4], ws = in[5], res = in[6] | ((uint32_t)in[7] << 8);
  const uint32_t cs = ld_u32_bytes(in + 8), nc = ld_u32_bytes(in + 12);
  const uint64_t n = ld_u64_bytes(in + 16), pb = ld_u64_bytes(in + 24);
  uint32_t st = kStatusOk;
  if (magic != kMagic || ver != kVersion || res != 0 || !word_size_ok(ws) || !chunk_size_ok(cs)) {
    st = kStatusCorrupt;
  } else {
    const uint64_t want = n / cs + ((n % cs) != 0);
    const uint64_t total = (uint64_t)kHeaderBytes + (uint64_t)kEntryBytes * nc + pb;
    if (want != nc || pb > n || pb > in_bytes || total > in_bytes) st = kStatusCorrupt;
    else if (n > out_capacity) st = kStatusCapacity;
    else if (nc > chunks_cap) st = kStatusCorrupt;
  }
  const uint32_t ntiles = (nc + T - 1u) / T;
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    P->n = n;
    P->pb = pb;
    P->base = (uint64_t)kHeaderBytes + (uint64_t)kEntryBytes * nc;
    P->cs = cs;
    P->ws = ws;
    P->nc = nc;
    P->status = st;
    P->T = T;
    P->ntiles = ntiles;
    *status = st;
    *out_bytes = st == kStatusOk ? n : 0u;
  }
  if (st != kStatusOk || blockIdx.x >= ntiles) return;
  const uint64_t t0 = (uint64_t)blockIdx.x * T;
  const uint64_t t1 = (t0 + T) < nc ? (t0 + T) : nc;
  uint64_t carry = 0;
  bool bad = false;
  for (uint64_t r0 = t0; r0 < t1; r0 += kScanRound) {
    const uint64_t c0 = r0 + (uint64_t)threadIdx.x * kScanPer;
    uint32_t sz[kScanPer];
    uint64_t local = 0;
#pragma unroll
    for (uint32_t j = 0; j < kScanPer; ++j) {
      const uint64_t c = c0 + j;
      sz[j] = 0;
      if (c < t1) {
        const uint2 e = read_row(in, c);
        const uint64_t start = c * cs;
        const uint32_t bc = (uint32_t)((n - start) < cs ? (n - start) : cs);
        if (row_ok(e, bc)) sz[j] = entry_payload(e.x, e.y);
        else bad = true;
      }
      local += sz[j];
    }
    uint64_t tot;
    uint64_t off = carry + block_exclusive_scan(local, &tot, sh);
#pragma unroll
    for (uint32_t j = 0; j < kScanPer; ++j) {
      const uint64_t c = c0 + j;
      if (c < t1) loc[c] = (uint32_t)(off - 0u);  // offset within the tile (< 2^32 by the tile sizing)
      off += sz[j];
    }
    carry += tot;
  }
  const bool anybad = __syncthreads_or(bad);
  if (threadIdx.x == 0) {
    tile_sum[blockIdx.x] = carry;
    tile_err[blockIdx.x] = anybad ? 1u : 0u;
  }
}

// ---- per-chunk decode -------------------------------------------------------------
// LDS per team: decoded bytes VAL (cs), source index per element SRC (2E),
// item-start bitmap STB (E/32 words) and its popcount prefix SPRE, flag words
// FW and their popcount prefix FPRE.
constexpr uint32_t kWaveArena = 4096 + 2048 + 4 * (32 + 33 + 33 + 34) + 64;  // bytes, E <= 1024 per wave
constexpr uint32_t kArena = kWaves * kWaveArena;

template <uint32_t TW>
struct Team {
  static constexpr uint32_t TL = 64u * TW;
  __device__ static void sync() {
    if (TW == 1) wave_sync();
    else __syncthreads();
  }
};

// Exclusive scan of one value per team lane; total to *tot.  (TW == 1: DPP
// shuffles in one wave; TW > 1: the workgroup scan.)
template <uint32_t TW>
__device__ __forceinline__ uint32_t team_scan(uint32_t v, uint32_t* tot, uint32_t* sh) {
  if constexpr (TW == 1) {
    const uint32_t lane = lane_id();
    uint32_t inc = v;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const uint32_t t = __shfl_up(inc, d, 64);
      if (lane >= (uint32_t)d) inc += t;
    }
    *tot = __shfl(inc, 63, 64);
    return inc - v;
  } else {
    return block_exclusive_scan(v, tot, sh);
  }
}

template <uint32_t TW>
__device__ __forceinline__ bool team_any(bool v) {
  if constexpr (TW == 1) return __ballot(v) != 0ull;
  else return __syncthreads_or(v);
}

// Decode one coded chunk.  pay: its payload (F flag bytes, D data bytes) in
// the stream; lim: end of the readable input.  Returns false on a rule
// violation.  Writes the chunk's real bytes to dst.
template <uint32_t TW>
__device__ bool decode_coded(const uint8_t* pay, const uint8_t* lim, uint32_t F, uint32_t D, uint32_t cs,
                             uint32_t ws, uint32_t bc, uint8_t* dst, uint8_t* arena, uint32_t* sh) {
  using Tm = Team<TW>;
  constexpr uint32_t TL = Tm::TL;
  const uint32_t g = threadIdx.x % TL;
  const uint32_t E = cs / ws;
  const uint32_t EW = E / 32u;
  const uint32_t NI = 8u * F;
  const uint32_t NW = (F + 3u) / 4u;  // flag words
  uint8_t* VAL = arena;
  uint16_t* SRC = (uint16_t*)(arena + cs);
  uint32_t* STB = (uint32_t*)(arena + cs + 2u * E);
  uint32_t* SPRE = STB + EW;
  uint32_t* FW = SPRE + EW + 1u;
  uint32_t* FPRE = FW + NW + 1u;
  const uint8_t* dat = pay + F;

  for (uint32_t w = g; w < NW; w += TL) {
    uint32_t v = load4_unaligned(pay + 4u * w, lim);
    const uint32_t nb = F - 4u * w;  // flag bytes in this word
    if (nb < 4u) v &= (1u << (8u * nb)) - 1u;
    FW[w] = v;
  }
  for (uint32_t w = g; w < EW; w += TL) STB[w] = 0u;
  Tm::sync();
  uint32_t mt_total = 0;
  for (uint32_t w0 = 0; w0 < NW; w0 += TL) {
    const uint32_t w = w0 + g;
    const uint32_t c = w < NW ? (uint32_t)__builtin_popcount(FW[w]) : 0u;
    uint32_t tot;
    const uint32_t ex = team_scan<TW>(c, &tot, sh);
    if (w < NW) FPRE[w] = mt_total + ex;
    mt_total += tot;
  }
  Tm::sync();

  // ---- a. items ----------------------------------------------------------------------
  uint32_t outpos = 0, K = 0, covered = 0;
  bool bad = false;
  for (uint32_t k0 = 0; k0 < NI && outpos < E; k0 += TL) {
    const uint32_t k = k0 + g;
    const bool inb = k < NI;
    uint32_t len = 0, O = 0, tp = 0;
    bool mt = false, readable = false;
    if (inb) {
      const uint32_t w = k >> 5, b = k & 31u, fw = FW[w];
      mt = (fw >> b) & 1u;
      const uint32_t m = FPRE[w] + (uint32_t)__builtin_popcount(fw & ((1u << b) - 1u));
      tp = ws * (k - m) + 2u * m;
      readable = tp + (mt ? 2u : ws) <= D;
      if (readable) {
        if (mt) {
          len = dat[tp];
          O = dat[tp + 1u];
        } else {
          len = 1u;
        }
      }
    }
    uint32_t tot;
    const uint32_t op = outpos + team_scan<TW>(len, &tot, sh);
    const bool live = inb && op < E;
    if (live) {
      if (!readable) bad = true;
      if (mt && (len == 0u || O == 0u || O > op || op + len > E)) bad = true;
      if (!bad) {
        atomicOr(&STB[op >> 5], 1u << (op & 31u));
        if (!mt) {
          const uint32_t v = load4_unaligned(dat + tp, lim);
          if (ws == 4u) *(uint32_t*)(VAL + 4u * op) = v;
          else if (ws == 2u) *(uint16_t*)(VAL + 2u * op) = (uint16_t)v;
          else VAL[op] = (uint8_t)v;
          SRC[op] = (uint16_t)op;
        }
      }
    }
    uint32_t nlive, llen;
    team_scan<TW>(live ? 1u : 0u, &nlive, sh);
    team_scan<TW>(live ? len : 0u, &llen, sh);
    K += nlive;
    covered += llen;
    outpos += tot;
  }
  // the live items cover exactly E elements, consume exactly D data bytes,
  // and no flag bit is set past the last one
  {
    uint32_t mK;
    if (K >= NI) {
      mK = mt_total;
    } else {
      const uint32_t w = K >> 5, b = K & 31u;
      mK = FPRE[w] + (uint32_t)__builtin_popcount(FW[w] & ((1u << b) - 1u));
    }
    if (covered != E || (K + 7u) / 8u != F || ws * (K - mK) + 2u * mK != D || mK != mt_total) bad = true;
  }
  if (team_any<TW>(bad)) return false;
  Tm::sync();

  // ---- b. element sources, pointer jumping ----------------------------------------------
  uint32_t spre_total = 0;
  for (uint32_t w0 = 0; w0 < EW; w0 += TL) {
    const uint32_t w = w0 + g;
    const uint32_t c = w < EW ? (uint32_t)__builtin_popcount(STB[w]) : 0u;
    uint32_t tot;
    const uint32_t ex = team_scan<TW>(c, &tot, sh);
    if (w < EW) SPRE[w] = spre_total + ex;
    spre_total += tot;
  }
  Tm::sync();
  bool cover_bad = false;
  for (uint32_t q = g; q < E; q += TL) {
    const uint32_t w = q >> 5, b = q & 31u;
    const uint32_t upto = b == 31u ? ~0u : ((2u << b) - 1u);
    uint32_t bits = STB[w] & upto, ww = w;
    const uint32_t cnt = SPRE[w] + (uint32_t)__builtin_popcount(bits);
    while (bits == 0u && ww > 0u) bits = STB[--ww];  // a match reaches back at most 255 elements
    if (bits == 0u) {  // element 0 always starts an item; this means no items cover q
      cover_bad = true;
      continue;
    }
    const uint32_t st = 32u * ww + 31u - (uint32_t)__builtin_clz(bits);
    const uint32_t k = cnt - 1u;
    const uint32_t fw = FW[k >> 5], kb = k & 31u;
    if (!((fw >> kb) & 1u)) continue;  // literal: already in place
    const uint32_t m = FPRE[k >> 5] + (uint32_t)__builtin_popcount(fw & ((1u << kb) - 1u));
    const uint32_t tp = ws * (k - m) + 2u * m;
    const uint32_t O = dat[tp + 1u];
    SRC[q] = (uint16_t)(st - O + (q - st) % O);
  }
  if (spre_total != K || team_any<TW>(cover_bad)) return false;
  Tm::sync();
  bool unres = true;
  for (int round = 0; round < 16 && unres; ++round) {
    unres = false;
    for (uint32_t q = g; q < E; q += TL) {
      const uint32_t s = SRC[q];
      if (s == q) continue;
      const uint32_t s2 = SRC[s];
      if (s2 == s) {
        if (ws == 4u) *(uint32_t*)(VAL + 4u * q) = *(const uint32_t*)(VAL + 4u * s);
        else if (ws == 2u) *(uint16_t*)(VAL + 2u * q) = *(const uint16_t*)(VAL + 2u * s);
        else VAL[q] = VAL[s];
        SRC[q] = (uint16_t)q;
      } else {
        SRC[q] = (uint16_t)s2;
        unres = true;
      }
    }
    unres = team_any<TW>(unres);
    Tm::sync();
  }
  if (unres) return false;  // chains always end within log2(items)+1 rounds

  // ---- c. store the real bytes; the padding must have decoded to zeros -----------------
  const bool al = (((uintptr_t)dst) & 3u) == 0;
  bool padbad = false;
  for (uint32_t i = g; i < cs / 4u; i += TL) {
    const uint32_t v = *(const uint32_t*)(VAL + 4u * i);
    const uint32_t b0 = 4u * i;
    if (b0 + 4u > bc) {
      const uint32_t keep = b0 >= bc ? 0u : bc - b0;
      if (keep < 4u && (v & (~0u << (8u * keep)))) padbad = true;
    }
    if (b0 >= bc) continue;
    if (al && b0 + 4u <= bc) {
      *(uint32_t*)(dst + b0) = v;
    } else {
      for (uint32_t b = 0; b < 4u; ++b)
        if (b0 + b < bc) dst[b0 + b] = (uint8_t)(v >> (8u * b));
    }
  }
  return !team_any<TW>(padbad);
}

template <uint32_t TW>
__device__ void decode_group(const DecP& p, const uint8_t* in, const uint8_t* lim, uint8_t* out,
                             const uint32_t* loc, const uint64_t* tile_sum, uint32_t* status, uint64_t* out_bytes,
                             uint8_t* arena_all, uint32_t* sh) {
  constexpr uint32_t TL = 64u * TW;
  constexpr uint32_t CPW = kWaves / TW;  // chunks per workgroup
  const uint32_t team = threadIdx.x / TL, g = threadIdx.x % TL;
  uint8_t* arena = arena_all + team * (kArena / CPW);
  const uint32_t ngroups = (p.nc + CPW - 1u) / CPW;
  for (uint32_t grp = blockIdx.x; grp < ngroups; grp += gridDim.x) {
    const uint64_t c = (uint64_t)grp * CPW + team;
    if (c >= p.nc) continue;  // CPW > 1 only when TW == 1: no workgroup barrier below
    const uint2 e = read_row(in, c);
    const uint64_t start = c * p.cs;
    const uint32_t bc = (uint32_t)((p.n - start) < p.cs ? (p.n - start) : p.cs);
    if (!row_ok(e, bc)) continue;  // reported by the scan kernel
    const uint32_t size = entry_payload(e.x, e.y);
    // payload offset = earlier tiles' totals + offset within the tile
    const uint32_t t = (uint32_t)(c / p.T);
    uint64_t tp = 0;
    for (uint32_t i = lane_id(); i < t; i += 64u) tp += tile_sum[i];
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) tp += __shfl_xor(tp, d, 64);
    const uint64_t off = tp + loc[c];
    if (off + size > p.pb) continue;  // sizes inconsistent with the header: reported by wave 0 below
    const uint8_t* pay = in + p.base + off;
    uint8_t* dst = out + start;
    const bool al = (((uintptr_t)dst) & 3u) == 0;
    if (e.x == 0u && e.y == 0u) {
      for (uint32_t i = g; i < (bc + 3u) / 4u; i += TL) {
        if (al && 4u * i + 4u <= bc) *(uint32_t*)(dst + 4u * i) = 0u;
        else
          for (uint32_t b = 0; b < 4u; ++b)
            if (4u * i + b < bc) dst[4u * i + b] = 0u;
      }
    } else if (e.x == 0u) {
      for (uint32_t i = g; i < (bc + 3u) / 4u; i += TL) {
        const uint32_t v = load4_unaligned(pay + 4u * i, lim);
        if (al && 4u * i + 4u <= bc) *(uint32_t*)(dst + 4u * i) = v;
        else
          for (uint32_t b = 0; b < 4u; ++b)
            if (4u * i + b < bc) dst[4u * i + b] = (uint8_t)(v >> (8u * b));
      }
    } else if (e.x > (p.cs / p.ws + 7u) / 8u) {  // more flag bytes than a chunk has items
      if (g == 0) raise_status(status, out_bytes, kStatusCorrupt);
    } else {
      if (!decode_coded<TW>(pay, lim, e.x, e.y, p.cs, p.ws, bc, dst, arena, sh) && g == 0)
        raise_status(status, out_bytes, kStatusCorrupt);
    }
    Team<TW>::sync();
  }
}

__global__ __launch_bounds__(kBlock) void chunks_kernel(const uint8_t* __restrict__ in, uint64_t in_bytes,
                                                        uint8_t* __restrict__ out, const DecP* __restrict__ P,
                                                        const uint32_t* __restrict__ loc,
                                                        const uint64_t* __restrict__ tile_sum,
                                                        const uint32_t* __restrict__ tile_err,
                                                        uint32_t* __restrict__ status,
                                                        uint64_t* __restrict__ out_bytes) {
  __shared__ __attribute__((aligned(16))) uint8_t arena[kArena];
  __shared__ uint32_t sh[kWaves];
  const DecP p = *P;
  if (p.status != kStatusOk) return;
  if (blockIdx.x == 0 && threadIdx.x < 64u) {
    // stream-wide checks: the tile totals must add up to the header's payload
    // size and no row may be invalid
    uint64_t s = 0;
    uint32_t err = 0;
    for (uint32_t i = lane_id(); i < p.ntiles; i += 64u) {
      s += tile_sum[i];
      err |= tile_err[i];
    }
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) {
      s += __shfl_xor(s, d, 64);
      err |= __shfl_xor(err, d, 64);
    }
    if (lane_id() == 0 && (s != p.pb || err)) raise_status(status, out_bytes, kStatusCorrupt);
  }
  const uint8_t* lim = in + in_bytes;
  const uint32_t E = p.cs / p.ws;
  if (E <= 1024u) decode_group<1>(p, in, lim, out, loc, tile_sum, status, out_bytes, arena, sh);
  else decode_group<4>(p, in, lim, out, loc, tile_sum, status, out_bytes, arena, sh);
}

}  // namespace

uint32_t decode_tile_chunks(uint32_t chunks_cap) {
  uint32_t T = (chunks_cap + kMaxTiles - 1u) / kMaxTiles;
  T = (T + kTileMin - 1u) / kTileMin * kTileMin;
  return T < kTileMin ? kTileMin : T;
}
uint64_t decode_params_bytes() { return sizeof(DecP); }

hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream) {
  const uint32_t T = decode_tile_chunks(a.chunks_cap);
  const uint32_t tiles = a.chunks_cap ? (a.chunks_cap + T - 1u) / T : 1u;
  hipLaunchKernelGGL(scan_kernel, dim3(tiles), dim3(kBlock), 0, stream, a.in, a.in_bytes, a.out_capacity,
                     a.chunks_cap, T, (DecP*)a.params, a.loc, a.tile_sums, a.tile_err, a.status, a.out_bytes);
  if (a.ev_start && hipEventRecord(a.ev_start, stream) != hipSuccess) return hipErrorUnknown;
  if (a.chunks_cap > 0) {
    uint32_t grid = (a.chunks_cap + kWaves - 1u) / kWaves;
    if (grid > kMaxGrid) grid = kMaxGrid;
    hipLaunchKernelGGL(chunks_kernel, dim3(grid), dim3(kBlock), 0, stream, a.in, a.in_bytes, a.out,
                       (const DecP*)a.params, (const uint32_t*)a.loc, (const uint64_t*)a.tile_sums,
                       (const uint32_t*)a.tile_err, a.status, a.out_bytes);
  }
  if (a.ev_stop && hipEventRecord(a.ev_stop, stream) != hipSuccess) return hipErrorUnknown;
  return hipGetLastError();
}

}  // namespace gpulz
