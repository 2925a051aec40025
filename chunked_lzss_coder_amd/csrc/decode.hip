// decode.hip -- stream decode for gfx950.
//
// The header and size table are read on the device, so nothing waits on the
// host and the call can be captured (the GPULZStage page notes that its own
// inverse needs blocking header reads; this one does not).
//   header_kernel:   validate the 32-byte header, capacity check, params;
//   tile_sums:       per tile, validate entries and sum payload sizes;
//   scan_tiles:      exclusive scan of tile sums, total must equal the header;
//   chunk_offsets:   offsets of every chunk's payload;
//   decode_chunks:   one workgroup per chunk (block-parallel decode paragraph):
//       zero entry -> zero fill; raw entry -> copy; otherwise
//       a. item k's token position follows from the flag popcount before k
//          (literal = word_size bytes, match = 2 bytes);
//       b. one workgroup scan of item output lengths gives every item's
//          output position; all token rules are checked here;
//       c. every element of a match item points into the data before the
//          match (q -> start - O + (q - start) mod O, always < start), then
//          pointer jumping resolves chains in at most log2(E)+1 rounds with
//          early exit (block-parallel decode paragraph);
//       d. coalesced stores of the chunk's real bytes;
//   finalize:        publish the status, zero the length on error.
#include "common.h"

namespace gpulz {
namespace {

constexpr uint32_t kMaxE = 4096;               // cs 4096 / ws 1
constexpr uint32_t kMaxItems = kMaxE + 8;      // 8 * ceil(E/8)
constexpr uint32_t kMaxW = kMaxItems / 32 + 1;  // bitmap words over items or elements

__device__ __forceinline__ uint32_t ld_u32_bytes(const uint8_t* p) {
  return (uint32_t)p[0] | ((uint32_t)p[1] << 8) | ((uint32_t)p[2] << 16) | ((uint32_t)p[3] << 24);
}
__device__ __forceinline__ uint64_t ld_u64_bytes(const uint8_t* p) {
  return (uint64_t)ld_u32_bytes(p) | ((uint64_t)ld_u32_bytes(p + 4) << 32);
}
__device__ __forceinline__ void flag_error(DecodeParams* P) { atomicMax(&P->status, kStatusCorrupt); }

__device__ __forceinline__ uint32_t chunk_real_bytes(const DecodeParams& P, uint64_t c) {
  const uint64_t start = c * P.cs;
  return (uint32_t)((P.n - start) < P.cs ? (P.n - start) : P.cs);
}

__global__ void header_kernel(const uint8_t* __restrict__ in, uint64_t in_bytes, uint64_t out_capacity,
                              uint32_t chunks_cap, DecodeParams* __restrict__ P, uint32_t* __restrict__ status,
                              uint64_t* __restrict__ out_bytes) {
  if (threadIdx.x != 0) return;
  const uint32_t magic = ld_u32_bytes(in);
  const uint32_t ver = in[4], ws = in[5], res = in[6] | ((uint32_t)in[7] << 8);
  const uint32_t cs = ld_u32_bytes(in + 8), nc = ld_u32_bytes(in + 12);
  const uint64_t n = ld_u64_bytes(in + 16), pb = ld_u64_bytes(in + 24);
  uint32_t st = kStatusOk;
  if (magic != kMagic || ver != kVersion || res != 0 || !word_size_ok(ws) || !chunk_size_ok(cs)) {
    st = kStatusCorrupt;
  } else {
    const uint64_t want_nc = n / cs + ((n % cs) != 0);
    const uint64_t total = (uint64_t)kHeaderBytes + (uint64_t)kEntryBytes * nc + pb;
    if (want_nc != nc || pb > n || pb > in_bytes || total > in_bytes) st = kStatusCorrupt;
    else if (n > out_capacity) st = kStatusCapacity;
    else if (nc > chunks_cap) st = kStatusCorrupt;
  }
  P->n = n;
  P->payload_bytes = pb;
  P->payload_base = (uint64_t)kHeaderBytes + (uint64_t)kEntryBytes * nc;
  P->cs = cs;
  P->ws = ws;
  P->num_chunks = nc;
  P->status = st;
  *status = st;
  *out_bytes = st == kStatusOk ? n : 0u;
}

__device__ __forceinline__ uint2 read_entry(const uint8_t* in, uint64_t c) {
  const uint8_t* e = in + kHeaderBytes + kEntryBytes * c;
  return make_uint2(ld_u32_bytes(e), ld_u32_bytes(e + 4));
}

__device__ __forceinline__ bool entry_ok(uint2 e, uint32_t bc) {
  if (e.x == 0u) return e.y == 0u || ((e.y & kRawBit) && (e.y & ~kRawBit) == bc);
  return !(e.y & kRawBit) && (uint64_t)e.x + e.y < bc;
}

__global__ __launch_bounds__(kBlock) void dec_tile_sums_kernel(const uint8_t* __restrict__ in,
                                                               DecodeParams* __restrict__ P,
                                                               uint64_t* __restrict__ tile_sums) {
  __shared__ uint64_t sh[kWaves];
  const DecodeParams p = *P;
  if (p.status != kStatusOk) return;
  const uint64_t t = blockIdx.x;
  if (t * kTile >= p.num_chunks) return;
  uint64_t s = 0;
  bool bad = false;
  for (uint32_t i = threadIdx.x; i < kTile; i += kBlock) {
    const uint64_t c = t * kTile + i;
    if (c < p.num_chunks) {
      const uint2 e = read_entry(in, c);
      bad |= !entry_ok(e, chunk_real_bytes(p, c));
      s += entry_payload(e.x, e.y);
    }
  }
  if (bad) flag_error(P);
  s = block_sum(s, sh);
  if (threadIdx.x == 0) tile_sums[t] = s;
}

__global__ __launch_bounds__(kBlock) void dec_scan_tiles_kernel(DecodeParams* __restrict__ P,
                                                                uint64_t* __restrict__ tile_sums) {
  __shared__ uint64_t sh[kWaves];
  if (P->status != kStatusOk) return;
  const uint32_t num_tiles = (P->num_chunks + kTile - 1) / kTile;
  uint64_t carry = 0;
  for (uint32_t b = 0; b < num_tiles; b += kBlock) {
    const uint32_t i = b + threadIdx.x;
    const uint64_t v = i < num_tiles ? tile_sums[i] : 0;
    uint64_t tot;
    const uint64_t ex = block_exclusive_scan(v, &tot, sh);
    if (i < num_tiles) tile_sums[i] = carry + ex;
    carry += tot;
  }
  if (threadIdx.x == 0 && carry != P->payload_bytes) flag_error(P);
}

__global__ __launch_bounds__(kBlock) void dec_offsets_kernel(const uint8_t* __restrict__ in,
                                                             const DecodeParams* __restrict__ P,
                                                             const uint64_t* __restrict__ tile_prefix,
                                                             uint64_t* __restrict__ offsets) {
  __shared__ uint64_t sh[kWaves];
  constexpr uint32_t PER = kTile / kBlock;
  const DecodeParams p = *P;
  if (p.status != kStatusOk) return;
  const uint64_t t = blockIdx.x;
  if (t * kTile >= p.num_chunks) return;
  const uint64_t c0 = t * kTile + (uint64_t)threadIdx.x * PER;
  uint32_t sz[PER];
  uint64_t local = 0;
#pragma unroll
  for (uint32_t j = 0; j < PER; ++j) {
    sz[j] = 0;
    if (c0 + j < p.num_chunks) {
      const uint2 e = read_entry(in, c0 + j);
      sz[j] = entry_payload(e.x, e.y);
    }
    local += sz[j];
  }
  uint64_t tot;
  uint64_t off = tile_prefix[t] + block_exclusive_scan(local, &tot, sh);
#pragma unroll
  for (uint32_t j = 0; j < PER; ++j) {
    if (c0 + j < p.num_chunks) offsets[c0 + j] = off;
    off += sz[j];
  }
}

// Write n bytes of zeros / of a word source at dst (any alignment).
__device__ __forceinline__ void store_word_or_bytes(uint8_t* dst, uint32_t i, uint32_t v, uint32_t nbytes,
                                                    bool aligned) {
  // word i covers bytes [4i, 4i+4) of dst; only bytes < nbytes are written
  const uint32_t b0 = 4u * i;
  if (aligned && b0 + 4u <= nbytes) {
    *(uint32_t*)(dst + b0) = v;
  } else {
    for (uint32_t b = 0; b < 4u; ++b)
      if (b0 + b < nbytes) dst[b0 + b] = (uint8_t)(v >> (8u * b));
  }
}

struct DecShared {
  uint32_t pb[kMaxE / 4 + 4];     // payload bytes (flags then data)
  uint32_t val[kMaxE];            // decoded element values
  uint16_t src[kMaxE];            // pointer-jumping source per element
  uint16_t iop[kMaxItems];        // item output position (saturated)
  uint16_t itp[kMaxItems];        // item token position in the data bytes
  uint32_t fw[kMaxW];             // flag bitmap as words
  uint32_t fpre[kMaxW + 1];       // matches before flag word w
  uint32_t starts[kMaxW];         // item start bitmap over elements
  uint32_t spre[kMaxW + 1];       // items before element word w
  uint32_t scan_sh[2 * kWaves];
  uint64_t red_sh[kWaves];
};

__global__ __launch_bounds__(kBlock) void decode_chunks_kernel(const uint8_t* __restrict__ in, uint64_t in_bytes,
                                                               DecodeParams* __restrict__ P,
                                                               const uint64_t* __restrict__ offsets,
                                                               uint8_t* __restrict__ out) {
  __shared__ DecShared S;
  const DecodeParams p = *P;
  if (p.status != kStatusOk) return;
  const uint32_t tid = threadIdx.x;
  const uint32_t ws = p.ws, cs = p.cs, E = cs / ws;
  const uint8_t* lim = in + in_bytes;
  const uint8_t* pay0 = in + p.payload_base;
  uint8_t* PB = (uint8_t*)S.pb;

  for (uint64_t c = blockIdx.x; c < p.num_chunks; c += gridDim.x) {
    const uint2 e = read_entry(in, c);
    const uint32_t bc = chunk_real_bytes(p, c);
    uint8_t* dst = out + c * cs;
    const bool dal = (((uintptr_t)dst) & 3u) == 0;
    const uint8_t* src = pay0 + offsets[c];
    const uint32_t nwords = (bc + 3u) / 4u;
    if (e.x == 0u && e.y == 0u) {
      for (uint32_t i = tid; i < nwords; i += kBlock) store_word_or_bytes(dst, i, 0u, bc, dal);
      continue;
    }
    if (e.x == 0u) {  // raw
      for (uint32_t i = tid; i < nwords; i += kBlock)
        store_word_or_bytes(dst, i, load4_unaligned(src + 4u * i, lim), bc, dal);
      continue;
    }
    const uint32_t F = e.x, D = e.y;
    if (F > (E + 7u) / 8u) {  // more flag bytes than a chunk can have items
      if (tid == 0) flag_error(P);
      continue;
    }
    // ---- load payload, flag words ---------------------------------------------
    const uint32_t sbytes = F + D;
    for (uint32_t i = tid; i < (sbytes + 3u) / 4u; i += kBlock) S.pb[i] = load4_unaligned(src + 4u * i, lim);
    __syncthreads();
    const uint32_t NI = 8u * F;
    const uint32_t NW = (NI + 31u) / 32u;
    for (uint32_t w = tid; w < NW; w += kBlock) {
      uint32_t v = 0;
      for (uint32_t b = 0; b < 4u; ++b)
        if (4u * w + b < F) v |= (uint32_t)PB[4u * w + b] << (8u * b);
      S.fw[w] = v;
    }
    __syncthreads();
    if (tid == 0) {
      uint32_t a = 0;
      for (uint32_t w = 0; w < NW; ++w) {
        S.fpre[w] = a;
        a += __builtin_popcount(S.fw[w]);
      }
      S.fpre[NW] = a;
    }
    __syncthreads();

    // ---- a./b. item geometry + checks -----------------------------------------
    const uint32_t IPT = (NI + kBlock - 1) / kBlock;  // items per thread (<= 17)
    const uint32_t k0 = tid * IPT;
    uint32_t lsum = 0;
    bool bad = false;
    for (uint32_t j = 0; j < IPT; ++j) {
      const uint32_t k = k0 + j;
      if (k >= NI) break;
      const uint32_t w = k >> 5, bit = 1u << (k & 31u);
      const uint32_t m = S.fpre[w] + __builtin_popcount(S.fw[w] & (bit - 1u));
      const uint32_t tp = ws * (k - m) + 2u * m;
      const bool mt = (S.fw[w] & bit) != 0u;
      const bool readable = tp + (mt ? 2u : ws) <= D;
      uint32_t len = 0;
      if (readable) len = mt ? PB[F + tp] : 1u;
      S.itp[k] = (uint16_t)(tp < 0xFFFFu ? tp : 0xFFFFu);
      lsum += len;
    }
    uint32_t tot;
    uint32_t op = block_exclusive_scan(lsum, &tot, S.scan_sh);
    uint32_t live = 0, live_len = 0;
    for (uint32_t j = 0; j < IPT; ++j) {
      const uint32_t k = k0 + j;
      if (k >= NI) break;
      const uint32_t w = k >> 5, bit = 1u << (k & 31u);
      const bool mt = (S.fw[w] & bit) != 0u;
      const uint32_t tp = S.itp[k];
      const bool readable = tp + (mt ? 2u : ws) <= D;
      uint32_t len = 0;
      if (readable) len = mt ? PB[F + tp] : 1u;
      S.iop[k] = (uint16_t)(op < 0xFFFFu ? op : 0xFFFFu);
      if (op < E) {  // a live item: the walk reaches it
        ++live;
        live_len += len;
        if (!readable) bad = true;
        if (mt) {
          const uint32_t O = readable ? PB[F + tp + 1] : 0u;
          if (len == 0u || O == 0u || O > op || op + len > E) bad = true;
        }
      }
      op += len;
    }
    const uint32_t K = block_sum(live, S.scan_sh);
    const uint32_t LL = block_sum(live_len, S.scan_sh);
    // the pad bits after the last live item and the data length must agree
    if (tid == 0) {
      if (LL != E || (K + 7u) / 8u != F) bad = true;
      uint32_t mK;
      if (K >= NI) mK = S.fpre[NW];
      else mK = S.fpre[K >> 5] + __builtin_popcount(S.fw[K >> 5] & ((1u << (K & 31u)) - 1u));
      if (ws * (K - mK) + 2u * mK != D) bad = true;
      if (mK != S.fpre[NW]) bad = true;  // a set flag bit past the last item
    }
    if (__syncthreads_or(bad)) {
      if (tid == 0) flag_error(P);
      continue;
    }

    // ---- c. element sources, pointer jumping -----------------------------------
    const uint32_t EW = E / 32u;
    for (uint32_t w = tid; w < EW; w += kBlock) S.starts[w] = 0u;
    __syncthreads();
    for (uint32_t j = 0; j < IPT; ++j) {
      const uint32_t k = k0 + j;
      if (k >= K) break;
      const uint32_t q = S.iop[k];
      atomicOr(&S.starts[q >> 5], 1u << (q & 31u));
    }
    __syncthreads();
    if (tid == 0) {
      uint32_t a = 0;
      for (uint32_t w = 0; w < EW; ++w) {
        S.spre[w] = a;
        a += __builtin_popcount(S.starts[w]);
      }
    }
    __syncthreads();
    for (uint32_t q = tid; q < E; q += kBlock) {
      const uint32_t w = q >> 5, b = q & 31u;
      const uint32_t upto = b == 31u ? ~0u : ((2u << b) - 1u);
      const uint32_t k = S.spre[w] + __builtin_popcount(S.starts[w] & upto) - 1u;
      const uint32_t tp = S.itp[k];
      if (S.fw[k >> 5] & (1u << (k & 31u))) {
        const uint32_t st = S.iop[k];
        const uint32_t O = PB[F + tp + 1];
        S.src[q] = (uint16_t)(st - O + (q - st) % O);
      } else {
        uint32_t v = 0;
        for (uint32_t bb = 0; bb < ws; ++bb) v |= (uint32_t)PB[F + tp + bb] << (8u * bb);
        S.val[q] = v;
        S.src[q] = (uint16_t)q;
      }
    }
    __syncthreads();
    for (int round = 0; round < 16; ++round) {
      bool unres = false;
      uint32_t ns[kMaxE / kBlock], nv[kMaxE / kBlock], sq[kMaxE / kBlock];
#pragma unroll
      for (uint32_t i = 0; i < kMaxE / kBlock; ++i) {
        const uint32_t q = tid + i * kBlock;
        sq[i] = q;
        if (q < E) {
          const uint32_t s = S.src[q];
          sq[i] = s;
          if (s != q) {
            ns[i] = S.src[s];
            nv[i] = S.val[s];
          }
        }
      }
      __syncthreads();
#pragma unroll
      for (uint32_t i = 0; i < kMaxE / kBlock; ++i) {
        const uint32_t q = tid + i * kBlock;
        if (q < E && sq[i] != q) {
          if (ns[i] == sq[i]) {
            S.val[q] = nv[i];
            S.src[q] = (uint16_t)q;
          } else {
            S.src[q] = (uint16_t)ns[i];
            unres = true;
          }
        }
      }
      if (!__syncthreads_or(unres)) break;
    }

    // ---- d. store the real bytes; the padding must have decoded to zero ---------
    bool padbad = false;
    for (uint32_t i = tid; i < cs / 4u; i += kBlock) {
      uint32_t v;
      if (ws == 4u) v = S.val[i];
      else if (ws == 2u) v = (S.val[2 * i] & 0xFFFFu) | (S.val[2 * i + 1] << 16);
      else v = (S.val[4 * i] & 0xFFu) | ((S.val[4 * i + 1] & 0xFFu) << 8) | ((S.val[4 * i + 2] & 0xFFu) << 16) |
               (S.val[4 * i + 3] << 24);
      if (4u * i + 4u > bc) {  // word reaching into the zero padding
        const uint32_t keep = 4u * i >= bc ? 0u : (bc - 4u * i);
        const uint32_t padmask = keep >= 4u ? 0u : (~0u << (8u * keep));
        if (v & padmask) padbad = true;
      }
      if (4u * i < bc) store_word_or_bytes(dst, i, v, bc, dal);
    }
    if (__syncthreads_or(padbad) && tid == 0) flag_error(P);
  }
}

__global__ void finalize_kernel(const DecodeParams* __restrict__ P, uint32_t* __restrict__ status,
                                uint64_t* __restrict__ out_bytes) {
  if (threadIdx.x != 0) return;
  const uint32_t st = P->status;
  *status = st;
  if (st != kStatusOk) *out_bytes = 0u;
}

}  // namespace

hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL(header_kernel, dim3(1), dim3(64), 0, stream, a.in, a.in_bytes, a.out_capacity, a.chunks_cap,
                     a.params, a.status, a.out_bytes);
  if (a.chunks_cap > 0) {
    hipLaunchKernelGGL(dec_tile_sums_kernel, dim3(a.tiles_cap), dim3(kBlock), 0, stream, a.in, a.params,
                       a.tile_sums);
    hipLaunchKernelGGL(dec_scan_tiles_kernel, dim3(1), dim3(kBlock), 0, stream, a.params, a.tile_sums);
    hipLaunchKernelGGL(dec_offsets_kernel, dim3(a.tiles_cap), dim3(kBlock), 0, stream, a.in,
                       (const DecodeParams*)a.params, (const uint64_t*)a.tile_sums, a.offsets);
    const uint32_t grid = a.chunks_cap < kMaxGrid ? a.chunks_cap : kMaxGrid;
    if (a.ev_start && hipEventRecord(a.ev_start, stream) != hipSuccess) return hipErrorUnknown;
    hipLaunchKernelGGL(decode_chunks_kernel, dim3(grid), dim3(kBlock), 0, stream, a.in, a.in_bytes, a.params,
                       (const uint64_t*)a.offsets, a.out);
    if (a.ev_stop && hipEventRecord(a.ev_stop, stream) != hipSuccess) return hipErrorUnknown;
  } else {
    if (a.ev_start && hipEventRecord(a.ev_start, stream) != hipSuccess) return hipErrorUnknown;
    if (a.ev_stop && hipEventRecord(a.ev_stop, stream) != hipSuccess) return hipErrorUnknown;
  }
  hipLaunchKernelGGL(finalize_kernel, dim3(1), dim3(64), 0, stream, (const DecodeParams*)a.params, a.status,
                     a.out_bytes);
  return hipGetLastError();
}

}  // namespace gpulz
