// decode.hip -- stream decode for gfx950 (two kernels, no host round trip).
//
// The header and size table are read on the device, so nothing waits on the
// host (the GPULZStage page's own inverse reads the header with blocking
// copies before it can launch; this one can be captured).
//
// scan_kernel (one workgroup per tile of T chunks, T sized on the device from
//   the header's chunk count; scan_tiles.h states the bounds): checks the
//   header, writes the parameters, the initial status and length; validates
//   every size-table row against its chunk's real bytes, writes each chunk's
//   payload offset within its tile, the tile's total and an error flag.
//   No workgroup waits on another.
// chunks_kernel (one wave per chunk; the four waves of a workgroup per
//   chunk when a chunk has more than 1024 elements, or has 1024 and the
//   stream fewer than 2048 chunks): the chunk's payload offset is its tile's
//   offset (sum of earlier tile totals) plus its offset in the tile; then
//     zero row -> zero fill; raw row -> copy; otherwise, per the
//     block-parallel decode paragraph of the GPULZStage page:
//     a. the payload is staged in LDS; lane g walks items [gR, gR + R) (R =
//        items per lane): an item's data offset follows from the matches
//        before it (flag popcounts, one team scan), its output length is 1
//        or the token's length, and a second team scan of the lengths gives
//        every item's output position; every token rule is checked (per
//        item what only the item shows, the rest through the counts after
//        the item that ends the chunk);
//     b. each element of a match item points into the data before the item,
//        start - O + (q - start) mod O, always < start; pointer jumping
//        resolves chains in at most log2(items)+1 rounds with early exit (a
//        one-wave chunk's 64-element windows in order, those in which no
//        item starts without any);
//     c. the chunk's real bytes are stored; the zero padding must have
//        decoded to zeros.
//   Errors only ever raise the status (and zero the length), so the kernel
//   order makes the first write of the status the header kernel's.
#include <type_traits>

#include "common.h"
#include "scan_tiles.h"

namespace gpulz {
namespace {

constexpr uint32_t kScanPer = 4;         // chunks per thread per scan round
constexpr uint32_t kScanRound = kScanPer * kBlock;
constexpr uint32_t kDecodeGrid = 8192;   // chunk-kernel workgroups at most (chunks shared by waves)
constexpr uint32_t kDecodeGridTeams = 16384;  // the same for chunks decoded by a whole workgroup
constexpr uint32_t kMaxTilesAlloc = 4096; // split mode: stride of the three tile-total arrays
constexpr uint32_t kOneWaveMinChunks = 2048;  // overlaid chunks: one per wave from this many chunks on
static_assert(kTileMin % kScanRound == 0 && (uint64_t)kTileMax * 4096u <= (1ull << 32), "tile sizes");

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
  if ((((uintptr_t)in) & 7u) == 0) return *(const uint2*)e;  // rows are 8-byte aligned with the stream
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
                                                      uint64_t out_capacity, uint32_t chunks_cap,
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
  // Tiles are sized for the stream's own chunk count (the host only knows
  // a bound): nc <= chunks_cap, so at most the launched workgroups are needed.
  const uint32_t T = scan_tile_chunks(nc);
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
// A workgroup's LDS is kWaves slots of kSlot bytes.  A chunk whose working set
// fits one slot is decoded by one wave (kWaves chunks per workgroup at once);
// a larger one by the whole workgroup in all slots.  A chunk's arena holds
//   VAL  the decoded chunk (CS bytes);
//   PB   the payload: flag bytes, then data bytes from a 4-byte boundary;
//        after the items are read, SRC, a u16 source index per element;
//   OB   per element, the offset of the match item starting there (0: none);
//   STB  the item-start bitmap, one u64 per 64 elements.
// A one-wave chunk that would not fit one slot this way (chunk 4096 at word
// size 4) stages its payload over VAL instead (OVL): every lane reads all of
// its items into registers before any value is stored.
constexpr uint32_t kSlot = 5376;
static_assert(kSlot % 16 == 0, "arenas must stay 16-byte aligned (64-bit LDS atomics)");
constexpr uint32_t kArena = kWaves * kSlot;

template <uint32_t CS, uint32_t WS, bool TEAMS = false>
struct Geo {
  static constexpr uint32_t E = CS / WS;                       // elements per chunk
  static constexpr uint32_t PBB = (CS > 2u * E ? CS : 2u * E) + 16u;
  static constexpr uint32_t NEED = CS + PBB + E + E / 8u;
  // OVL: the payload (at most CS + 3 bytes, staged in whole dwords) shares
  // VAL's bytes, so the chunk needs CS + 16 + E + E / 8 bytes: one slot for
  // 1024 elements (chunk 4096 at word size 4), decoded by one wave.
  static constexpr bool OVL = !TEAMS && NEED > kSlot && CS + 16u + E + E / 8u <= kSlot && E <= 1024u;
  static constexpr uint32_t TW = (NEED <= kSlot || OVL) ? 1u : kWaves;  // waves per chunk
  static constexpr uint32_t PB_AT = OVL ? 0u : CS;               // byte offsets in the arena
  static constexpr uint32_t OB_AT = OVL ? CS + 16u : CS + PBB;
  static constexpr uint32_t STB_AT = OB_AT + E;
  static constexpr uint32_t TL = 64u * TW;                     // lanes per chunk
  static constexpr uint32_t J = E / TL;                        // elements per lane
  static constexpr uint32_t NB = E / 64u;                      // 64-element blocks
  static constexpr uint32_t RMAX = J + 1u;                     // items per lane, at most
  static_assert(STB_AT + E / 8u <= TW * kSlot && STB_AT % 16u == 0u, "chunk working set exceeds its arena");
  static_assert(E % TL == 0 && NB <= 64u && RMAX < 25u, "lane mapping");
};

template <uint32_t TW>
__device__ __forceinline__ void team_sync() {
  if constexpr (TW == 1) wave_sync();
  else __syncthreads();
}

// Collectives over a chunk's team.  One wave: DPP moves and ballots only.  A
// whole workgroup: every wave posts its partial to one of two LDS rows (they
// alternate between calls), one barrier, then every wave reads the row.  A row
// is written again only two calls later, after every wave has passed the
// barrier in between, so one barrier per call suffices; that barrier also
// orders all earlier LDS writes of the team.
template <uint32_t TW>
struct TeamX {
  uint32_t* rows;  // 2 x kWaves words
  uint32_t par;

  __device__ __forceinline__ uint32_t* next_row() {
    uint32_t* r = rows + par * kWaves;
    par ^= 1u;
    return r;
  }
  // exclusive scan of one value per team lane; total to *tot
  __device__ __forceinline__ uint32_t scan(uint32_t v, uint32_t* tot) {
    const uint32_t inc = wave_incl_add(v);
    const uint32_t wt = lane63(inc);
    if constexpr (TW == 1) {
      *tot = wt;
      return inc - v;
    } else {
      const uint32_t w = threadIdx.x >> 6;
      uint32_t* r = next_row();
      if (lane_id() == 0) r[w] = wt;
      __syncthreads();
      uint32_t pre = 0, t = 0;
#pragma unroll
      for (uint32_t i = 0; i < TW; ++i) {
        const uint32_t x = r[i];
        pre += i < w ? x : 0u;
        t += x;
      }
      *tot = t;
      return pre + inc - v;
    }
  }
  __device__ __forceinline__ uint32_t sum(uint32_t v) {
    uint32_t t;
    scan(v, &t);
    return t;
  }
  __device__ __forceinline__ bool any(bool b) {
    const bool wb = __ballot(b) != 0ull;
    if constexpr (TW == 1) {
      return wb;
    } else {
      uint32_t* r = next_row();
      if (lane_id() == 0) r[threadIdx.x >> 6] = wb ? 1u : 0u;
      __syncthreads();
      uint32_t o = 0;
#pragma unroll
      for (uint32_t i = 0; i < TW; ++i) o |= r[i];
      return o != 0u;
    }
  }
};

// d mod o for d < 256, 1 <= o < 256: the quotient of d + 1/2 by o is computed
// in fp32 with an approximate reciprocal; it lies at least 1/(2o) >= 1/510
// away from every integer, far beyond the reciprocal's error, so the
// truncated quotient is exact.
__device__ __forceinline__ uint32_t small_mod(uint32_t d, uint32_t o) {
  const uint32_t q = (uint32_t)(((float)d + 0.5f) * __builtin_amdgcn_rcpf((float)o));
  return d - __umul24(q, o);  // q, o < 256: a full-rate 24-bit product
}

// Split mode: where a coded chunk's items are (the GPULZStage page's
// split-mode decode paragraph: items are read straight out of the ports, no
// re-packing into one stream).
struct SplitSrc {
  const uint8_t* flags;  // its (K + 7) / 8 flag bytes, in the meta port
  const uint8_t* lit;    // its K - M literal words
  const uint8_t* lens;   // its M match lengths
  const uint8_t* offs;   // its M match offsets
  uint32_t K, M;
};

// Decode one coded chunk.  One stream: pay is its payload (F flag bytes, D
// data bytes).  Split mode: sp locates its items in the ports (pay, F, D
// unused).  bc: the chunk's real
// bytes, written to dst.  Returns false on a rule violation.
template <uint32_t CS, uint32_t WS, bool SPLIT = false, bool TEAMS = false>
__device__ __forceinline__ bool decode_coded(const uint8_t* pay, uint32_t F, uint32_t D, uint32_t bc,
                             uint8_t* dst, uint8_t* arena, uint32_t* sh, const SplitSrc& sp) {
  using G = Geo<CS, WS, TEAMS>;
  constexpr uint32_t E = G::E, TW = G::TW, TL = G::TL, J = G::J, NB = G::NB;
  TeamX<TW> tx{sh, 0u};
  const uint32_t g = threadIdx.x % TL, lane = lane_id();
  uint8_t* VAL = arena;
  uint8_t* PB = arena + G::PB_AT;
  uint16_t* SRC = (uint16_t*)PB;  // several waves per chunk only (never OVL)
  uint8_t* OB = arena + G::OB_AT;
  uint64_t* STB = (uint64_t*)(arena + G::STB_AT);

  if constexpr (SPLIT) F = (sp.K + 7u) / 8u;
  // every live item covers at least one element: at most E items, so at most
  // (E + 7) / 8 flag bytes
  if (F > (E + 7u) / 8u) return false;
  // stage len bytes from src into PB (dword i = source bytes 4i..4i+3): the
  // aligned source dwords holding a byte of [src, src + len) are read (no
  // read leaves the pages those bytes lie in), each dword realigned with the
  // one after it; up to four loads per lane in flight before their stores
  auto stage = [&](const uint8_t* src, uint32_t len) {
    const uint32_t sh = (uint32_t)((uintptr_t)src & 3u);
    const uint32_t* A = (const uint32_t*)(src - sh);
    const uint32_t nA = (sh + len + 3u) >> 2;  // aligned dwords holding a byte of the span
    const uint32_t nd = (len + 3u) >> 2;
    uint32_t* P32 = (uint32_t*)PB;
    if (nd <= TL) {  // one dword per lane
      const uint32_t a = g < nA ? A[g] : 0u;
      const uint32_t b = (sh != 0u && g + 1u < nA) ? A[g + 1u] : 0u;
      if (g < nd) P32[g] = __builtin_amdgcn_alignbyte(b, a, sh);
      return;
    }
#pragma unroll 1
    for (uint32_t i0 = 0; i0 < nd; i0 += 4u * TL) {
      uint32_t a[4], b[4];
#pragma unroll
      for (uint32_t r = 0; r < 4u; ++r) {
        const uint32_t i = i0 + g + r * TL;
        a[r] = i < nA ? A[i] : 0u;
        b[r] = (sh != 0u && i + 1u < nA) ? A[i + 1u] : 0u;
      }
#pragma unroll
      for (uint32_t r = 0; r < 4u; ++r) {
        const uint32_t i = i0 + g + r * TL;
        if (i < nd) P32[i] = __builtin_amdgcn_alignbyte(b[r], a[r], sh);
      }
    }
  };
  // ---- load the items; clear the start bitmap and the offsets -----------------------------
  // One stream: the payload, data bytes from a 4-byte boundary.  Split mode:
  // flags | literals | lengths | offsets, each from a 4-byte boundary (they
  // total F + D + 9 bytes at most, with F + D < bc).
  const uint8_t *FL, *PD, *LITB, *LENB, *OFFB;
  const uint32_t NL = SPLIT ? sp.K - sp.M : 0u;  // split: literal words
  if constexpr (SPLIT) {
    const uint32_t lo = (F + 3u) & ~3u, mo = (lo + WS * NL + 3u) & ~3u, oo = (mo + sp.M + 3u) & ~3u;
    // the four regions in one pass, so their loads are in flight together:
    // dword i of PB belongs to the region whose dword range holds it (the
    // gaps between regions get zeros); only aligned dwords holding a byte of
    // the region are read, so no read leaves the pages its bytes lie in
    const uint32_t d1 = lo >> 2, d2 = mo >> 2, d3 = oo >> 2;
    const uint32_t e0 = (F + 3u) >> 2, e1 = d1 + ((WS * NL + 3u) >> 2), e2 = d2 + ((sp.M + 3u) >> 2),
                   e3 = d3 + ((sp.M + 3u) >> 2);
    if (e0 <= TL && e1 - d1 <= TL && e2 - d2 <= TL && e3 - d3 <= TL) {
      // every region fits one dword per lane (small payloads): lane g takes
      // dword g of each, the four regions' loads issued before any store
      const uint8_t* const src4[4] = {sp.flags, sp.lit, sp.lens, sp.offs};
      const uint32_t len4[4] = {F, WS * NL, sp.M, sp.M}, at4[4] = {0u, d1, d2, d3};
      uint32_t v[4];
#pragma unroll
      for (uint32_t r = 0; r < 4u; ++r) {
        const uint32_t sh = (uint32_t)((uintptr_t)src4[r] & 3u);
        const uint32_t* A = (const uint32_t*)(src4[r] - sh);
        const uint32_t nA = (sh + len4[r] + 3u) >> 2;  // aligned dwords holding a byte of the region
        uint32_t lo = 0, hi = 0;
        if (g < ((len4[r] + 3u) >> 2)) {
          lo = A[g];
          if (sh != 0u && g + 1u < nA) hi = A[g + 1u];
        }
        v[r] = __builtin_amdgcn_alignbyte(hi, lo, sh);
      }
#pragma unroll
      for (uint32_t r = 0; r < 4u; ++r)
        if (g < ((len4[r] + 3u) >> 2)) ((uint32_t*)PB)[at4[r] + g] = v[r];
    } else {
#pragma unroll 1
      for (uint32_t i0 = 0; i0 < e3; i0 += 4u * TL) {
        uint32_t v[4];
#pragma unroll
        for (uint32_t r = 0; r < 4u; ++r) {
          const uint32_t i = i0 + g + r * TL;
          const uint8_t* src = nullptr;
          uint32_t len = 0, b = 0;
          if (i < e0) {
            src = sp.flags, len = F, b = i;
          } else if (i >= d1 && i < e1) {
            src = sp.lit, len = WS * NL, b = i - d1;
          } else if (i >= d2 && i < e2) {
            src = sp.lens, len = sp.M, b = i - d2;
          } else if (i >= d3 && i < e3) {
            src = sp.offs, len = sp.M, b = i - d3;
          }
          // the aligned dwords holding bytes 4b .. 4b + 3 (only those holding
          // a byte of the region), realigned
          uint32_t lo = 0, hi = 0, sh = 0;
          if (src) {
            sh = (uint32_t)((uintptr_t)src & 3u);
            const uint32_t* A = (const uint32_t*)(src - sh);
            const uint32_t nA = (sh + len + 3u) >> 2;
            lo = A[b];
            if (sh != 0u && b + 1u < nA) hi = A[b + 1u];
          }
          v[r] = __builtin_amdgcn_alignbyte(hi, lo, sh);
        }
#pragma unroll
        for (uint32_t r = 0; r < 4u; ++r) {
          const uint32_t i = i0 + g + r * TL;
          if (i < e3) ((uint32_t*)PB)[i] = v[r];
        }
      }
    }
    FL = PB;
    LITB = PB + lo;
    LENB = PB + mo;
    OFFB = PB + oo;
    PD = PB;
  } else {
    const uint32_t s0 = (4u - (F & 3u)) & 3u;
    stage(pay - s0, s0 + F + D);
    FL = PB + s0;
    PD = PB + s0 + F;
    LITB = LENB = OFFB = PD;
  }
  {
#pragma unroll
    for (uint32_t i = g; i < E / 4u; i += TL) ((uint32_t*)OB)[i] = 0u;
    if (g < NB) STB[g] = 0ull;
  }
  team_sync<TW>();

  // ---- a. items: lane g reads items [g*R, g*R + nit) one after another --------------------
  // An item's data (one stream: its data offset; split mode: its literal or
  // match index) follows from the matches before it; two team scans
  // (matches, then output lengths) place every item.
  const uint32_t NI = SPLIT ? sp.K : 8u * F;
  const uint32_t R = (NI + TL - 1u) / TL;  // <= RMAX
  const uint32_t k0 = g * R;
  const uint32_t nit = k0 < NI ? (NI - k0 < R ? NI - k0 : R) : 0u;
  uint32_t fb = 0;  // this lane's flag bits, item k0 in bit 0
  if (nit) {
    // flag bytes k0 / 8 .. + 3 from the two aligned LDS dwords holding them
    // (bytes past the F flag bytes land in bits past nit, masked off)
    const uint32_t fa = (uint32_t)(FL - PB) + (k0 >> 3);
    const uint32_t* fw = (const uint32_t*)(PB + (fa & ~3u));
    fb = __builtin_amdgcn_alignbyte(fw[1], fw[0], fa & 3u);
    fb = (fb >> (k0 & 7u)) & ((1u << nit) - 1u);
  }
  uint32_t mt_total;
  const uint32_t m0 = tx.scan((uint32_t)__builtin_popcount(fb), &mt_total);
  // cursor of item k: one stream, its data offset; split mode, its literal
  // index (matches: the match index m)
  const uint32_t c0 = SPLIT ? k0 - m0 : WS * (k0 - m0) + 2u * m0;
  auto advance = [&](uint32_t& cur, uint32_t& m, bool mt) {
    if constexpr (SPLIT) {
      if (mt) ++m;
      else ++cur;
    } else {
      cur += mt ? 2u : WS;
      m += mt ? 1u : 0u;
    }
  };
  // An item's record: a match's length | offset << 8, a literal's value.
  // Reads are unconditional and unchecked, and both kinds are read so the
  // walk has no branch: a cursor never passes its lane's last item by more
  // than RMAX items, so every address stays inside the chunk's arena, and an
  // item that does not fit the payload makes the totals of the live items
  // disagree with the chunk's sizes (checked after the walk).
  auto item_rec = [&](uint32_t cur, uint32_t m, bool mt) -> uint32_t {
    if constexpr (SPLIT) {
      const uint32_t mr = (uint32_t)LENB[m] | ((uint32_t)OFFB[m] << 8);
      const uint8_t* w = LITB + WS * cur;
      uint32_t lr;
      if constexpr (WS == 4) lr = *(const uint32_t*)w;  // literal words are 4-byte aligned in LDS
      else if constexpr (WS == 2) lr = (uint32_t)*(const uint16_t*)w;
      else lr = (uint32_t)*w;
      return mt ? mr : lr;
    } else {
      const uint8_t* w = PD + cur;  // 2-byte aligned for WS >= 2
      if constexpr (WS == 4) {
        // the two aligned dwords around the item, realigned (an LDS dword
        // read from a 2-byte boundary costs far more than two aligned ones);
        // PD is 4-byte aligned, so cur & 3 is the item's offset in the first
        const uint32_t* A = (const uint32_t*)(PD + (cur & ~3u));
        const uint32_t v = __builtin_amdgcn_alignbyte(A[1], A[0], cur & 3u);
        return mt ? (v & 0xFFFFu) : v;
      } else if constexpr (WS == 2) {
        return (uint32_t)*(const uint16_t*)w;
      } else {
        const uint32_t lo = *w, hi = w[1];
        return mt ? (lo | (hi << 8)) : lo;
      }
    }
  };
  uint32_t len_total = 0, op = 0;
  uint32_t rend = 0;  // 1 + the lane's item that ends at element E (0: none)
  bool badm = false;  // a live match of length 0 or reaching before the chunk
  bool pad = false;
  uint32_t* const STB32 = (uint32_t*)STB;
  // place item r of the lane (record rc) at element op
  auto place = [&](uint32_t r, bool mt, uint32_t rc) {
    const uint32_t len = mt ? (rc & 0xFFu) : 1u;
    if (r < nit && op < E) {  // live: starts before the chunk's end
      if (mt) {
        OB[op] = (uint8_t)(rc >> 8);
      } else {
        if constexpr (WS == 4) *(uint32_t*)(VAL + 4u * op) = rc;
        else if constexpr (WS == 2) *(uint16_t*)(VAL + 2u * op) = (uint16_t)rc;
        else VAL[op] = (uint8_t)rc;
      }
      atomicOr(STB32 + (op >> 5), 1u << (op & 31u));
      badm = badm || (mt && (len == 0u || (rc >> 8) - 1u >= op));
      if (op + len == E) rend = r + 1u;
    }
    op += len;
  };
  // split mode: the flag bits past the last item must be 0 (read before OVL
  // values may land on the flag bytes)
  auto pad_bits = [&]() { return SPLIT && (sp.K & 7u) != 0u && (FL[F - 1u] >> (sp.K & 7u)) != 0u; };
  // the lane's output length: one element per literal (nit - popcount(fb)
  // of them), plus the match lengths summed in the walk
  const uint32_t lit_len = nit - (uint32_t)__builtin_popcount(fb);
  if constexpr (G::OVL) {
    // Every lane reads all its items into registers (unrolled, so the
    // records stay registers) before any value lands on the payload bytes.
    // The walk is instantiated for 2, 4, 8, 12 and 16 items per lane and the
    // wave takes the smallest that holds R (a wave uniform), so a chunk with
    // few items per lane does not step through RMAX masked slots.
    auto walk = [&](auto nr) {
      constexpr uint32_t NR = decltype(nr)::value;
      uint32_t rec[NR];
      uint32_t sum = lit_len, cur = c0, m = m0;
#pragma unroll
      for (uint32_t r = 0; r < NR; ++r) {
        const bool mt = (fb >> r) & 1u;  // 0 past the lane's items
        rec[r] = item_rec(cur, m, mt);
        sum += mt ? (rec[r] & 0xFFu) : 0u;
        advance(cur, m, mt);
      }
      op = tx.scan(sum, &len_total);
      pad = pad_bits();
      wave_sync();
      // the flag bits again through a DPP identity move, so the compiler
      // takes each item's kind afresh here rather than keeping all NR lane
      // masks of the reading loop alive across the scan
      const uint32_t fbp = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)fb, 0xE4, 0xF, 0xF, false);
#pragma unroll
      for (uint32_t r = 0; r < NR; ++r) place(r, (fbp >> r) & 1u, rec[r]);
    };
    // F <= (E + 7) / 8 was checked, so R <= 8F / 64 = E / 512 * 8 <= 16
    static_assert(E <= 1024u, "at most 16 items per lane");
    if (R <= 2u) walk(std::integral_constant<uint32_t, 2u>{});
    else if (R <= 4u) walk(std::integral_constant<uint32_t, 4u>{});
    else if (R <= 8u) walk(std::integral_constant<uint32_t, 8u>{});
    else if (R <= 12u) walk(std::integral_constant<uint32_t, 12u>{});
    else walk(std::integral_constant<uint32_t, 16u>{});
  } else {
    // R (<= RMAX) bounds every lane's items
    uint32_t sum = lit_len;
    {
      uint32_t cur = c0, m = m0;
#pragma unroll 2
      for (uint32_t r = 0; r < R; ++r) {
        const bool mt = (fb >> r) & 1u;
        const uint32_t lb = SPLIT ? (uint32_t)LENB[m] : (uint32_t)PD[cur];  // read unconditionally
        sum += mt ? lb : 0u;
        advance(cur, m, mt);
      }
    }
    op = tx.scan(sum, &len_total);
    pad = pad_bits();
    uint32_t cur = c0, m = m0;
#pragma unroll 2
    for (uint32_t r = 0; r < R; ++r) {
      const bool mt = (fb >> r) & 1u;
      place(r, mt, item_rec(cur, m, mt));
      advance(cur, m, mt);
    }
  }
  {
    // The lane holding the item that ends the chunk reports the item count,
    // the data cursor and the match count after that item (at most one lane
    // does, unless the items are bad).  Item counts <= 4103 (13 bits), lane
    // counts <= 256 (9 bits), cursors <= 4 * 4103 (16 bits).
    uint32_t endl = 0, cend = 0;
    if (rend) {
      const uint32_t mm = (uint32_t)__builtin_popcount(fb & ((1u << rend) - 1u));  // rend <= RMAX < 25
      endl = (k0 + rend) | (1u << 13);
      cend = (SPLIT ? 0u : c0 + WS * (rend - mm) + 2u * mm) | ((m0 + mm) << 16);
    }
    const uint32_t r0 = tx.sum(endl | ((badm ? 1u : 0u) << 22));
    const uint32_t r1 = tx.sum(cend);
    const uint32_t Kt = r0 & 0x1FFFu, endst = (r0 >> 13) & 0x1FFu, badt = r0 >> 22;
    const uint32_t Dt = r1 & 0xFFFFu, MKt = r1 >> 16;
    if constexpr (SPLIT) {
      // all K items are live and cover exactly E elements, M of them are
      // matches, and the flag bits past the last item are 0
      if (badt || endst != 1u || Kt != sp.K || MKt != sp.M || mt_total != sp.M || pad) return false;
    } else {
      // the live items cover exactly E elements, use exactly D data bytes and
      // leave no match flag set after the last of them
      if (badt || endst != 1u || (Kt + 7u) / 8u != F || Dt != D || MKt != mt_total) return false;
    }
  }
  team_sync<TW>();

  // ---- b. element sources: start - O + (q - start) mod O, always < start -----------------
  // lane l (< NB) holds the last item start in 64-element block l; an exclusive
  // prefix maximum gives the last start before each block
  uint32_t before;
  {
    uint32_t run = 0;
    if (lane < NB) {
      const uint64_t m = STB[lane];
      run = m ? 64u * lane + 63u - (uint32_t)__builtin_clzll(m) : 0u;
    }
    before = dpp0<kWaveShr1>(wave_incl_max(run));
  }
  const uint32_t wv = __builtin_amdgcn_readfirstlane(g >> 6);  // wave within the team
  const uint64_t upto = lane == 63u ? ~0ull : ((2ull << lane) - 1ull);
  if constexpr (TW == 1) {
    // One wave: 64-element windows in order, lane i on element 64w + i.  A
    // source before the window already holds its final value; one inside it
    // is followed over the window's lanes (pointer jumping on lane indices;
    // every link goes to a lower lane, so six rounds suffice) to an element
    // that is final (a literal, or one whose source lies before the window).
    // A window in which no item starts lies inside one match (items are
    // contiguous and a literal covers one element), all of whose sources
    // lie before it, so its sources take no start search and no jumps.  The
    // sources of four windows are found first (indices only, independent of
    // each other), then their values are copied window by window.
    static_assert(NB % 4u == 0u, "windows in groups of four");
#pragma unroll 1
    for (uint32_t w0 = 0; w0 < NB; w0 += 4u) {
      // x: bits 0-15 the source element; bits 16+ the byte address (4 x lane)
      // of the lane it still links to, or 256 once the source is final
      // (ds_bpermute reads lane (address / 4) mod 64, so 256 stays harmless)
      uint32_t x[4];
#pragma unroll
      for (uint32_t j = 0; j < 4u; ++j) {
        const uint32_t w = w0 + j;
        const uint32_t base = 64u * w, q = base + lane;
        const uint64_t mw = STB[w];  // the same word in every lane
        const uint32_t bw = (uint32_t)__builtin_amdgcn_readlane((int)before, (int)w);
        if (__builtin_amdgcn_readfirstlane((int)((uint32_t)mw | (uint32_t)(mw >> 32))) == 0) {
          const uint32_t O = OB[bw];
          x[j] = (bw - O + small_mod(q - bw, O)) | (256u << 16);
        } else {
          const uint64_t m = mw & upto;
          const uint32_t st = m ? base + 63u - (uint32_t)__builtin_clzll(m) : bw;
          const uint32_t O = OB[st];
          const uint32_t e0 = O ? st - O + small_mod(q - st, O) : q;
          const uint32_t r = e0 - base;  // < 64 iff the source lies in this window
          x[j] = e0 | ((O && r < 64u ? r << 2 : 256u) << 16);
        }
      }
      // the four windows jump in step: one exchange per window per round
      for (uint32_t round = 0;; ++round) {
        bool open[4];
        uint64_t any = 0;
#pragma unroll
        for (uint32_t j = 0; j < 4u; ++j) {
          open[j] = (x[j] >> 16) < 256u;
          any |= __ballot(open[j]);
        }
        if (!any) break;
        if (round == 6u) return false;  // unreachable for validated items
        uint32_t y[4];
#pragma unroll
        for (uint32_t j = 0; j < 4u; ++j) y[j] = (uint32_t)__builtin_amdgcn_ds_bpermute((int)(x[j] >> 16), (int)x[j]);
#pragma unroll
        for (uint32_t j = 0; j < 4u; ++j)
          if (open[j]) x[j] = y[j];
      }
      uint32_t src[4];
#pragma unroll
      for (uint32_t j = 0; j < 4u; ++j) src[j] = x[j] & 0xFFFFu;
#pragma unroll
      for (uint32_t j = 0; j < 4u; ++j) {
        const uint32_t q = 64u * (w0 + j) + lane, e = src[j];
        if (e != q) {
          if constexpr (WS == 4) *(uint32_t*)(VAL + 4u * q) = *(const uint32_t*)(VAL + 4u * e);
          else if constexpr (WS == 2) *(uint16_t*)(VAL + 2u * q) = *(const uint16_t*)(VAL + 2u * e);
          else VAL[q] = VAL[e];
        }
      }
    }
  } else {
    uint32_t src[J];
    uint32_t pend = 0;  // bit j: element j still points at a match element
#pragma unroll
    for (uint32_t j = 0; j < J; ++j) {
      const uint32_t blk = wv + TW * j;  // element q's block, uniform in the wave
      const uint32_t q = 64u * blk + lane;
      const uint64_t m = STB[blk] & upto;
      const uint32_t st = m ? 64u * blk + 63u - (uint32_t)__builtin_clzll(m)
                            : (uint32_t)__builtin_amdgcn_readlane((int)before, (int)blk);
      const uint32_t O = OB[st];
      const uint32_t s = O ? st - O + small_mod(q - st, O) : q;
      src[j] = s;
      SRC[q] = (uint16_t)s;
      if (O) pend |= 1u << j;
    }
    // pointer jumping: a source that is itself a literal ends the chain (the
    // exchange's barrier at the top of each round orders the writes before it)
    for (uint32_t round = 0;; ++round) {
      if (!tx.any(pend != 0u)) break;
      if (round == 16u) return false;  // chains resolve within log2(E) + 1 rounds
#pragma unroll
      for (uint32_t j = 0; j < J; ++j) {
        if ((pend >> j) & 1u) {
          const uint32_t s2 = SRC[src[j]];
          if (s2 == src[j]) {
            pend &= ~(1u << j);
          } else {
            src[j] = s2;
            SRC[64u * (wv + TW * j) + lane] = (uint16_t)s2;
          }
        }
      }
    }
    // copy every match element from its literal
#pragma unroll
    for (uint32_t j = 0; j < J; ++j) {
      const uint32_t q = 64u * (wv + TW * j) + lane;
      if (src[j] != q) {
        if constexpr (WS == 4) *(uint32_t*)(VAL + 4u * q) = *(const uint32_t*)(VAL + 4u * src[j]);
        else if constexpr (WS == 2) *(uint16_t*)(VAL + 2u * q) = *(const uint16_t*)(VAL + 2u * src[j]);
        else VAL[q] = VAL[src[j]];
      }
    }
  }
  team_sync<TW>();

  // ---- c. store the real bytes; the padding must have decoded to zeros -----------------
  const uintptr_t da = (uintptr_t)dst;
  bool padbad = false;
  for (uint32_t i = g; i < CS / 16u; i += TL) {
    const uint4 v = *(const uint4*)(VAL + 16u * i);
    const uint32_t b0 = 16u * i;
    if (b0 + 16u <= bc && (da & 15u) == 0u) {
      *(uint4*)(dst + b0) = v;
      continue;
    }
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (uint32_t t = 0; t < 4u; ++t) {
      const uint32_t a = b0 + 4u * t;
      if (a + 4u <= bc && (da & 3u) == 0u) {
        *(uint32_t*)(dst + a) = w[t];
      } else {
        for (uint32_t bb = 0; bb < 4u; ++bb) {
          const uint8_t x = (uint8_t)(w[t] >> (8u * bb));
          if (a + bb < bc) dst[a + bb] = x;
          else if (x) padbad = true;
        }
      }
    }
  }
  return !tx.any(padbad);
}

template <uint32_t CS, uint32_t WS, bool TEAMS>
__device__ __forceinline__ void decode_group_teams(const DecP& p, const uint8_t* in, uint8_t* out,
                                                   const uint32_t* loc, const uint64_t* tile_sum, uint32_t* status,
                                                   uint64_t* out_bytes, uint8_t* arena_all, uint32_t* sh,
                                                   uint64_t pre) {
  using G = Geo<CS, WS, TEAMS>;
  constexpr uint32_t TL = G::TL;
  constexpr uint32_t CPW = kWaves / G::TW;  // chunks per workgroup
  // the team index is a wave uniform (TL is a multiple of 64): kept in a
  // scalar register, so is every LDS base derived from it
  const uint32_t team = (uint32_t)__builtin_amdgcn_readfirstlane((int)(threadIdx.x / TL)), g = threadIdx.x % TL;
  uint8_t* arena = arena_all + team * (G::TW * kSlot);
  // The metadata of 64 of the team's chunks (size-table row and payload
  // offset) is loaded at once, one chunk per lane, and handed out by
  // readlane: one load latency per 64 chunks, not one per chunk.  A payload
  // offset is its tile's offset (the earlier tiles' totals: lane t of `pre`
  // for streams of up to 64 tiles) plus its offset within the tile.
  // Chunks decoded a workgroup each use the whole grid (up to one chunk per
  // workgroup, so one chunk's serial phases overlap other workgroups', not
  // wait in line); chunks shared by waves use at most kDecodeGrid workgroups
  // (each wave then covers enough chunks to use its metadata batches), the
  // rest of the grid leaves at once.
  const uint32_t grid = (CPW > 1u && gridDim.x > kDecodeGrid) ? kDecodeGrid : gridDim.x;
  if (blockIdx.x >= grid) return;
  const uint64_t stride = (uint64_t)grid * CPW;
  const uint64_t c0 = (uint64_t)blockIdx.x * CPW + team;
  const uint32_t lane = lane_id();
  uint2 me = make_uint2(0u, 0u);
  uint64_t moff = 0;
  auto batch = [&](uint64_t k0) {
    const uint64_t cc = c0 + (k0 + lane) * stride;
    const bool live = cc < p.nc;
    const uint32_t t = live ? (uint32_t)(cc >> __builtin_ctz(p.T)) : 0u;
    const uint32_t lo = (uint32_t)__builtin_amdgcn_ds_bpermute((int)((t & 63u) << 2), (int)(uint32_t)pre);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_ds_bpermute((int)((t & 63u) << 2), (int)(uint32_t)(pre >> 32));
    uint64_t tp = (uint64_t)lo | ((uint64_t)hi << 32);
    me = make_uint2(0u, 0u);
    moff = 0;
    if (live) {
      me = read_row(in, cc);
      if (p.ntiles > 64u) {  // huge streams only: this lane adds the earlier tiles itself
        tp = 0;
        for (uint32_t i = 0; i < t; ++i) tp += tile_sum[i];
      }
      moff = tp + loc[cc];
    }
  };
  for (uint64_t k = 0;; ++k) {  // CPW > 1 only for one-wave teams: no workgroup barrier below
    const uint64_t c = c0 + k * stride;
    if (c >= p.nc) break;
    if ((k & 63u) == 0u) batch(k);
    const int j = (int)(k & 63u);
    const uint2 e = make_uint2((uint32_t)__builtin_amdgcn_readlane((int)me.x, j),
                               (uint32_t)__builtin_amdgcn_readlane((int)me.y, j));
    const uint64_t off = (uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)moff, j) |
                         ((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(moff >> 32), j) << 32);
    const uint64_t start = c * CS;
    const uint32_t bc = (uint32_t)((p.n - start) < CS ? (p.n - start) : CS);
    if (!row_ok(e, bc)) continue;  // reported by the scan kernel
    const uint32_t size = entry_payload(e.x, e.y);
    if (off + size > p.pb) continue;  // sizes inconsistent with the header: reported by wave 0 below
    const uint8_t* pay = in + p.base + off;
    uint8_t* dst = out + start;
    if (e.x == 0u) {
      // zero or raw chunk: each wave of the team fills or copies its share
      // (whole 16-byte blocks but the last), one block per lane per round
      constexpr uint32_t TW = G::TW;
      const uint32_t share = ((bc + 16u * TW - 1u) / (16u * TW)) * 16u;
      const uint32_t w0 = (g >> 6) * share;
      const uint32_t len = w0 < bc ? (bc - w0 < share ? bc - w0 : share) : 0u;
      if (e.y == 0u) zero_bytes16(dst + w0, len, lane);
      else if constexpr (G::OVL) copy_bytes16_r2(dst + w0, pay + w0, len, lane);
      else copy_bytes16_r1(dst + w0, pay + w0, len, lane);
    } else {
      // A whole chunk of one repeated word as the encoder codes it (a
      // literal, then matches (min(255, rest), 1) while the encoder's minimum
      // match remains, the rest as literals) decodes to that word throughout,
      // filled at the rate of a zero chunk.  Only a payload equal to that
      // form byte for byte takes this route; any other is decoded and checked
      // in full.  Every wave of the team tests the same bytes.
      constexpr uint32_t EW = CS / WS, KN = (EW - 1u) / 255u, KR = (EW - 1u) % 255u;
      constexpr uint32_t MMe = WS >= 4 ? 1u : (WS == 2 ? 2u : 3u);
      constexpr uint32_t KM = KN + (KR >= MMe ? 1u : 0u), KK = KM + 1u + (KR >= MMe ? 0u : KR);
      constexpr uint32_t KF = (KK + 7u) / 8u, KD = WS * (KK - KM) + 2u * KM;
      static_assert(KF + KD <= 64u, "the one-word form fits one byte per lane");
      bool one_word = false;
      uint32_t rep = 0;
      // (the one-wave layout of 1024-element chunks only: elsewhere the extra
      // registers cost the coded chunks more than the shortcut saves)
      if (G::OVL && bc == CS && e.x == KF && e.y == KD) {
        const uint32_t j = lane;
        const uint32_t b = j < KF + KD ? (uint32_t)pay[j] : 0u;
        uint32_t w = 0;  // the literal word, payload bytes KF .. KF + WS
#pragma unroll
        for (uint32_t k = 0; k < WS; ++k) w |= (uint32_t)__builtin_amdgcn_readlane((int)b, (int)(KF + k)) << (8u * k);
        rep = WS == 4 ? w : (WS == 2 ? w * 0x10001u : w * 0x01010101u);
        uint32_t want;
        if (j < KF) {
          const uint32_t lo = 8u * j, hi = lo + 8u;
          const uint32_t a0 = lo > 1u ? lo : 1u, a1 = hi < KM + 1u ? hi : KM + 1u;
          want = a0 < a1 ? ((1u << (a1 - lo)) - (1u << (a0 - lo))) & 0xFFu : 0u;
        } else {
          const uint32_t d = j - KF;
          if (d < WS) want = (rep >> (8u * d)) & 0xFFu;
          else if (d < WS + 2u * KM) want = ((d - WS) & 1u) ? 1u : (((d - WS) >> 1) < KN ? 255u : KR);
          else want = (rep >> (8u * ((d - WS - 2u * KM) % WS))) & 0xFFu;
        }
        one_word = __ballot(j < KF + KD && b != want) == 0ull;
      }
      if (one_word) {
        constexpr uint32_t TW = G::TW;
        const uint32_t share = ((bc + 16u * TW - 1u) / (16u * TW)) * 16u;
        const uint32_t w0 = (g >> 6) * share;
        const uint32_t len = w0 < bc ? (bc - w0 < share ? bc - w0 : share) : 0u;
        fill_bytes16(dst + w0, len, lane, rep);
      } else if (!decode_coded<CS, WS, false, TEAMS>(pay, e.x, e.y, bc, dst, arena, sh, SplitSrc{}) && g == 0) {
        raise_status(status, out_bytes, kStatusCorrupt);
      }
    }
    team_sync<G::TW>();
  }
}

template <uint32_t CS, uint32_t WS>
__device__ __forceinline__ void decode_group(const DecP& p, const uint8_t* in, uint8_t* out,
                             const uint32_t* loc, const uint64_t* tile_sum, uint32_t* status, uint64_t* out_bytes,
                             uint8_t* arena_all, uint32_t* sh, uint64_t pre) {
  // Chunks that fit one slot only with the payload over the values go one
  // per wave when there are enough of them to keep every CU busy; a small
  // stream decodes faster with a workgroup per chunk.
  if constexpr (Geo<CS, WS>::OVL) {
    if (p.nc >= kOneWaveMinChunks) {
      decode_group_teams<CS, WS, false>(p, in, out, loc, tile_sum, status, out_bytes, arena_all, sh, pre);
      return;
    }
  }
  decode_group_teams<CS, WS, true>(p, in, out, loc, tile_sum, status, out_bytes, arena_all, sh, pre);
}

template <uint32_t CS>
__device__ __forceinline__ void decode_by_ws(const DecP& p, const uint8_t* in, uint8_t* out,
                             const uint32_t* loc, const uint64_t* tile_sum, uint32_t* status, uint64_t* out_bytes,
                             uint8_t* arena, uint32_t* sh, uint64_t pre) {
  if (p.ws == 4u) decode_group<CS, 4>(p, in, out, loc, tile_sum, status, out_bytes, arena, sh, pre);
  else if (p.ws == 2u) decode_group<CS, 2>(p, in, out, loc, tile_sum, status, out_bytes, arena, sh, pre);
  else decode_group<CS, 1>(p, in, out, loc, tile_sum, status, out_bytes, arena, sh, pre);
}

__global__ __launch_bounds__(kBlock) __attribute__((amdgpu_waves_per_eu(7))) void chunks_kernel(const uint8_t* __restrict__ in, uint64_t in_bytes,
                                                        uint8_t* __restrict__ out, const DecP* __restrict__ P,
                                                        const uint32_t* __restrict__ loc,
                                                        const uint64_t* __restrict__ tile_sum,
                                                        const uint32_t* __restrict__ tile_err,
                                                        uint32_t* __restrict__ status,
                                                        uint64_t* __restrict__ out_bytes) {
  __shared__ __attribute__((aligned(16))) uint8_t arena[kArena];
  __shared__ uint32_t sh[2 * kWaves];
  // the first 64 tile totals (the workspace holds at least that many slots),
  // loaded before the parameters so that the two loads overlap
  const uint64_t ts_lane = tile_sum[lane_id()];
  const DecP p = *P;
  if (p.status != kStatusOk) return;
  // lane t: the payload bytes of the tiles before tile t (streams of up to
  // 64 tiles; larger ones add the totals per chunk)
  uint64_t pre = 0;
  if (p.ntiles <= 64u) {
    const uint64_t v = lane_id() < p.ntiles ? ts_lane : 0ull;
    pre = wave_incl_add64(v) - v;
  }
  if (blockIdx.x == 0 && threadIdx.x < 64u) {
    // stream-wide checks: the tile totals must add up to the header's payload
    // size and no row may be invalid
    uint64_t s = 0;
    uint32_t err = 0;
    for (uint32_t i = lane_id(); i < p.ntiles; i += 64u) {
      s += tile_sum[i];
      err |= tile_err[i];
    }
    s = lane63_64(wave_incl_add64(s));
    err = lane63(wave_incl_add(err));
    if (lane_id() == 0 && (s != p.pb || err)) raise_status(status, out_bytes, kStatusCorrupt);
  }
  // the header kernel accepted cs and ws, so they are among these
  if (p.cs == 1024u) decode_by_ws<1024>(p, in, out, loc, tile_sum, status, out_bytes, arena, sh, pre);
  else if (p.cs == 2048u) decode_by_ws<2048>(p, in, out, loc, tile_sum, status, out_bytes, arena, sh, pre);
  else decode_by_ws<4096>(p, in, out, loc, tile_sum, status, out_bytes, arena, sh, pre);
}

// ---- split mode ------------------------------------------------------------------
// The three per-chunk sizes of a split-mode entry {items K, matches M}: flag
// bytes, literal bytes (a raw chunk's bytes too) and matches.  False if the
// entry breaks a rule (zero: (0,0); raw: (0, bit 31 | real bytes); coded:
// 1 <= K <= E, M <= K, and its one-stream form smaller than the chunk).
__device__ __forceinline__ bool split_sizes(uint2 e, uint32_t bc, uint32_t cs, uint32_t ws, uint32_t* f,
                                            uint32_t* l, uint32_t* m) {
  *f = *l = *m = 0;
  if (e.x == 0u) {
    if (e.y == 0u) return true;
    if ((e.y & kRawBit) && (e.y & ~kRawBit) == bc) {
      *l = bc;
      return true;
    }
    return false;
  }
  const uint32_t K = e.x, M = e.y, E = cs / ws;
  if (K > E || M > K) return false;
  const uint32_t F = (K + 7u) / 8u;
  if ((uint64_t)F + (uint64_t)ws * (K - M) + 2ull * M >= bc) return false;
  *f = F;
  *l = ws * (K - M);
  *m = M;
  return true;
}

// Header and entry checks of a split stream, per tile of T chunks: each
// chunk's three offsets within its tile, the tile's three totals.
__global__ __launch_bounds__(kBlock) void split_scan_kernel(const uint8_t* __restrict__ meta, uint64_t meta_bytes,
                                                            uint64_t out_capacity, uint32_t chunks_cap,
                                                            DecP* __restrict__ P, uint32_t* __restrict__ loc,
                                                            uint64_t* __restrict__ tile_sum,
                                                            uint32_t* __restrict__ tile_err,
                                                            uint32_t* __restrict__ status,
                                                            uint64_t* __restrict__ out_bytes) {
  __shared__ uint64_t sh[kWaves];
  const uint32_t magic = ld_u32_bytes(meta);
  const uint32_t ver = meta[4], ws = meta[5], res = meta[6] | ((uint32_t)meta[7] << 8);
  const uint32_t cs = ld_u32_bytes(meta + 8), nc = ld_u32_bytes(meta + 12);
  const uint64_t n = ld_u64_bytes(meta + 16), nflag = ld_u64_bytes(meta + 24);
  uint32_t st = kStatusOk;
  if (magic != kMagic || ver != kSplitVersion || res != 0 || !word_size_ok(ws) || !chunk_size_ok(cs)) {
    st = kStatusCorrupt;
  } else {
    const uint64_t want = n / cs + ((n % cs) != 0);
    const uint64_t table_end = (uint64_t)kHeaderBytes + (uint64_t)kEntryBytes * nc;
    if (want != nc || table_end > meta_bytes || nflag > meta_bytes - table_end) st = kStatusCorrupt;
    else if (n > out_capacity) st = kStatusCapacity;
    else if (nc > chunks_cap) st = kStatusCorrupt;
  }
  // tiles sized for the stream's own chunk count, as in the one-stream scan
  // (the launch covers them: nc <= chunks_cap)
  const uint32_t T = scan_tile_chunks(nc);
  const uint32_t ntiles = (nc + T - 1u) / T;
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    P->n = n;
    P->pb = nflag;
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
  uint64_t carry[3] = {0, 0, 0};
  bool bad = false;
  for (uint64_t r0 = t0; r0 < t1; r0 += kScanRound) {
    const uint64_t c0 = r0 + (uint64_t)threadIdx.x * kScanPer;
    uint32_t sz[3][kScanPer];
    uint64_t local[3] = {0, 0, 0};
#pragma unroll
    for (uint32_t j = 0; j < kScanPer; ++j) {
      const uint64_t c = c0 + j;
      sz[0][j] = sz[1][j] = sz[2][j] = 0;
      if (c < t1) {
        const uint2 e = read_row(meta, c);
        const uint64_t start = c * cs;
        const uint32_t bc = (uint32_t)((n - start) < cs ? (n - start) : cs);
        if (!split_sizes(e, bc, cs, ws, &sz[0][j], &sz[1][j], &sz[2][j])) bad = true;
      }
#pragma unroll
      for (uint32_t q = 0; q < 3u; ++q) local[q] += sz[q][j];
    }
#pragma unroll
    for (uint32_t q = 0; q < 3u; ++q) {
      uint64_t tot;
      uint64_t off = carry[q] + block_exclusive_scan(local[q], &tot, sh);
#pragma unroll
      for (uint32_t j = 0; j < kScanPer; ++j) {
        const uint64_t c = c0 + j;
        if (c < t1) loc[(uint64_t)q * chunks_cap + c] = (uint32_t)off;  // < 2^32 by the tile sizing
        off += sz[q][j];
      }
      carry[q] += tot;
    }
  }
  const bool anybad = __syncthreads_or(bad);
  if (threadIdx.x == 0) {
#pragma unroll
    for (uint32_t q = 0; q < 3u; ++q) tile_sum[(uint64_t)q * kMaxTilesAlloc + blockIdx.x] = carry[q];
    tile_err[blockIdx.x] = anybad ? 1u : 0u;
  }
}

template <uint32_t CS, uint32_t WS>
__device__ __forceinline__ void decode_group_split(const DecP& p, const SplitDecodeArgs& a, const uint32_t* loc,
                                                   const uint64_t* tile_sum, uint8_t* arena_all, uint32_t* sh) {
  using G = Geo<CS, WS>;
  constexpr uint32_t TL = G::TL;
  constexpr uint32_t CPW = kWaves / G::TW;  // chunks per workgroup
  // a wave uniform, kept in a scalar register (TL is a multiple of 64)
  const uint32_t team = (uint32_t)__builtin_amdgcn_readfirstlane((int)(threadIdx.x / TL)), g = threadIdx.x % TL,
                 lane = lane_id();
  uint8_t* arena = arena_all + team * (G::TW * kSlot);
  const uint8_t* flags = a.meta + p.base;
  const uint64_t stride = (uint64_t)gridDim.x * CPW;
  const uint64_t c0 = (uint64_t)blockIdx.x * CPW + team;
  // The metadata of 64 of the team's chunks (entry and the three port
  // offsets) is loaded at once, one chunk per lane, and handed out by
  // readlane, as in the one-stream decode.  A port offset is the bytes of
  // that port in the earlier tiles plus the offset within the tile.
  uint2 me = make_uint2(0u, 0u);
  uint64_t mo[3] = {0ull, 0ull, 0ull};
  auto batch = [&](uint64_t k0) {
    const uint64_t cc = c0 + (k0 + lane) * stride;
    const bool live = cc < p.nc;
    const uint32_t t = live ? (uint32_t)(cc >> __builtin_ctz(p.T)) : 0u;
    me = live ? read_row(a.meta, cc) : make_uint2(0u, 0u);
#pragma unroll
    for (uint32_t q = 0; q < 3u; ++q) {
      const uint64_t* ts = tile_sum + (uint64_t)q * kMaxTilesAlloc;
      uint64_t tp = 0;
      if (p.ntiles <= 64u) {  // lane i: the tiles before tile i, handed to each chunk's lane
        const uint64_t v = lane < p.ntiles ? ts[lane] : 0ull;
        const uint64_t pr = wave_incl_add64(v) - v;
        const uint32_t lo = (uint32_t)__builtin_amdgcn_ds_bpermute((int)((t & 63u) << 2), (int)(uint32_t)pr);
        const uint32_t hi = (uint32_t)__builtin_amdgcn_ds_bpermute((int)((t & 63u) << 2), (int)(uint32_t)(pr >> 32));
        tp = (uint64_t)lo | ((uint64_t)hi << 32);
      } else if (live) {  // huge streams only: this lane adds the earlier tiles itself
        for (uint32_t i = 0; i < t; ++i) tp += ts[i];
      }
      mo[q] = live ? tp + loc[(uint64_t)q * a.chunks_cap + cc] : 0ull;
    }
  };
  for (uint64_t k = 0;; ++k) {
    const uint64_t c = c0 + k * stride;
    if (c >= p.nc) break;
    if ((k & 63u) == 0u) batch(k);
    const int j = (int)(k & 63u);
    const uint2 e = make_uint2((uint32_t)__builtin_amdgcn_readlane((int)me.x, j),
                               (uint32_t)__builtin_amdgcn_readlane((int)me.y, j));
    uint64_t pre[3];
#pragma unroll
    for (uint32_t q = 0; q < 3u; ++q)
      pre[q] = (uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)mo[q], j) |
               ((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(mo[q] >> 32), j) << 32);
    const uint64_t start = c * CS;
    const uint32_t bc = (uint32_t)((p.n - start) < CS ? (p.n - start) : CS);
    uint32_t fz, lz, mz;
    if (!split_sizes(e, bc, CS, WS, &fz, &lz, &mz)) continue;  // reported by the scan kernel
    // sizes inconsistent with the ports: reported by workgroup 0 below
    if (pre[0] + fz > p.pb || pre[1] + lz > a.lit_bytes || pre[2] + mz > a.tok_bytes) continue;
    uint8_t* dst = a.out + start;
    if (e.x == 0u) {
      // zero or raw chunk: each wave of the team fills or copies its share
      // (whole 16-byte blocks but the last), one block per lane per round
      constexpr uint32_t TW = G::TW;
      const uint32_t share = ((bc + 16u * TW - 1u) / (16u * TW)) * 16u;
      const uint32_t w0 = (g >> 6) * share;
      const uint32_t len = w0 < bc ? (bc - w0 < share ? bc - w0 : share) : 0u;
      if (e.y == 0u) zero_bytes16(dst + w0, len, lane);
      else copy_bytes16_r1(dst + w0, a.lit + pre[1] + w0, len, lane);
    } else {
      const SplitSrc sp{flags + pre[0], a.lit + pre[1], a.lens + pre[2], a.offs + pre[2], e.x, e.y};
      if (!decode_coded<CS, WS, true>(nullptr, 0u, 0u, bc, dst, arena, sh, sp) && g == 0)
        raise_status(a.status, a.out_bytes, kStatusCorrupt);
    }
    team_sync<G::TW>();
  }
}

template <uint32_t CS>
__device__ __forceinline__ void decode_split_by_ws(const DecP& p, const SplitDecodeArgs& a, const uint32_t* loc,
                                                   const uint64_t* tile_sum, uint8_t* arena, uint32_t* sh) {
  if (p.ws == 4u) decode_group_split<CS, 4>(p, a, loc, tile_sum, arena, sh);
  else if (p.ws == 2u) decode_group_split<CS, 2>(p, a, loc, tile_sum, arena, sh);
  else decode_group_split<CS, 1>(p, a, loc, tile_sum, arena, sh);
}

__global__ __launch_bounds__(kBlock) __attribute__((amdgpu_waves_per_eu(7))) void split_chunks_kernel(
    SplitDecodeArgs a, const DecP* __restrict__ P) {
  __shared__ __attribute__((aligned(16))) uint8_t arena[kArena];
  __shared__ uint32_t sh[2 * kWaves];
  const DecP p = *P;
  if (p.status != kStatusOk) return;
  if (blockIdx.x == 0 && threadIdx.x < 64u) {
    // port-wide checks: the flag totals must add up to the header's, the
    // other ports must hold what the entries say, no entry may be invalid
    uint64_t s0 = 0, s1 = 0, s2 = 0;
    uint32_t err = 0;
    for (uint32_t i = lane_id(); i < p.ntiles; i += 64u) {
      s0 += a.tile_sums[i];
      s1 += a.tile_sums[kMaxTilesAlloc + i];
      s2 += a.tile_sums[2u * kMaxTilesAlloc + i];
      err |= a.tile_err[i];
    }
    s0 = lane63_64(wave_incl_add64(s0));
    s1 = lane63_64(wave_incl_add64(s1));
    s2 = lane63_64(wave_incl_add64(s2));
    err = lane63(wave_incl_add(err));
    if (lane_id() == 0 && (s0 != p.pb || s1 > a.lit_bytes || s2 > a.tok_bytes || err))
      raise_status(a.status, a.out_bytes, kStatusCorrupt);
  }
  if (p.cs == 1024u) decode_split_by_ws<1024>(p, a, a.loc, a.tile_sums, arena, sh);
  else if (p.cs == 2048u) decode_split_by_ws<2048>(p, a, a.loc, a.tile_sums, arena, sh);
  else decode_split_by_ws<4096>(p, a, a.loc, a.tile_sums, arena, sh);
}

// ---- one thread per chunk ----------------------------------------------------------
// The decode shape the GPULZStage page attributes to upstream (its
// block-parallel decode paragraph): a whole chunk on one thread, replaying
// its items in order.  Kept as a measured baseline; same stream rules and
// results as chunks_kernel.  Bytes past the chunk's real end are never
// stored: they must decode to zero, so a match source there reads as zero.
__global__ __launch_bounds__(kBlock) void serial_chunks_kernel(const uint8_t* __restrict__ in, uint64_t in_bytes,
                                                               uint8_t* __restrict__ out, const DecP* __restrict__ P,
                                                               const uint32_t* __restrict__ loc,
                                                               const uint64_t* __restrict__ tile_sum,
                                                               const uint32_t* __restrict__ tile_err,
                                                               uint32_t* __restrict__ status,
                                                               uint64_t* __restrict__ out_bytes) {
  const DecP p = *P;
  if (p.status != kStatusOk) return;
  if (blockIdx.x == 0 && threadIdx.x < 64u) {
    uint64_t s = 0;
    uint32_t err = 0;
    for (uint32_t i = lane_id(); i < p.ntiles; i += 64u) {
      s += tile_sum[i];
      err |= tile_err[i];
    }
    s = lane63_64(wave_incl_add64(s));
    err = lane63(wave_incl_add(err));
    if (lane_id() == 0 && (s != p.pb || err)) raise_status(status, out_bytes, kStatusCorrupt);
  }
  const uint32_t cs = p.cs, ws = p.ws, E = cs / ws;
  const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
  for (uint64_t c = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; c < p.nc; c += stride) {
    const uint2 e = read_row(in, c);
    const uint64_t start = c * cs;
    const uint32_t bc = (uint32_t)((p.n - start) < cs ? (p.n - start) : cs);
    if (!row_ok(e, bc)) continue;  // reported by the scan kernel
    const uint32_t size = entry_payload(e.x, e.y);
    const uint32_t t = (uint32_t)(c >> __builtin_ctz(p.T));
    uint64_t off = loc[c];
    for (uint32_t i = 0; i < t; ++i) off += tile_sum[i];
    if (off + size > p.pb) continue;  // reported by the tile-total check
    const uint8_t* pay = in + p.base + off;
    uint8_t* dst = out + start;
    if (e.x == 0u) {
      const bool zero = e.y == 0u;
      for (uint32_t y = 0; y < bc; ++y) dst[y] = zero ? 0u : pay[y];
      continue;
    }
    const uint32_t F = e.x, D = e.y;
    const uint8_t* fl = pay;
    const uint8_t* dt = pay + F;
    uint32_t q = 0, d = 0, k = 0;
    bool ok = true;
    // whole-element loads and stores when the element is real and aligned
    const bool wal = (((uintptr_t)dst) & (ws - 1u)) == 0;
    auto get_el = [&](uint32_t i) -> uint32_t {  // element i of the output (0 past the real bytes)
      if (wal && (i + 1u) * ws <= bc) {
        if (ws == 4u) return *(const uint32_t*)(dst + 4u * i);
        if (ws == 2u) return *(const uint16_t*)(dst + 2u * i);
        return dst[i];
      }
      uint32_t v = 0;
      for (uint32_t b = 0; b < ws; ++b)
        if (i * ws + b < bc) v |= (uint32_t)dst[i * ws + b] << (8u * b);
      return v;
    };
    auto put_el = [&](uint32_t i, uint32_t v) {  // padding elements must decode to zero
      if (wal && (i + 1u) * ws <= bc) {
        if (ws == 4u) *(uint32_t*)(dst + 4u * i) = v;
        else if (ws == 2u) *(uint16_t*)(dst + 2u * i) = (uint16_t)v;
        else dst[i] = (uint8_t)v;
        return;
      }
      for (uint32_t b = 0; b < ws; ++b) {
        const uint8_t x = (uint8_t)(v >> (8u * b));
        if (i * ws + b < bc) dst[i * ws + b] = x;
        else if (x != 0u) ok = false;
      }
    };
    while (ok && q < E) {
      if (k >= 8u * F) {
        ok = false;
        break;
      }
      if ((fl[k >> 3] >> (k & 7u)) & 1u) {
        if (d + 2u > D) {
          ok = false;
          break;
        }
        const uint32_t L = dt[d], O = dt[d + 1u];
        d += 2u;
        if (L == 0u || O == 0u || O > q || q + L > E) {
          ok = false;
          break;
        }
        for (uint32_t j = 0; j < L; ++j) put_el(q + j, get_el(q + j - O));  // overlapping copies run forward
        q += L;
      } else {
        if (d + ws > D) {
          ok = false;
          break;
        }
        uint32_t v = 0;
        for (uint32_t b = 0; b < ws; ++b) v |= (uint32_t)dt[d + b] << (8u * b);
        put_el(q, v);
        d += ws;
        ++q;
      }
      ++k;
    }
    if (ok) {
      if (d != D || (k + 7u) / 8u != F) ok = false;
      for (uint32_t b = k; ok && b < 8u * F; ++b)
        if ((fl[b >> 3] >> (b & 7u)) & 1u) ok = false;
    }
    if (!ok) raise_status(status, out_bytes, kStatusCorrupt);
  }
}

}  // namespace

uint64_t decode_params_bytes() { return sizeof(DecP); }

hipError_t launch_decode_split(const SplitDecodeArgs& a, hipStream_t stream) {
  const uint32_t tiles = scan_groups(a.chunks_cap);
  if (tiles > kMaxTilesAlloc) return hipErrorInvalidValue;
  hipLaunchKernelGGL(split_scan_kernel, dim3(tiles), dim3(kBlock), 0, stream, a.meta, a.meta_bytes, a.out_capacity,
                     a.chunks_cap, (DecP*)a.params, a.loc, a.tile_sums, a.tile_err, a.status, a.out_bytes);
  if (a.chunks_cap > 0) {
    uint32_t grid = (a.chunks_cap + kWaves - 1u) / kWaves;
    if (grid > kDecodeGrid) grid = kDecodeGrid;
    hipLaunchKernelGGL(split_chunks_kernel, dim3(grid), dim3(kBlock), 0, stream, a, (const DecP*)a.params);
  }
  return hipGetLastError();
}

hipError_t launch_decode_serial(const DecodeArgs& a, hipStream_t stream) {
  const uint32_t tiles = scan_groups(a.chunks_cap);
  hipLaunchKernelGGL(scan_kernel, dim3(tiles), dim3(kBlock), 0, stream, a.in, a.in_bytes, a.out_capacity,
                     a.chunks_cap, (DecP*)a.params, a.loc, a.tile_sums, a.tile_err, a.status, a.out_bytes);
  if (a.ev_start && hipEventRecord(a.ev_start, stream) != hipSuccess) return hipErrorUnknown;
  if (a.chunks_cap > 0) {
    uint32_t grid = (a.chunks_cap + kBlock - 1u) / kBlock;
    if (grid > kDecodeGrid) grid = kDecodeGrid;
    hipLaunchKernelGGL(serial_chunks_kernel, dim3(grid), dim3(kBlock), 0, stream, a.in, a.in_bytes, a.out,
                       (const DecP*)a.params, (const uint32_t*)a.loc, (const uint64_t*)a.tile_sums,
                       (const uint32_t*)a.tile_err, a.status, a.out_bytes);
  }
  if (a.ev_stop && hipEventRecord(a.ev_stop, stream) != hipSuccess) return hipErrorUnknown;
  return hipGetLastError();
}

hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream) {
  const uint32_t tiles = scan_groups(a.chunks_cap);
  hipLaunchKernelGGL(scan_kernel, dim3(tiles), dim3(kBlock), 0, stream, a.in, a.in_bytes, a.out_capacity,
                     a.chunks_cap, (DecP*)a.params, a.loc, a.tile_sums, a.tile_err, a.status, a.out_bytes);
  if (a.ev_start && hipEventRecord(a.ev_start, stream) != hipSuccess) return hipErrorUnknown;
  if (a.chunks_cap > 0) {
    // workgroups loop over chunk groups: enough of them to fill every CU a few
    // times over, not one per group (their launch would cost more than the
    // work for zero and raw chunks)
    uint32_t grid = (a.chunks_cap + kWaves - 1u) / kWaves;
    if (grid > kDecodeGridTeams) grid = kDecodeGridTeams;
    hipLaunchKernelGGL(chunks_kernel, dim3(grid), dim3(kBlock), 0, stream, a.in, a.in_bytes, a.out,
                       (const DecP*)a.params, (const uint32_t*)a.loc, (const uint64_t*)a.tile_sums,
                       (const uint32_t*)a.tile_err, a.status, a.out_bytes);
  }
  if (a.ev_stop && hipEventRecord(a.ev_stop, stream) != hipSuccess) return hipErrorUnknown;
  return hipGetLastError();
}

}  // namespace gpulz
