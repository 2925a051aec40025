// encode.hip -- chunked LZSS encode for gfx950: a chunk kernel and an
// assembly kernel.
//
// encode_kernel: a "team" of WPC wave64s owns one chunk (WPC = 1 for chunks
// of up to 512 elements, so most of the work needs no workgroup barrier; a
// workgroup holds CPW teams).  Per chunk (GPULZStage page paragraphs in
// brackets):
//   1. load the chunk (zero padded past its real bytes) into LDS as E words;
//      all zero -> entry (0,0), no payload [zero-chunk paragraph];
//   2. omask[p], bit o-1 = (x[p] == x[p-o]), o = 1..32 [exact-search
//      paragraph]: each lane holds 8 consecutive positions and the 32 words
//      before them in registers, so the 256 comparisons per lane read LDS once;
//      no bit set anywhere -> at level 0 the chunk is raw, steps 3-6 skipped
//      (word size 4: a chunk whose sampled positions have no match is first
//      tested by compares alone, and skips the masks if that finds none);
//   3. level 0, window 32, up to 1024 elements: S_4 and a short descent give
//      the exact (L, O) below 16 and mark longer matches, whose exact length
//      is found only where the parse starts an item (step 5).  Otherwise a
//      base-4 doubling table S_k[p] = AND of omask over [p, p+k) for
//      k = 1, 4, 16 (S_64 read as the AND of four S_16 entries, not stored),
//      and a 4-round descent per position (up to three steps of k per round,
//      so L <= 255).  Either way: the exact longest run of any offset, capped
//      at 255, and the smallest offset reaching it [exact-search and
//      long-match paragraphs];
//   4. level 1: 2048-bucket table of position+1 per sub-block, lookups and
//      max inserts separated by barriers [hashed-table paragraphs];
//   5. greedy parse [provenance paragraph], in parallel: every 8-position
//      segment computes, for each entry position, where the parse leaves the
//      segment and which positions start items; a short chain of hops over
//      segments then fixes the real entry of each segment;
//   6. counts: lane g takes segment g; one packed scan of its items and
//      matches (two item sizes only) -> flag bytes F and data bytes D; raw
//      when F + D >= real bytes [raw-fallback paragraph];
//   7. the size-table row goes straight into the stream; a coded payload
//      (flag bitmap, then data bytes; each lane writes its segment's items)
//      is built in LDS and written to the chunk's fixed-stride staging slot.
//      A raw chunk's payload is its input bytes: it is never staged, the
//      assembly copies it from the input.
// compact_kernel: one workgroup per tile of 64 chunks scans the tile's sizes,
//   finds the tile's offset by decoupled look-back over the tiles before it
//   and moves every payload to its place in the stream with 16-byte stores;
//   the last tile writes the header.
// split_compact_kernel: the same assembly into the four split-mode ports.
// advancing_encode_kernel: the upstream-style advancing-window search, a
//   measured baseline with the same stream rules (its own comment says how).
#include "common.h"

namespace gpulz {
namespace {

constexpr uint64_t kFlagAgg = 1ull << 62;
constexpr uint64_t kFlagIncl = 2ull << 62;
constexpr uint64_t kFlagVal = (1ull << 62) - 1ull;
constexpr uint32_t kSpinLimit = 1u << 20;

template <int WS>
constexpr uint32_t min_match() {
  // a match is taken only when its 2-byte token is shorter than the literals
  return WS >= 4 ? 1u : (WS == 2 ? 2u : 3u);
}

constexpr uint32_t cmax(uint32_t a, uint32_t b) { return a > b ? a : b; }

__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

template <int WPC>
__device__ __forceinline__ void team_sync() {
  if (WPC == 1) wave_sync();
  else __syncthreads();
}

__device__ __forceinline__ uint32_t lane_id() { return threadIdx.x & 63u; }

__device__ __forceinline__ uint32_t mbcnt64(uint64_t m) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

__device__ __forceinline__ uint64_t wave_sum_u64(uint64_t v) {
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) v += __shfl_xor(v, d, 64);
  return v;
}

// The short descent's mark for a position whose longest match is 16 or
// longer (its exact length is found only if the parse starts an item there),
// and the segment-exit flag that sends the parse to such a position.
constexpr uint32_t kLongMark = 0xFFu;
constexpr uint32_t kLongExit = 0x8000u;

// DPP lane move whose out-of-row or masked-off lanes read all ones (the
// identity of AND).
template <int CTRL, int ROWS = 0xF>
__device__ __forceinline__ uint32_t dpp_ones(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp((int)0xFFFFFFFF, (int)v, CTRL, ROWS, 0xF, false);
}

// Inclusive AND scan over the 64 lanes (lane i: AND of lanes 0..i).
__device__ __forceinline__ uint32_t wave_incl_and(uint32_t v) {
  v &= dpp_ones<kRowShr1>(v);
  v &= dpp_ones<kRowShr2>(v);
  v &= dpp_ones<kRowShr4>(v);
  v &= dpp_ones<kRowShr8>(v);
  v &= dpp_ones<kRowBcast15, 0xA>(v);
  v &= dpp_ones<kRowBcast31, 0xC>(v);
  return v;
}

// Exact capped longest match at position r (uniform; every lane of the wave
// takes part), GPULZStage page, exact longest-match search and long-match
// paragraphs: L = the largest k <= min(255, E - r) such that some offset
// matches at all of r .. r + k - 1, i.e. the AND of omask over [r, r + k) is
// not empty; O = the smallest offset left in that AND.  One round: lane j
// takes positions r + 4j .. r + 4j + 3 (256 >= 255), ANDs them in order,
// and an exclusive AND scan over the lanes supplies what comes before; the
// running ANDs only shrink, so the non-empty ones are a prefix and L is
// their count.  Returns L | O << 8.
__device__ __forceinline__ uint32_t long_match(const uint32_t* S1, uint32_t r, uint32_t E) {
  const uint32_t lane = lane_id();
  const uint32_t lim = (E - r) < kMaxLen ? (E - r) : kMaxLen;
  const uint32_t i0 = 4u * lane;
  const uint32_t m0 = i0 < lim ? S1[r + i0] : 0u;
  const uint32_t m1 = i0 + 1u < lim ? S1[r + i0 + 1u] : 0u;
  const uint32_t m2 = i0 + 2u < lim ? S1[r + i0 + 2u] : 0u;
  const uint32_t m3 = i0 + 3u < lim ? S1[r + i0 + 3u] : 0u;
  const uint32_t a1 = m0 & m1, a2 = a1 & m2, a3 = a2 & m3;
  // AND of every earlier lane's four (all ones for lane 0)
  const uint32_t incl = wave_incl_and(a3);
  const uint32_t ex = lane ? dpp_ones<kWaveShr1>(incl) : ~0u;
  const uint32_t p0 = ex & m0, p1 = ex & a1, p2 = ex & a2, p3 = ex & a3;
  const uint32_t cnt = (uint32_t)(p0 != 0u) + (uint32_t)(p1 != 0u) + (uint32_t)(p2 != 0u) + (uint32_t)(p3 != 0u);
  // the first lane whose four are not all non-empty ends the run
  const uint64_t part = __ballot(cnt < 4u);
  const uint32_t jl = part ? (uint32_t)__builtin_ctzll(part) : 63u;
  const uint32_t L = 4u * jl + (uint32_t)__builtin_amdgcn_readlane((int)cnt, (int)jl);
  // survivors at position L - 1: lane (L - 1) / 4, running AND (L - 1) % 4
  const uint32_t k = (L - 1u) & 3u;
  const uint32_t pk = k == 0u ? p0 : (k == 1u ? p1 : (k == 2u ? p2 : p3));
  const uint32_t fin = (uint32_t)__builtin_amdgcn_readlane((int)pk, (int)((L - 1u) >> 2));
  return L | (((uint32_t)__builtin_ctz(fin) + 1u) << 8);
}

// Decoupled look-back over the chunks' published payload sizes (one wave).
// Each flag is one 64-bit word {state:2, value:62}, written with one atomic
// store, so a reader never sees a state without its value.  Nothing else is
// published through a flag, so relaxed device-scope atomics suffice: they go
// to the device coherence point without the L2 writeback / invalidate that
// release / acquire ordering costs on a part with one L2 per XCD.
// Returns the exclusive prefix (output offset of chunk c's payload).
__device__ uint64_t look_back(uint64_t* flags, uint32_t c, uint64_t agg, uint32_t* err) {
  const uint32_t lane = lane_id();
  if (c == 0) {
    if (lane == 0) __hip_atomic_store(&flags[0], kFlagIncl | agg, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return 0;
  }
  if (lane == 0) __hip_atomic_store(&flags[c], kFlagAgg | agg, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  uint64_t prefix = 0;
  int64_t j = (int64_t)c - 1;
  uint32_t spins = 0;
  while (true) {
    const int64_t idx = j - (int64_t)lane;
    uint64_t f = kFlagIncl;  // before chunk 0: an inclusive prefix of 0
    if (idx >= 0) f = __hip_atomic_load(&flags[idx], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const uint64_t incl = __ballot((f >> 62) == 2u);
    const uint64_t inval = __ballot((f >> 62) == 0u);
    const uint32_t first = incl ? (uint32_t)__builtin_ctzll(incl) : 64u;
    const uint64_t need = first >= 63u ? ~0ull : ((2ull << first) - 1ull);
    if (inval & need) {
      if (++spins > kSpinLimit) {  // never expected; turns a stall into an error
        if (lane == 0) atomicOr(err, 1u);
        break;
      }
      __builtin_amdgcn_s_sleep(1);
      continue;
    }
    prefix += wave_sum_u64(lane <= first ? (f & kFlagVal) : 0ull);
    if (first < 64u) break;
    j -= 64;
  }
  if (lane == 0)
    __hip_atomic_store(&flags[c], kFlagIncl | (prefix + agg), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return prefix;
}

__device__ __forceinline__ void put_le(uint8_t* p, uint64_t v, int nb) {
  for (int i = 0; i < nb; ++i) p[i] = (uint8_t)(v >> (8 * i));
}

// acc = acc * 2^16 + (16 match bits, a[0] first): bit = (a[i] == v).  Each
// compare writes a lane mask to an SGPR pair and an add-with-carry shifts it
// into acc, two instructions per compare.  A VALU write of an SGPR must be at
// least two instructions ahead of a VALU read of it as carry, so three pairs
// rotate: every add reads the pair written three compares earlier.
__device__ __forceinline__ void match_bits16(uint32_t& acc, const uint32_t* a, uint32_t v) {
  uint64_t m0, m1, m2;
#define GLZ_C(k, m) "v_cmp_eq_u32_e64 %[" #m "], %[a" #k "], %[v]\n"
#define GLZ_A(m) "v_addc_co_u32_e64 %[acc], %[" #m "], %[acc], %[acc], %[" #m "]\n"
  asm volatile(GLZ_C(0, m0) GLZ_C(1, m1) GLZ_C(2, m2)
               GLZ_A(m0) GLZ_C(3, m0) GLZ_A(m1) GLZ_C(4, m1) GLZ_A(m2) GLZ_C(5, m2)
               GLZ_A(m0) GLZ_C(6, m0) GLZ_A(m1) GLZ_C(7, m1) GLZ_A(m2) GLZ_C(8, m2)
               GLZ_A(m0) GLZ_C(9, m0) GLZ_A(m1) GLZ_C(10, m1) GLZ_A(m2) GLZ_C(11, m2)
               GLZ_A(m0) GLZ_C(12, m0) GLZ_A(m1) GLZ_C(13, m1) GLZ_A(m2) GLZ_C(14, m2)
               GLZ_A(m0) GLZ_C(15, m0) GLZ_A(m1) GLZ_A(m2) GLZ_A(m0)
               : [acc] "+v"(acc), [m0] "=&s"(m0), [m1] "=&s"(m1), [m2] "=&s"(m2)
               : [v] "v"(v), [a0] "v"(a[0]), [a1] "v"(a[1]), [a2] "v"(a[2]), [a3] "v"(a[3]), [a4] "v"(a[4]),
                 [a5] "v"(a[5]), [a6] "v"(a[6]), [a7] "v"(a[7]), [a8] "v"(a[8]), [a9] "v"(a[9]),
                 [a10] "v"(a[10]), [a11] "v"(a[11]), [a12] "v"(a[12]), [a13] "v"(a[13]), [a14] "v"(a[14]),
                 [a15] "v"(a[15]));
#undef GLZ_C
#undef GLZ_A
}

struct EncCtl {
  uint32_t error;  // set if a look-back ever gave up waiting
  uint32_t pad[63];
};

constexpr uint32_t kCTile = 64;  // chunks per compaction tile
__host__ __device__ inline uint32_t num_tiles_of(uint32_t chunks) { return (chunks + kCTile - 1u) / kCTile; }

// Offset masks: one bit per near-window offset, 32 or 64 bits.
template <int W>
struct MaskOf {
  using T = uint32_t;
};
template <>
struct MaskOf<48> {
  using T = uint64_t;
};
template <>
struct MaskOf<64> {
  using T = uint64_t;
};

template <int WS, int E, int LEVEL, int W>
struct Lay {
  static constexpr uint32_t CS = (uint32_t)E * WS;
  static constexpr uint32_t MW = W > 32 ? 2u : 1u;  // words per offset mask
  static constexpr uint32_t NW64 = E / 64;  // 64-position words
  static constexpr uint32_t NSEG = E / 8;   // 8-position parse segments
  // Word offsets inside the per-chunk region.  The chunk's words X are
  // loaded at its start.  At level 0 only the offset masks read them, so S_1
  // overwrites them and the payload's literal words are read again from the
  // input.  Level 1 needs the words again for the candidate checks: chunks
  // of up to 1024 elements keep X in a region of its own ahead of the rest
  // (XW = E); larger ones (XL) overlay X as level 0 does and load the words
  // again from the input behind the hash table after the descent, which
  // saves 8-16 KB per chunk, a third more chunks per CU.
  //   search: S_1 | S_4 | S_16, each E masks followed by zero padding that
  //           the descent may read (3, 9 and 177 or 33 masks, rounded); S_64 is
  //           not stored: its values are ANDs of four S_16 entries
  //   level 1: LO (E) | hash table (2048) [| X again (E), XL]
  //   parse:   LO (E) | XQ (E) | ISB (E/32) | LMB (E/32) | FLG (E/32) | STG (CS/4 + 8)
  static constexpr uint32_t RP = 2u * E + 3u * (E / 32u) + CS / 4u + 8u;
  static constexpr uint32_t TOFF[3] = {0u, E + 4u, 2u * E + 16u};  // table offsets, in masks
  // Chunks of up to 512 elements guard the descent's first-round reads with
  // the chunk's end, so S_16 needs 33 padding masks instead of 177 (a 7 %
  // smaller chunk, one more workgroup per CU); larger chunks are bound by the
  // parse region and skip the guards.
  static constexpr bool GUARD64 = E <= 512;
  static constexpr uint32_t PAD = GUARD64 ? 52u : 196u;  // padding words of S_1, S_4, S_16 (4, 12, rest)
  static constexpr uint32_t SEARCH = MW * (3u * E + PAD);
  static constexpr bool XL = LEVEL == 1 && E >= 2048;                // level 1, X reloaded
  static constexpr uint32_t XW = LEVEL == 1 && !XL ? (uint32_t)E : 0u;  // words of a separate X
  // Level 0 with the 32-offset window and chunks of up to 1024 elements
  // (LAZY): the descent finds lengths below 16 at every position and marks
  // longer ones; the exact length of a long match is found only where the
  // parse starts an item (most positions inside long matches are never item
  // starts).  Regions, in words:
  //   S_1 [0, E) + 16 zero words (the long-match scan and the short descent
  //       read S_1; the payload staging overlays it once the parse is done)
  //   S_4 [E + 16, 2E + 16) + 12 zero words; after the descent the same words
  //       hold LOX: (L | O << 8) in the low half, and from the segment pass
  //       on, the position's segment exit in the high half
  //   IM  [2E + 28, 2E + 28 + E/4) the item-start bits of the segment walk
  //       from each position, a byte each
  //   ISB | LMB (E/32 each) the item-start and match bits of each segment,
  //       a byte each
  // so a 512-element chunk takes under 5 KB of LDS.
  static constexpr bool LAZY = LEVEL == 0 && W == 32 && E <= 1024;
  static constexpr uint32_t WPC_ = E <= 512 ? 1u : (uint32_t)E / 512u;  // waves per chunk (launch_one)
  static constexpr uint32_t LZ_T4 = E + 16u;
  static constexpr uint32_t LZ_IM = 2u * E + 28u;
  static constexpr uint32_t LZ_ISB = LZ_IM + E / 4u;
  static constexpr uint32_t LZ_R = LZ_ISB + 2u * (E / 32u);
  static_assert(!LAZY || CS / 4u + 4u <= E + 16u, "payload staging fits over S_1");
  // level 1 with chunks of up to 512 elements: 16-bit buckets (positions + 1
  // fit), half the table's LDS, so half again as many chunks per CU
  static constexpr bool HT16 = LEVEL == 1 && E <= 512;
  static constexpr uint32_t TW_ = HT16 ? kHashSize / 2u : kHashSize;  // table words
  static constexpr uint32_t R =
      LAZY ? ((LZ_R + 3u) & ~3u)
           : (cmax(cmax(SEARCH, LEVEL ? (XL ? 2u : 1u) * E + TW_ : 0u), RP) + 3u) & ~3u;
  static constexpr uint32_t MISC = WPC_ > 1u ? 8u : 0u;  // a team's per-wave counts (multi-wave chunks)
  // 32 zero words ahead of X (32-offset window): every lane of the offset-mask
  // pass loads its 32 + 8 words with the same 16-byte loads, the first lanes'
  // window running into the zeros (the bits they give are masked off)
  static constexpr uint32_t XPAD = W == 32 ? 32u : 0u;
  static constexpr uint32_t TOTAL = (XPAD + XW + R + MISC + 3u) & ~3u;  // words per chunk, 16-byte multiple
};

template <int WS, int E, int LEVEL, int W, int WPC, int CPW>
__global__ __launch_bounds__(64 * WPC * CPW) void encode_kernel(const uint8_t* __restrict__ in, uint64_t n,
                                                                 uint32_t num_chunks, uint8_t* __restrict__ out,
                                                                 uint8_t* __restrict__ staging,
                                                                 uint64_t* __restrict__ tile_flags,
                                                                 uint32_t num_tiles, uint32_t flag_sets,
                                                                 uint2* __restrict__ km, EncCtl* __restrict__ ctl) {
  using L = Lay<WS, E, LEVEL, W>;
  using Mask = typename MaskOf<W>::T;
  static_assert(W == 32 || W == 48 || W == 64, "near window");
  constexpr uint32_t CS = L::CS;
  constexpr uint32_t TL = 64u * WPC;  // lanes per team
  constexpr uint32_t PPL = E / TL;    // positions per lane (strided p = g + i*TL)
  constexpr uint32_t NR = E / 64u;    // 64-position words
  constexpr uint32_t MM = min_match<WS>();
  static_assert(WPC == 1 || CPW == 1, "a team is one wave or the whole workgroup");
  static_assert(E % (8 * TL) == 0 || E == 256, "omask passes");
  __shared__ __attribute__((aligned(16))) uint32_t lds_all[CPW * L::TOTAL];
  const uint32_t team = threadIdx.x / TL;
  const uint32_t g = threadIdx.x % TL;  // lane within the team
  const uint32_t lane = lane_id();
  uint32_t* X = lds_all + team * L::TOTAL + L::XPAD;
  uint32_t* LV = X + L::XW;  // X and S_1 share their words unless X has its own region
  // level 1: the words for the candidate checks (its own region, or loaded
  // again behind the hash table)
  uint32_t* XL = L::XL ? LV + E + L::TW_ : X;
  Mask* LVm = (Mask*)LV;  // the search tables
  uint32_t* LO = L::LAZY ? LV + L::LZ_T4 : LV;  // LAZY: LOX
  uint32_t* XQ = LV + E;                         // not LAZY: exit | item-start bits << 16
  uint8_t* IM = (uint8_t*)(LV + L::LZ_IM);       // LAZY: item-start bits
  uint32_t* T = LV + E;
  uint32_t* ISB = L::LAZY ? LV + L::LZ_ISB : LV + 2u * E;
  uint32_t* LMB = ISB + E / 32u;
  uint32_t* FLG = LMB + E / 32u;
  uint8_t* STG = L::LAZY ? (uint8_t*)LV : (uint8_t*)(FLG + E / 32u);
  // segment exit of position p and the item-start bits of the walk from it
  // (exit | bits << 16)
  auto xq_at = [&](uint32_t p) -> uint32_t {
    if constexpr (L::LAZY) return (LO[p] >> 16) | ((uint32_t)IM[p] << 16);
    else return XQ[p];
  };
  uint32_t* KB = LV + L::R;  // per wave of a multi-wave team: its item and match counts
  uint8_t* table = out + kHeaderBytes;

  // ---- chunk of this team -----------------------------------------------------------
  const uint32_t c = blockIdx.x * (uint32_t)CPW + team;
  if (c >= num_chunks) return;
  const uint64_t base = (uint64_t)c * CS;
  const uint32_t bc = (uint32_t)((n - base) < CS ? (n - base) : CS);
  const uint8_t* src = in + base;
  // element p of the chunk (0 past its real bytes), from the input
  const bool fast = bc == CS && (((uintptr_t)src) & 3u) == 0;
  auto word_at = [&](uint32_t p) -> uint32_t {
    const uint32_t b = p * (uint32_t)WS;
    uint32_t v = fast ? (((const uint32_t*)src)[b >> 2] >> (8u * (b & 3u))) : load4_unaligned(src + b, src + bc);
    return WS == 4 ? v : (WS == 2 ? (v & 0xFFFFu) : (v & 0xFFu));
  };

  // ---- 1. load + zero vote ---------------------------------------------------------
  // PRE: level 0, 32-offset window, word size 4, one mask pass per chunk (the
  // offset-mask pass below tries a cheaper test first)
  constexpr bool PRE = L::LAZY && WS == 4 && E / ((E == 256 ? 4u : 8u) * TL) == 1u;
  for (uint32_t i = g; i < L::XPAD; i += TL) X[(int)i - (int)L::XPAD] = 0u;
  uint32_t any = 0;
  // diff: nonzero unless every word equals the chunk's first (rep: that word
  // repeated over 32 bits); only the aligned whole-chunk load tests it
  uint32_t diff = 1u, rep = 0u;
  if (bc == CS && (((uintptr_t)src) & 15u) == 0) {
    const uint4* s4 = (const uint4*)src;
    const uint32_t w0 = *(const uint32_t*)src;
    rep = WS == 4 ? w0 : (WS == 2 ? (w0 & 0xFFFFu) * 0x10001u : (w0 & 0xFFu) * 0x01010101u);
    diff = 0u;
    for (uint32_t i = g; i < CS / 16u; i += TL) {
      const uint4 v = s4[i];
      any |= v.x | v.y | v.z | v.w;
      diff |= (v.x ^ rep) | (v.y ^ rep) | (v.z ^ rep) | (v.w ^ rep);
      const uint32_t w[4] = {v.x, v.y, v.z, v.w};
      if (WS == 4) {
        *(uint4*)(X + 4 * i) = v;
      } else if (WS == 2) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          X[8 * i + 2 * j] = w[j] & 0xFFFFu;
          X[8 * i + 2 * j + 1] = w[j] >> 16;
        }
      } else {
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int b = 0; b < 4; ++b) X[16 * i + 4 * j + b] = (w[j] >> (8 * b)) & 0xFFu;
      }
    }
  } else {
    for (uint32_t i = g; i < (uint32_t)E; i += TL) {
      uint32_t w = 0;
#pragma unroll
      for (int b = 0; b < WS; ++b) {
        const uint32_t j = i * WS + b;
        if (j < bc) w |= (uint32_t)src[j] << (8 * b);
      }
      X[i] = w;
      any |= w;
    }
  }
  bool nonzero, konst;
  if (WPC == 1) {
    nonzero = __ballot(any != 0u) != 0ull;
    konst = __ballot(diff != 0u) == 0ull;
    wave_sync();
  } else {
    nonzero = __syncthreads_or(any != 0u);
    konst = !__syncthreads_or(diff != 0u);
  }
  // A chunk of one repeated nonzero word (konst): the near search at every
  // position p >= 1 finds offset 1 (the smallest) running to the cap or the
  // chunk's end, and no farther candidate can be strictly longer, at either
  // level and for any window.  So the greedy parse is fixed: a literal, then
  // matches (min(255, E - p), 1) while at least MM words remain, then the
  // remaining words as literals; its payload is written directly below.
  konst = konst && nonzero;

  uint32_t K = 0, M = 0;
  // segment g's item-start and match bits, and the items (low half) and
  // matches (high half) of the segments before it
  uint32_t it8 = 0, mt8 = 0, kex = 0;
  constexpr uint32_t KN = ((uint32_t)E - 1u) / kMaxLen, KR = ((uint32_t)E - 1u) % kMaxLen;  // konst: full matches, rest
  if (konst) {
    M = KN + (KR >= MM ? 1u : 0u);
    K = M + 1u + (KR >= MM ? 0u : KR);
  } else if (nonzero) {
    // ---- 2. omask: 8 consecutive positions per lane, window in registers -------------
    Mask any_om = 0;  // OR of this lane's masks
    {
      constexpr uint32_t PPASS = (E == 256 ? 4u : 8u);  // positions per lane per pass
      constexpr uint32_t NPASS = E / (PPASS * TL);
#pragma unroll 1
      for (uint32_t ps = 0; ps < NPASS; ++ps) {
        const uint32_t p0 = (ps * TL + g) * PPASS;
        uint32_t w[32 + PPASS];
        if (L::XPAD != 0u || p0 >= 32u) {
#pragma unroll
          for (uint32_t i = 0; i < (32 + PPASS) / 4; ++i) {
            const uint4 v = *(const uint4*)(X + p0 - 32u + 4u * i);
            w[4 * i] = v.x;
            w[4 * i + 1] = v.y;
            w[4 * i + 2] = v.z;
            w[4 * i + 3] = v.w;
          }
        } else {
#pragma unroll
          for (uint32_t i = 0; i < 32 + PPASS; ++i) {
            const int32_t idx = (int32_t)p0 - 32 + (int32_t)i;
            w[i] = idx >= 0 ? X[idx] : 0u;
          }
        }
        Mask om[PPASS];
        // offsets 32..17, then 16..1: bit o-1 compares w[32+q] with w[32+q-o]
        auto mask_of = [&](uint32_t q) -> uint32_t {
          uint32_t m = 0;
          match_bits16(m, &w[q], w[32 + q]);
          match_bits16(m, &w[q + 16], w[32 + q]);
          return m;
        };
        if constexpr (PRE) {
          // Each lane's last position first.  If none of them has a near
          // match, the other positions are first tested by compares alone
          // (one instruction each, their lane masks OR-ed in scalar registers,
          // eight accumulators so the ORs form no chain); a chunk where that
          // finds nothing either is raw, and its masks are all zero.  Words
          // ahead of the chunk read as zeros there, which can only report a
          // match that is not there (then the masks are computed).
          constexpr uint32_t QS = PPASS - 1u;
          om[QS] = mask_of(QS);
          if (p0 + QS < 32u) om[QS] &= (1u << (p0 + QS)) - 1u;
          bool full = WPC == 1 ? __ballot(om[QS] != 0u) != 0ull : __syncthreads_or(om[QS] != 0u);
          if (!full) {
            uint64_t ha[8] = {0ull, 0ull, 0ull, 0ull, 0ull, 0ull, 0ull, 0ull};
#pragma unroll
            for (uint32_t q = 0; q < QS; ++q)
#pragma unroll
              for (uint32_t o = 1; o <= 32u; ++o) ha[o & 7u] |= __ballot(w[32 + q - o] == w[32 + q]);
            const uint64_t h = (ha[0] | ha[1]) | (ha[2] | ha[3]) | (ha[4] | ha[5]) | (ha[6] | ha[7]);
            full = WPC == 1 ? h != 0ull : __syncthreads_or(h != 0ull);
          }
#pragma unroll
          for (uint32_t q = 0; q < QS; ++q) om[q] = full ? mask_of(q) : 0u;
        } else {
#pragma unroll
          for (uint32_t q = 0; q < PPASS; ++q) om[q] = mask_of(q);
        }
        if (p0 < 32u) {  // offsets reach back to the chunk start at most: bits o - 1 < p
#pragma unroll
          for (uint32_t q = 0; q < PPASS; ++q) {
            const uint32_t p = p0 + q;
            if (p < 32u) om[q] &= (1u << p) - 1u;
          }
        }
        if constexpr (W > 32) {
          // offsets 33..W into bits 32..W-1, from the W - 32 + PPASS words
          // X[p0 - W ..]; offsets past the chunk start are masked off
          constexpr uint32_t HW = (uint32_t)W - 32u;
          uint32_t w2[HW + PPASS];
          if (p0 >= (uint32_t)W) {
#pragma unroll
            for (uint32_t i = 0; i < (HW + PPASS) / 4; ++i) {
              const uint4 v = *(const uint4*)(X + p0 - (uint32_t)W + 4u * i);
              w2[4 * i] = v.x;
              w2[4 * i + 1] = v.y;
              w2[4 * i + 2] = v.z;
              w2[4 * i + 3] = v.w;
            }
          } else {
#pragma unroll
            for (uint32_t i = 0; i < HW + PPASS; ++i) {
              const int32_t idx = (int32_t)p0 - W + (int32_t)i;
              w2[i] = idx >= 0 ? X[idx] : 0u;
            }
          }
#pragma unroll
          for (uint32_t q = 0; q < PPASS; ++q) {
            uint32_t hm = 0;
#pragma unroll
            for (uint32_t h = 0; h < HW / 16u; ++h) match_bits16(hm, &w2[q + 16u * h], w[32 + q]);
            const uint32_t p = p0 + q;
            hm = p >= (uint32_t)W ? hm : (p > 32u ? (hm & ((1u << (p - 32u)) - 1u)) : 0u);
            om[q] |= (Mask)hm << 32;
          }
        }
        // the masks overwrite X, which the whole team has read by now
        if (L::XW == 0) team_sync<WPC>();
#pragma unroll
        for (uint32_t q = 0; q < PPASS; ++q) {
          any_om |= om[q];
          LVm[p0 + q] = om[q];
        }
      }
    }
    // No near match anywhere in the chunk: every length is 0.  At level 0 the
    // parse is then E literals, F + D = E / 8 + CS > bc, so the chunk is raw
    // and the search and parse are skipped; level 1 still runs its table.
    // reloaded words for the candidate checks, loaded from the input now so
    // the loads overlap the descent (stored to XL after it)
    uint32_t xr[L::XL ? PPL : 1];
    if constexpr (L::XL) {
#pragma unroll
      for (uint32_t i = 0; i < PPL; ++i) xr[i] = word_at(g + i * TL);
    }
    bool near;
    if (WPC == 1) {
      near = __ballot(any_om != 0) != 0ull;
      wave_sync();
    } else {
      near = __syncthreads_or(any_om != 0);
    }
    if (LEVEL == 0 && !near) {
      K = (uint32_t)E;
    } else {
      if (L::LAZY && near) {
        // ---- 3 (short form). S_4 and a two-round descent for lengths below 16 ---------
        // S_4[p] = AND of S_1 over [p, p + 4) (0 past the chunk).  At each
        // position: t_j = AND of S_1 over [p, p + 4j) for j = 1..4 (nested
        // sets); t_4 not empty means L >= 16 and the position gets the long
        // mark.  Otherwise a = the number of non-empty t_1..t_3, then up to
        // three single steps from p + 4a: L = 4a + b < 16 exactly, O = the
        // smallest offset left.  S_1 and S_4 are followed by 16 zero words,
        // so no read needs a bounds check.
        uint32_t* S1 = LV;
        uint32_t* S4 = LV + L::LZ_T4;
        for (uint32_t i = g; i < 28u; i += TL) {
          if (i < 16u) S1[E + i] = 0u;
          else S4[E + i - 16u] = 0u;
        }
#pragma unroll
        for (uint32_t i = 0; i < PPL; ++i) {
          const uint32_t p = g + i * TL;
          uint32_t v = 0;
          if (p + 4u <= (uint32_t)E) v = S1[p] & S1[p + 1] & S1[p + 2] & S1[p + 3];
          S4[p] = v;
        }
        team_sync<WPC>();
        uint32_t lo[PPL];
#pragma unroll
        for (uint32_t i = 0; i < PPL; ++i) {
          const uint32_t p = g + i * TL;
          const uint32_t* T4 = S4 + p;
          const uint32_t t1 = T4[0], t2 = t1 & T4[4], t3 = t2 & T4[8], t4 = t3 & T4[12];
          const uint32_t a = (uint32_t)(t1 != 0u) + (uint32_t)(t2 != 0u) + (uint32_t)(t3 != 0u);
          const uint32_t sa = t3 ? t3 : (t2 ? t2 : (t1 ? t1 : ~0u));
          const uint32_t* T1 = S1 + p + 4u * a;
          const uint32_t u1 = sa & T1[0], u2 = u1 & T1[1], u3 = u2 & T1[2];
          const uint32_t b = (uint32_t)(u1 != 0u) + (uint32_t)(u2 != 0u) + (uint32_t)(u3 != 0u);
          const uint32_t fin = u3 ? u3 : (u2 ? u2 : (u1 ? u1 : sa));
          const uint32_t Ls = 4u * a + b;
          lo[i] = t4 ? kLongMark : (Ls ? (Ls | (((uint32_t)__builtin_ctz(fin) + 1u) << 8)) : 0u);
        }
        team_sync<WPC>();
#pragma unroll
        for (uint32_t i = 0; i < PPL; ++i) LO[g + i * TL] = lo[i];  // over S_4
        team_sync<WPC>();
      } else if (near) {
        // ---- 3. base-4 doubling table S_4, S_16 and a 4-round descent -----------------
        // S_k[p] = AND of omask over [p, p+k) when p + k <= E, else 0; every
        // table is followed by zeros, so descent reads past the chunk need no
        // bounds checks.  S_64[p] = S_16[p] & S_16[p+16] & S_16[p+32] &
        // S_16[p+48] is read that way in the first round instead of being
        // stored: one table less in LDS, so more chunks per CU.
        for (uint32_t i = g; i < L::PAD; i += TL) {  // padding word i of level lv is at (lv + 1) E + i
          const uint32_t lv = i < 4u ? 0u : (i < 16u ? 1u : 2u);
          LVm[(lv + 1u) * (uint32_t)E + i] = 0;
        }
#pragma unroll
        for (uint32_t lv = 1; lv < 3; ++lv) {
          const uint32_t k = 1u << (2 * lv), step = k >> 2;
          const Mask* prev = LVm + L::TOFF[lv - 1];
          Mask* cur = LVm + L::TOFF[lv];
#pragma unroll
          for (uint32_t i = 0; i < PPL; ++i) {
            const uint32_t p = g + i * TL;
            Mask v = 0;
            if (p + k <= (uint32_t)E) v = prev[p] & prev[p + step] & prev[p + 2 * step] & prev[p + 3 * step];
            cur[p] = v;
          }
          team_sync<WPC>();
        }
        // The descent at p: digits of L in base 4, most significant first, at
        // most 3 steps of k per round, so L <= 3 * (64 + 16 + 4 + 1) = 255, the
        // length cap.  Without the rounds of 64 and 16 (full false) it finds
        // exactly the lengths below 16.
        auto descend = [&](uint32_t p, bool full) -> uint32_t {
          Mask surv = ~(Mask)0;
          uint32_t Ln = 0;
          if (full) {
            // round of k = 64 (Ln = 0): S_64 at p, p + 64, p + 128 from S_16,
            // reads up to p + 176, inside S_16's padding (or guarded)
            const Mask* S = LVm + L::TOFF[2] + p;
            Mask s0 = 0, s1 = 0, s2 = 0;  // S_64 at p, p + 64, p + 128 (0 past the chunk)
            if (!L::GUARD64 || p + 64u <= (uint32_t)E) {
              s0 = S[0] & S[16] & S[32] & S[48];
              if (!L::GUARD64 || p + 128u <= (uint32_t)E) {
                s1 = S[64] & S[80] & S[96] & S[112];
                if (!L::GUARD64 || p + 192u <= (uint32_t)E) s2 = S[128] & S[144] & S[160] & S[176];
              }
            }
            const Mask t1 = surv & s0, t2 = t1 & s1, t3 = t2 & s2;
            const uint32_t n = (uint32_t)(t1 != 0) + (uint32_t)(t2 != 0) + (uint32_t)(t3 != 0);
            surv = t3 ? t3 : (t2 ? t2 : (t1 ? t1 : surv));
            Ln += n << 6;
          }
#pragma unroll
          for (int lv = 2; lv >= 0; --lv) {
            if (lv == 2 && !full) continue;
            const uint32_t k = 1u << (2 * lv);
            // p + Ln <= E (every surviving position is inside the chunk), so the
            // three reads end within the table's padding
            const Mask* S = LVm + L::TOFF[lv] + p + Ln;
            const Mask t1 = surv & S[0], t2 = t1 & S[k], t3 = t2 & S[2u * k];
            const uint32_t n = (uint32_t)(t1 != 0) + (uint32_t)(t2 != 0) + (uint32_t)(t3 != 0);
            surv = t3 ? t3 : (t2 ? t2 : (t1 ? t1 : surv));
            Ln += n << (2 * lv);
          }
          const uint32_t o = W > 32 ? (uint32_t)__builtin_ctzll((uint64_t)surv) : (uint32_t)__builtin_ctz((uint32_t)surv);
          return Ln ? (Ln | ((o + 1u) << 8)) : 0u;
        };
        // A wave none of whose positions g + i TL has S_16 non-empty (no
        // length of 16 or more; S_64 lies inside S_16) gains nothing from the
        // rounds of 64 and 16 and skips them there: most positions of most
        // data have short lengths only.  The votes come first, so that each
        // position takes one of the two descents (a wave-uniform branch).
        uint32_t lo[PPL];
        uint32_t longm = 0;  // bit i: the wave has a long length among positions g + i TL
#pragma unroll
        for (uint32_t i = 0; i < PPL; ++i)
          if (__ballot(LVm[L::TOFF[2] + g + i * TL] != (Mask)0) != 0ull) longm |= 1u << i;
#pragma unroll
        for (uint32_t i = 0; i < PPL; ++i) {
          if ((longm >> i) & 1u) lo[i] = descend(g + i * TL, true);
          else lo[i] = descend(g + i * TL, false);
        }
        team_sync<WPC>();
#pragma unroll
        for (uint32_t i = 0; i < PPL; ++i) LO[g + i * TL] = lo[i];
        team_sync<WPC>();
      } else {
#pragma unroll
        for (uint32_t i = 0; i < PPL; ++i) LO[g + i * TL] = 0u;
        team_sync<WPC>();
      }

      // ---- 4. level 1 ----------------------------------------------------------------------
      // matched: some position has a match (near or hashed); otherwise the
      // parse would be E literals, so the chunk is raw without one
      bool matched = true;
      if (LEVEL == 1) {
        bool hit = false;
        uint16_t* T16 = (uint16_t*)T;
        for (uint32_t i = g; i < L::TW_; i += TL) T[i] = 0u;
        if constexpr (L::XL) {
#pragma unroll
          for (uint32_t i = 0; i < PPL; ++i) XL[g + i * TL] = xr[i];
        }
        team_sync<WPC>();  // T (and a reloaded XL) overlay dead table levels
        constexpr uint32_t SB = E / kSubBlocks;
        static_assert(SB <= TL, "one position per lane per sub-block");
        // The next sub-block's key words and near lengths are loaded while
        // this one runs: the walk writes neither (it writes only the table and
        // the current sub-block's (L, O)).
        uint32_t nx0 = 0, nx1 = 0, nlo = 0;
        if (g < SB) {
          nx0 = XL[g];
          nx1 = XL[g + 1u];
          nlo = LO[g];
        }
#pragma unroll 1
        for (uint32_t s = 0; s < kSubBlocks; ++s) {
          const uint32_t x0 = nx0, x1 = nx1, lo_p = nlo;
          if (s + 1u < kSubBlocks && g < SB) {
            const uint32_t pn = (s + 1u) * SB + g;
            nx0 = XL[pn];
            nx1 = XL[pn + 1u];  // past the chunk only at pn = E - 1 (no key there; still inside LDS)
            nlo = LO[pn];
          }
          // One position per lane (consecutive lanes, consecutive positions).
          // A candidate replaces the near match only if its run is strictly
          // longer, so it must match at p + Lnear, and Lnear must leave room.
          // Each lane first measures its candidate's run itself, up to 8
          // compares.  Runs still open after that are shared along lanes:
          // when lanes l and l + 1 are open at the same offset, run(p) =
          // min(lim(p), run(p + 1) + 1), so only the last lane of such a chain
          // measures on, with the whole wave, 64 compares per step.  A
          // sub-block has at most one position per lane (SB <= TL); its
          // bucket is kept for the insert below.
          const uint32_t p = s * SB + g;
          const bool ins = g < SB && p + 1 < (uint32_t)E;
          const uint32_t bk = ins ? bucket_of(x0, x1) : 0u;
          if (g < SB) {
            uint32_t o = 0, Lnear = 0, lim = 0;
            bool need = false;
            uint32_t r = 0;
            bool open = false;
            if (ins) {
              const uint32_t v = L::HT16 ? (uint32_t)T16[bk] : T[bk];
              o = p - (v - 1u);  // entries come from earlier sub-blocks: o >= 1
              lim = (uint32_t)E - p < kMaxLen ? (uint32_t)E - p : kMaxLen;
              Lnear = lo_p & 0xFFu;
              if (v != 0u && o <= kMaxFar && Lnear < lim) {
                // The word at p + Lnear first (the candidate must match there
                // to be longer), then, only where it does, the first 8 word
                // pairs.  Words past the chunk's end (p + 7 < E + 8) still lie
                // in the team's LDS, since the word region is followed by
                // other regions, and their bits are set by j >= lim anyway.
                const uint32_t xa = XL[p + Lnear], xb = XL[p + Lnear - o];
                need = xa == xb;
                if (need) {
                  uint32_t wa[8], wb[8];
#pragma unroll
                  for (uint32_t j = 0; j < 8u; ++j) {
                    wa[j] = XL[p + j];
                    wb[j] = XL[p + j - o];
                  }
                  uint32_t stop = 0;
#pragma unroll
                  for (uint32_t j = 0; j < 8u; ++j) stop |= (uint32_t)((j >= lim) | (wa[j] != wb[j])) << j;
                  r = stop ? (uint32_t)__builtin_ctz(stop) : 8u;
                  open = stop == 0u;
                }
              }
            }
            const uint64_t openm = __ballot(open);
            if (openm) {  // long runs (lim > 8 for every open lane)
              const uint32_t o_next =
                  (uint32_t)__builtin_amdgcn_ds_bpermute((int)(((lane + 1u) & 63u) << 2), (int)o);
              const bool link = open && lane < 63u && ((openm >> (lane + 1u)) & 1ull) && o_next == o;
              const uint64_t ends = openm & ~__ballot(link);
              uint32_t r_end = r;
              for (uint64_t m = ends; m;) {
                const uint32_t e = (uint32_t)__builtin_ctzll(m);
                m &= m - 1ull;
                const uint32_t pe = (uint32_t)__builtin_amdgcn_readlane((int)p, (int)e);
                const uint32_t oe = (uint32_t)__builtin_amdgcn_readlane((int)o, (int)e);
                const uint32_t le = (uint32_t)__builtin_amdgcn_readlane((int)lim, (int)e);
                // its first 8 matched; then 64 compares, and if the run goes
                // on, the other three rounds of 64 (le <= 255) with all their
                // words read at once, so a long run waits on two LDS latencies
                // instead of four.  Words past the run (idx >= le) are read
                // too, still inside the team's LDS (the regions after the
                // words hold more than 264), and do not count.
                uint32_t re;
                {
                  const uint32_t idx = 8u + lane;
                  const uint64_t sm = __ballot(idx >= le || XL[pe + idx] != XL[pe + idx - oe]);
                  re = sm ? 8u + (uint32_t)__builtin_ctzll(sm) : 72u;
                }
                if (re == 72u && le > 72u) {
                  uint32_t xa[3], xb[3];
#pragma unroll
                  for (uint32_t u = 0; u < 3u; ++u) {
                    const uint32_t idx = 72u + 64u * u + lane;
                    xa[u] = XL[pe + idx];
                    xb[u] = XL[pe + idx - oe];
                  }
#pragma unroll
                  for (int u = 2; u >= 0; --u) {
                    const uint32_t idx = 72u + 64u * (uint32_t)u + lane;
                    const uint64_t sm = __ballot(idx >= le || xa[u] != xb[u]);
                    if (sm) re = 72u + 64u * (uint32_t)u + (uint32_t)__builtin_ctzll(sm);
                  }
                }
                if (lane == e) r_end = re;
              }
              // chain members: run = min(lim, distance to the chain's end + its run)
              const uint64_t after = lane == 63u ? 0ull : (ends >> (lane + 1u)) << (lane + 1u);
              const uint32_t e = ((ends >> lane) & 1ull) ? lane : (after ? (uint32_t)__builtin_ctzll(after) : lane);
              const uint32_t re = (uint32_t)__builtin_amdgcn_ds_bpermute((int)(e << 2), (int)r_end);
              const uint32_t run = re + (e - lane);
              if (open) r = run < lim ? run : lim;
            }
            if (need && r > Lnear) {
              LO[p] = r | (o << 8);
              hit = true;
            }
          }
          team_sync<WPC>();
          if constexpr (L::HT16) {
            // every insert of this sub-block is larger than anything stored
            // before, so the bucket must end with the largest of them: plain
            // 16-bit stores, then whoever still sees a smaller value stores
            // again until nobody does (the same result as atomicMax)
            if (ins) T16[bk] = (uint16_t)(p + 1u);
            team_sync<WPC>();
            while (true) {
              const bool lose = ins && (uint32_t)T16[bk] < p + 1u;
              const bool again = WPC == 1 ? __ballot(lose) != 0ull : __syncthreads_or(lose);
              if (!again) break;
              if (lose) T16[bk] = (uint16_t)(p + 1u);
              team_sync<WPC>();
            }
          } else {
            if (ins) atomicMax(&T[bk], p + 1u);
            team_sync<WPC>();
          }
        }
        if (WPC == 1) matched = near || __ballot(hit) != 0ull;
        else matched = near || __syncthreads_or(hit);
      }

      if (!matched) {
        K = (uint32_t)E;
      } else {
        // ---- 5. parallel greedy parse --------------------------------------------------------
        // (a) per segment of 8 positions: for every entry q, the exit position and
        //     the item-start mask of the parse walked from q.
        for (uint32_t sg = g; sg < L::NSEG; sg += TL) {
          const uint32_t p0 = sg * 8u;
          const uint4 a = *(const uint4*)(LO + p0);
          const uint4 b = *(const uint4*)(LO + p0 + 4);
          const uint32_t l8[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
          // Byte q of a lo / hi pair of words describes position p0 + q (q < 4
          // in lo).  perm(h, l, s) is v_perm_b32: byte i of the result is byte
          // s_i of the 8-byte table {h:l} (0-7), or 0 for s_i = 12, so it
          // looks up eight bytes at once by a word of byte indices.
          auto perm = [](uint32_t h, uint32_t l, uint32_t sel) -> uint32_t {
            return __builtin_amdgcn_perm(h, l, sel);
          };
          constexpr uint32_t H = 0x80808080u;
          // per-byte unsigned a >= b for bytes b < 128: bit 7 of each byte
          auto ge = [](uint32_t a, uint32_t b) -> uint32_t { return (((a | H) - b) | a) & H; };
          auto full = [](uint32_t t) -> uint32_t { return (t - (t >> 7)) | t; };  // bit 7 -> 0xFF
          // the lengths (low byte of each (L, O))
          const uint32_t LEN[2] = {perm(l8[1], l8[0], 0x0c0c0400u) | perm(l8[3], l8[2], 0x04000c0cu),
                                   perm(l8[5], l8[4], 0x0c0c0400u) | perm(l8[7], l8[6], 0x04000c0cu)};
          constexpr uint32_t THR[2] = {0x05060708u, 0x01020304u};  // 8 - q
          constexpr uint32_t QI[2] = {0x03020100u, 0x07060504u};   // q
          uint32_t MT[2], STEP[2], N[2], I[2] = {0x08040201u, 0x80402010u}, LG[2];
#pragma unroll
          for (uint32_t h = 0; h < 2u; ++h) {
            MT[h] = full(ge(LEN[h], MM * 0x01010101u));                       // a match starts here
            STEP[h] = (MT[h] & LEN[h]) | (~MT[h] & 0x01010101u);              // its item's length
            const uint32_t out = full(ge(STEP[h], THR[h]));                   // the item leaves the segment
            N[h] = QI[h] + (STEP[h] & ~out);                                  // next entry (itself if out)
            // level 0: a long mark (length byte 0xFF, all others below 16)
            // ends the walk at its own position with a flagged exit
            LG[h] = L::LAZY ? full(LEN[h] & H) : 0u;
          }
          // pointer doubling on the segment: after round r, N = the entry
          // 2^r items on (or the last one, whose item leaves), I = the item
          // starts passed on the way (7 items at most: three rounds)
#pragma unroll
          for (uint32_t r = 0; r < 3u; ++r) {
            const uint32_t i0 = I[0] | perm(I[1], I[0], N[0]), i1 = I[1] | perm(I[1], I[0], N[1]);
            const uint32_t n0 = perm(N[1], N[0], N[0]), n1 = perm(N[1], N[0], N[1]);
            I[0] = i0, I[1] = i1, N[0] = n0, N[1] = n1;
          }
          // exit = p0 + last + its length (long mark: p0 + last, flagged);
          // two exits per word, one in each 16-bit half
          const uint32_t SX[2] = {STEP[0] & ~LG[0], STEP[1] & ~LG[1]};
          const uint32_t P0P0 = p0 | (p0 << 16);
          uint32_t ex2[4];
#pragma unroll
          for (uint32_t h = 0; h < 2u; ++h) {
            const uint32_t sf = perm(SX[1], SX[0], N[h]);
            const uint32_t lf = L::LAZY ? perm(LG[1], LG[0], N[h]) : 0u;
#pragma unroll
            for (uint32_t k = 0; k < 2u; ++k) {
              const uint32_t sel = k ? 0x0c030c02u : 0x0c010c00u;  // bytes 2k, 2k + 1 to the halves
              uint32_t e = perm(0u, N[h], sel) + perm(0u, sf, sel) + P0P0;
              if constexpr (L::LAZY) e |= perm(0u, lf, k ? 0x030c020cu : 0x010c000cu) & 0x80008000u;
              ex2[2u * h + k] = e;
            }
          }
          const uint32_t lmb = __builtin_amdgcn_sad_u8(MT[1] & 0x80402010u, 0u,
                                                       __builtin_amdgcn_sad_u8(MT[0] & 0x08040201u, 0u, 0u));
          if constexpr (L::LAZY) {
            // the exit beside (L, O), the bits in their own bytes
            uint32_t w[8];
#pragma unroll
            for (uint32_t q = 0; q < 8u; ++q) w[q] = perm(ex2[q / 2u], l8[q], (q & 1u) ? 0x07060100u : 0x05040100u);
            *(uint4*)(LO + p0) = make_uint4(w[0], w[1], w[2], w[3]);
            *(uint4*)(LO + p0 + 4) = make_uint4(w[4], w[5], w[6], w[7]);
            *(uint2*)(IM + p0) = make_uint2(I[0], I[1]);
          } else {
            // exit | item-start bits << 16
            uint32_t w[8];
#pragma unroll
            for (uint32_t q = 0; q < 8u; ++q) {
              const uint32_t eb = (q & 1u) ? 0x0302u : 0x0100u;           // the exit's two bytes
              const uint32_t ib = 0x04u + (q & 3u);                        // byte q & 3 of I
              w[q] = perm(I[q / 4u], ex2[q / 2u], 0x0c000000u | (ib << 16) | eb);
            }
            *(uint4*)(XQ + p0) = make_uint4(w[0], w[1], w[2], w[3]);
            *(uint4*)(XQ + p0 + 4) = make_uint4(w[4], w[5], w[6], w[7]);
          }
          ((uint8_t*)LMB)[sg] = (uint8_t)lmb;
          ((uint8_t*)ISB)[sg] = 0;  // the rebuild below sets the bytes of the segments the parse passes
        }
        team_sync<WPC>();
        // (b) hops: the parse's real entry into every segment it passes through
        if constexpr (WPC < 4) {
          // One or two waves (up to 16 words): the first wave does it all, in
          // three steps.  First, for every position p, where the parse leaves
          // p's 64-position word if it enters the word at p: one word at a
          // time, lane j on position 64w + j, a segment hop is a lane
          // exchange and three rounds of pointer doubling cover the word's 8
          // segments.  A long-match exit (level 0: flagged, past every word
          // bound) ends a chain like a word exit.  The exits stay in
          // registers, two 16-bit ones to a register.  Second, the parse
          // itself, a word at a time (one readlane per hop; where a long
          // match starts, the wave finds its exact length, stores it and
          // goes on after it).  Third, lane w rebuilds word w's item-start
          // bits from the parse's first entry into the word (at most 8 hops,
          // the lengths of long matches read back).
          static_assert(NR % 2u == 0u && NR <= 64u, "word exits in pairs, one lane per word");
          if (g < 64u) {
            // (positions are carried times 4, the byte address of their lane:
            // ds_bpermute ignores the bits above the lane index)
            uint32_t wxp[NR / 2u];
#pragma unroll
            for (uint32_t k = 0; k < NR; ++k) {
              const uint32_t wend4 = 256u * (k + 1u);
              uint32_t x4 = (xq_at(64u * k + lane) & 0xFFFFu) << 2;
#pragma unroll
              for (uint32_t r = 0; r < 3u; ++r) {
                const uint32_t y4 = (uint32_t)__builtin_amdgcn_ds_bpermute((int)x4, (int)x4);
                if (x4 < wend4) x4 = y4;
              }
              if (k & 1u) wxp[k / 2u] |= (x4 >> 2) << 16;
              else wxp[k / 2u] = x4 >> 2;
            }
            uint32_t P = 0, ent = 0xFFFFu;  // lane w: the parse's first entry into word w
#pragma unroll
            for (uint32_t w = 0; w < NR; ++w) {
              if (lane == w && P < 64u * (w + 1u)) ent = P;
              while (P < 64u * (w + 1u)) {
                const uint32_t v = (uint32_t)__builtin_amdgcn_readlane((int)wxp[w / 2u], (int)(P & 63u));
                const uint32_t X = (w & 1u) ? v >> 16 : v & 0xFFFFu;
                if (L::LAZY && (X & kLongExit)) {
                  const uint32_t r = X & ~kLongExit;  // a long match starts at r
                  const uint32_t lv = long_match(LV, r, (uint32_t)E);
                  if (lane == 0u) *(uint16_t*)(LO + r) = (uint16_t)lv;  // (L, O); the exit half stays
                  P = r + ((lv & 0xFFu) ? (lv & 0xFFu) : 1u);  // L >= 16 here; the select only guards progress
                } else {
                  P = X;
                }
              }
            }
            wave_sync();  // the long matches' lengths, before the rebuild reads them
            if (lane < NR && ent != 0xFFFFu) {
              // a segment's exit lies past its end, and a long match found in
              // a segment ends at least 16 positions on: each hop passes a
              // segment, whose item-start byte it writes
              const uint32_t wend = 64u * (lane + 1u);
              uint32_t Q = ent;
#pragma unroll
              for (uint32_t h = 0; h < 8u; ++h) {
                if (Q < wend) {
                  const uint32_t xq = xq_at(Q);
                  ((uint8_t*)ISB)[Q >> 3] = (uint8_t)(xq >> 16);
                  uint32_t X = xq & 0xFFFFu;
                  if (L::LAZY && (X & kLongExit)) {
                    const uint32_t r = X & ~kLongExit;
                    const uint32_t Lr = LO[r] & 0xFFu;
                    X = r + (Lr ? Lr : 1u);
                  }
                  Q = X;
                }
              }
            }
          }
          team_sync<WPC>();
        } else {
          // four or more waves: the same three steps, the first one shared by
          // all waves (a wave takes one word at a time, all positions at
          // once), its exits passed to the first wave through WX, a u16 per
          // position (there are no long-match exits here).  WX uses
          // space that is free here: the staging area (word sizes 2 and 4)
          // or the dead search tables past the parse region (word size 1).
          static_assert(NR <= 64u, "one lane per 64-position word");
          static_assert(WS >= 2 || L::RP + E / 2u <= L::R, "word exits fit past the parse region");
          uint16_t* WX = (uint16_t*)(WS >= 2 ? (uint32_t*)STG : LV + L::RP);
          {
            // P[i]: where the parse is after 2^r segment hops from
            // position g + i TL, or the word exit once it has left the
            // word (every exit inside the word lies in this wave's lanes);
            // carried times 4, the byte address of the lane, as above
            uint32_t P[PPL];
#pragma unroll
            for (uint32_t i = 0; i < PPL; ++i) P[i] = (XQ[g + i * TL] & 0xFFFFu) << 2;
#pragma unroll
            for (uint32_t r = 0; r < 3u; ++r) {
#pragma unroll
              for (uint32_t i = 0; i < PPL; ++i) {
                const uint32_t wend4 = (((g + i * TL) | 63u) + 1u) << 2;
                const uint32_t y = (uint32_t)__builtin_amdgcn_ds_bpermute((int)P[i], (int)P[i]);
                if (P[i] < wend4) P[i] = y;
              }
            }
#pragma unroll
            for (uint32_t i = 0; i < PPL; ++i) WX[g + i * TL] = (uint16_t)(P[i] >> 2);
          }
          team_sync<WPC>();
          if (g < 64u) {
            // every word's exits in registers first, two to a register
            // (word w in half w & 1 of register w / 2, lane j: position
            // 64w + j), so that each hop is one readlane and no hop waits
            // for a load
            static_assert(NR % 2u == 0u, "word exits in pairs");
            uint32_t wxp[NR / 2u];
#pragma unroll
            for (uint32_t k = 0; k < NR / 2u; ++k)
              wxp[k] = (uint32_t)WX[128u * k + lane] | ((uint32_t)WX[128u * k + 64u + lane] << 16);
            uint32_t P = 0, ent = 0xFFFFu;  // lane w: the parse's entry into word w
#pragma unroll
            for (uint32_t w = 0; w < NR; ++w) {
              if (P < 64u * (w + 1u)) {  // else a match spans the whole word
                if (lane == w) ent = P;
                const uint32_t v = (uint32_t)__builtin_amdgcn_readlane((int)wxp[w / 2u], (int)(P & 63u));
                P = (w & 1u) ? v >> 16 : v & 0xFFFFu;
              }
            }
            if (lane < NR && ent != 0xFFFFu) {
              const uint32_t wend = 64u * (lane + 1u);
              uint32_t Q = ent;
#pragma unroll
              for (uint32_t h = 0; h < 8u; ++h) {
                if (Q < wend) {
                  const uint32_t xq = XQ[Q];
                  ((uint8_t*)ISB)[Q >> 3] = (uint8_t)(xq >> 16);
                  Q = xq & 0xFFFFu;
                }
              }
            }
          }
          team_sync<WPC>();
        }
        // ---- 6. counts: lane g takes segment g (there are never more
        // segments than lanes); one packed scan gives the items and matches
        // of the segments before it and the chunk's totals
        static_assert(L::NSEG <= TL, "a segment per lane");
        it8 = g < L::NSEG ? (uint32_t)((const uint8_t*)ISB)[g] : 0u;
        mt8 = g < L::NSEG ? (uint32_t)((const uint8_t*)LMB)[g] & it8 : 0u;
        const uint32_t cnt = (uint32_t)__builtin_popcount(it8) | ((uint32_t)__builtin_popcount(mt8) << 16);
        const uint32_t inc = wave_incl_add(cnt);
        uint32_t tot;
        if constexpr (WPC == 1) {
          tot = lane63(inc);
          kex = inc - cnt;
        } else {
          const uint32_t wv = g >> 6;
          if (lane == 63u) KB[wv] = inc;
          team_sync<WPC>();
          uint32_t pre = 0;
          tot = 0;
#pragma unroll
          for (uint32_t w = 0; w < (uint32_t)WPC; ++w) {
            const uint32_t t = KB[w];
            pre += w < wv ? t : 0u;
            tot += t;
          }
          kex = pre + inc - cnt;
        }
        K = tot & 0xFFFFu;
        M = tot >> 16;
      }  // some match
    }  // near match, or level 1
  }  // nonzero
  const uint32_t F = (K + 7u) / 8u;
  const uint32_t D = (uint32_t)WS * (K - M) + 2u * M;
  const bool raw = nonzero && F + D >= bc;

  // ---- 7. size-table row, payload into the chunk's staging slot --------------------
  // Flags first (bit k of the bitmap = item k is a match), then the data bytes
  // right after them, so the slot holds the payload exactly as it will appear
  // in the stream; the compaction kernel moves it to its final offset.  In
  // LDS the data bytes start on a 4-byte boundary DB and the flag bytes end
  // there (the payload is STG[DB - F, DB + D)), so literals and match tokens
  // go in with 16-bit writes (word sizes 2 and 4); the copy to the slot
  // realigns by DB - F bytes.
  uint32_t* STG32 = (uint32_t*)STG;
  uint32_t* slot = (uint32_t*)(staging + base);
  if (konst) {
    // payload byte j by lane j (F + D < 64): flag bits 1 .. M set (the
    // matches are items 1 .. M); data: the word, M tokens (255 or the rest,
    // offset 1), then the trailing literals, each the word again
    const uint32_t j = g;
    if (j < F + D) {
      uint32_t b;
      if (j < F) {
        const uint32_t lo = 8u * j, hi = lo + 8u;                 // items [lo, hi)
        const uint32_t a0 = lo > 1u ? lo : 1u, a1 = hi < M + 1u ? hi : M + 1u;  // matches in it
        b = a0 < a1 ? ((1u << (a1 - lo)) - (1u << (a0 - lo))) & 0xFFu : 0u;
      } else {
        const uint32_t d = j - F;
        if (d < (uint32_t)WS) {
          b = (rep >> (8u * d)) & 0xFFu;
        } else if (d < (uint32_t)WS + 2u * M) {
          const uint32_t t = d - (uint32_t)WS;
          b = (t & 1u) ? 1u : ((t >> 1) < KN ? kMaxLen : KR);
        } else {
          b = (rep >> (8u * ((d - (uint32_t)WS - 2u * M) % (uint32_t)WS))) & 0xFFu;
        }
      }
      (staging + base)[j] = (uint8_t)b;
    }
  } else if (nonzero && !raw) {
    // Lane g places the items of segment g (positions 8g .. 8g + 7): they are
    // items kex.lo .. of the chunk and their data bytes are consecutive.  The
    // segment's (L, O) and literal words are loaded before the flag words are
    // cleared, so the loads overlap.
    const uint32_t DB = (F + 3u) & ~3u;
    const uint32_t S0 = DB - F;  // payload byte 0 is STG byte S0
    const uint32_t p0 = 8u * g;
    uint32_t lo8[8], xw[8];
#pragma unroll
    for (uint32_t q = 0; q < 8u; ++q) lo8[q] = xw[q] = 0u;
    if (g < L::NSEG) {
      const uint4 a = *(const uint4*)(LO + p0), b = *(const uint4*)(LO + p0 + 4u);
      lo8[0] = a.x, lo8[1] = a.y, lo8[2] = a.z, lo8[3] = a.w, lo8[4] = b.x, lo8[5] = b.y, lo8[6] = b.z, lo8[7] = b.w;
      if constexpr (L::XW != 0u) {  // the words in their own region
        const uint4 u = *(const uint4*)(X + p0), v = *(const uint4*)(X + p0 + 4u);
        xw[0] = u.x, xw[1] = u.y, xw[2] = u.z, xw[3] = u.w, xw[4] = v.x, xw[5] = v.y, xw[6] = v.z, xw[7] = v.w;
      } else if (bc == CS && (((uintptr_t)src) & 15u) == 0u) {  // from the input, 8 WS bytes at once
        if constexpr (WS == 4) {
          const uint4 u = ((const uint4*)src)[2u * g], v = ((const uint4*)src)[2u * g + 1u];
          xw[0] = u.x, xw[1] = u.y, xw[2] = u.z, xw[3] = u.w, xw[4] = v.x, xw[5] = v.y, xw[6] = v.z, xw[7] = v.w;
        } else if constexpr (WS == 2) {
          const uint4 u = ((const uint4*)src)[g];
          const uint32_t w4[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
          for (uint32_t j = 0; j < 4u; ++j) {
            xw[2u * j] = w4[j] & 0xFFFFu;
            xw[2u * j + 1u] = w4[j] >> 16;
          }
        } else {
          const uint2 u = ((const uint2*)src)[g];
#pragma unroll
          for (uint32_t j = 0; j < 4u; ++j) {
            xw[j] = (u.x >> (8u * j)) & 0xFFu;
            xw[4u + j] = (u.y >> (8u * j)) & 0xFFu;
          }
        }
      } else {
#pragma unroll
        for (uint32_t q = 0; q < 8u; ++q) xw[q] = word_at(p0 + q);
      }
    }
    for (uint32_t i = g; i < DB / 4u; i += TL) STG32[i] = 0u;
    team_sync<WPC>();
    // item k: flag bit 8 S0 + k of STG; data bytes at DB + WS (k - m) + 2 m
    // (m = matches before it).  The segment's items are consecutive, so its
    // data pointer and item count just advance.
    const uint32_t k0 = kex & 0xFFFFu, m0 = kex >> 16;
    uint8_t* dp = STG + DB + (uint32_t)WS * (k0 - m0) + 2u * m0;
    uint32_t j = 0, fl = 0;
#pragma unroll
    for (uint32_t q = 0; q < 8u; ++q) {
      if (!((it8 >> q) & 1u)) continue;
      if ((mt8 >> q) & 1u) {
        fl |= 1u << j;
        if (WS >= 2) {
          *(uint16_t*)dp = (uint16_t)lo8[q];
        } else {
          dp[0] = (uint8_t)lo8[q];
          dp[1] = (uint8_t)(lo8[q] >> 8);
        }
        dp += 2;
      } else {
        if (WS == 4) {
          *(uint16_t*)dp = (uint16_t)xw[q];
          *(uint16_t*)(dp + 2) = (uint16_t)(xw[q] >> 16);
        } else if (WS == 2) {
          *(uint16_t*)dp = (uint16_t)xw[q];
        } else {
          dp[0] = (uint8_t)xw[q];
        }
        dp += WS;
      }
      ++j;
    }
    // the segment's flag bits (at most 8, in item order) into the bitmap
    if (fl) {
      const uint32_t fb = 8u * S0 + k0, sh = fb & 31u;
      atomicOr(&STG32[fb >> 5], fl << sh);
      if (sh > 24u && (fl >> (32u - sh)) != 0u) atomicOr(&STG32[(fb >> 5) + 1u], fl >> (32u - sh));
    }
    team_sync<WPC>();
    const uint32_t nd = (F + D + 3u) / 4u;
    for (uint32_t i = g; i < nd; i += TL) {
      const uint32_t a = STG32[i], b = STG32[i + 1];
      slot[i] = S0 ? __builtin_amdgcn_alignbyte(b, a, S0) : a;
    }
  }
  if (g == 0) {
    const uint2 ent = !nonzero ? make_uint2(0u, 0u) : (raw ? make_uint2(0u, kRawBit | bc) : make_uint2(F, D));
    uint8_t* row = table + kEntryBytes * (uint64_t)c;
    if ((((uintptr_t)row) & 7u) == 0) {
      *(uint2*)row = ent;
    } else {
      put_le(row, ent.x, 4);
      put_le(row + 4, ent.y, 4);
    }
    // items and matches of the chunk, for the split-mode assembly (coded
    // chunks; zero and raw chunks report none)
    if (km) km[c] = (nonzero && !raw) ? make_uint2(K, M) : make_uint2(0u, 0u);
    // the first team of workgroup b clears tile flag b of every flag set of
    // the assembly kernel (there are never more tiles than workgroups),
    // workgroup 0 the error flag
    if (team == 0 && blockIdx.x < num_tiles)
      for (uint32_t k = 0; k < flag_sets; ++k) tile_flags[(uint64_t)k * num_tiles + blockIdx.x] = 0ull;
    if (team == 0 && blockIdx.x == 0) ctl->error = 0u;
  }
}

// Compaction: one workgroup per tile of kCTile chunks.  Reads the tile's
// size-table rows, scans the payload sizes, finds the tile's output offset
// by decoupled look-back over the tiles before it, then moves every payload
// to its place in the stream: a coded chunk's from its staging slot, a raw
// chunk's straight from the input.  The last tile writes the header and the
// stream length.
template <uint32_t NB>
__global__ __launch_bounds__(NB) void compact_kernel(const uint8_t* __restrict__ in,
                                                         const uint8_t* __restrict__ staging, uint32_t cs,
                                                         uint32_t ws, uint64_t n, uint32_t num_chunks,
                                                         uint32_t num_tiles, uint8_t* __restrict__ out,
                                                         uint64_t* __restrict__ out_bytes,
                                                         uint64_t* __restrict__ tile_flags,
                                                         EncCtl* __restrict__ ctl) {
  __shared__ uint64_t tile_pre;
  const uint32_t tid = threadIdx.x, lane = lane_id(), wave = tid >> 6;
  const uint8_t* table = out + kHeaderBytes;
  uint8_t* payload = out + kHeaderBytes + (uint64_t)kEntryBytes * num_chunks;
  if (num_chunks == 0) {  // empty input: the header is the whole stream
    if (tid == 0) {
      put_le(out + 0, kMagic, 4);
      out[4] = (uint8_t)kVersion;
      out[5] = (uint8_t)ws;
      out[6] = 0;
      out[7] = 0;
      put_le(out + 8, cs, 4);
      put_le(out + 12, 0u, 4);
      put_le(out + 16, n, 8);
      put_le(out + 24, 0ull, 8);
      *out_bytes = kHeaderBytes;
    }
    return;
  }
  const uint32_t t = blockIdx.x;
  const uint64_t c0 = (uint64_t)t * kCTile;
  // Wave w moves chunks PW w .. PW w + PW - 1 of the tile.  The first 256
  // bytes of each of their staging slots (one dword per lane) are loaded
  // before any size or offset is known, so the loads overlap the row reads
  // and the look-back (a raw chunk's slot is never read past this).
  constexpr uint32_t PW = kCTile / (NB / 64u);
  typedef uint32_t pv_t __attribute__((ext_vector_type(PW)));  // a value, never memory
  pv_t pv;
#pragma unroll
  for (uint32_t u = 0; u < PW; ++u) {
    const uint64_t c = c0 + wave * PW + u;
    pv[u] = c < num_chunks ? ((const uint32_t*)(staging + c * cs))[lane] : 0u;
  }
  // Every wave reads the tile's rows (one chunk per lane) and scans the sizes
  // itself, so only the tile's offset has to be shared.
  static_assert(kCTile == 64, "one chunk per lane");
  uint32_t size = 0, raw = 0;
  {
    const uint64_t c = c0 + lane;
    if (c < num_chunks) {
      const uint8_t* row = table + kEntryBytes * c;
      uint2 e;
      if ((((uintptr_t)table) & 7u) == 0) {
        e = *(const uint2*)row;
      } else {
        e.x = (uint32_t)row[0] | ((uint32_t)row[1] << 8) | ((uint32_t)row[2] << 16) | ((uint32_t)row[3] << 24);
        e.y = (uint32_t)row[4] | ((uint32_t)row[5] << 8) | ((uint32_t)row[6] << 16) | ((uint32_t)row[7] << 24);
      }
      // a row never stands for more than the chunk's real bytes; the clamp
      // keeps every write inside the stream even if a row were wrong
      const uint64_t start = c * cs;
      const uint32_t bc = (uint32_t)((n - start) < cs ? (n - start) : cs);
      const uint32_t s0 = entry_payload(e.x, e.y);
      size = s0 < bc ? s0 : bc;
      raw = (e.x == 0u && (e.y & kRawBit)) ? 1u : 0u;
    }
  }
  const uint32_t inc = wave_incl_add(size);
  const uint32_t excl = inc - size;
  if (wave == 0) {
    const uint64_t tot = (uint64_t)lane63(inc);
    const uint64_t pre = look_back(tile_flags, t, tot, &ctl->error);
    if (lane == 0) {
      tile_pre = pre;
      if (t == num_tiles - 1u) {
        const uint64_t pb = pre + tot;
        put_le(out + 0, kMagic, 4);
        out[4] = (uint8_t)kVersion;
        out[5] = (uint8_t)ws;
        out[6] = 0;
        out[7] = 0;
        put_le(out + 8, cs, 4);
        put_le(out + 12, num_chunks, 4);
        put_le(out + 16, n, 8);
        put_le(out + 24, pb, 8);
        *out_bytes = __hip_atomic_load(&ctl->error, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                         ? 0ull
                         : (uint64_t)kHeaderBytes + (uint64_t)kEntryBytes * num_chunks + pb;
      }
    }
  }
  __syncthreads();
  uint8_t* const dst0 = payload + tile_pre;
  // the first bytes of every coded payload, from the loaded dwords
#pragma unroll
  for (uint32_t u = 0; u < PW; ++u) {
    const uint32_t j = wave * PW + u;
    const uint32_t sz = (uint32_t)__builtin_amdgcn_readlane((int)size, (int)j);
    if (sz == 0u || __builtin_amdgcn_readlane((int)raw, (int)j)) continue;
    uint8_t* dst = dst0 + (uint32_t)__builtin_amdgcn_readlane((int)excl, (int)j);
    // head bytes up to dst's next 4-byte boundary, then aligned dwords, then
    // the tail; payload byte b is byte b & 3 of slot dword b >> 2
    const uint32_t a4 = (uint32_t)((4u - ((uintptr_t)dst & 3u)) & 3u);
    const uint32_t h = a4 > sz ? sz : a4;
    const uint32_t nb = (sz - h) / 4u;
    const uint32_t d0 = (uint32_t)__builtin_amdgcn_readfirstlane((int)pv[u]);
    if (lane < h) dst[lane] = (uint8_t)(d0 >> (8u * lane));
    uint32_t* dw = (uint32_t*)(dst + h);
    // body dword k takes slot dwords k and k + 1 (the next lane's)
    const uint32_t nxt = dpp0<kWaveShl1>(pv[u]);
    if (lane < (nb < 63u ? nb : 63u)) dw[lane] = __builtin_amdgcn_alignbyte(nxt, pv[u], h);
    if (nb < 63u) {
      const uint32_t tb = h + 4u * nb + lane;  // at most 3 tail bytes, below h + 251
      const uint32_t tv = (uint32_t)__builtin_amdgcn_ds_bpermute((int)((tb >> 2) & 63u) << 2, (int)pv[u]);
      if (tb < sz) dst[tb] = (uint8_t)(tv >> (8u * (tb & 3u)));
    }
  }
  // the rest of coded payloads longer than that, and raw chunks, whose
  // payload is their input bytes
#pragma unroll 1
  for (uint32_t u = 0; u < PW; ++u) {
    const uint32_t j = wave * PW + u;
    const uint32_t sz = (uint32_t)__builtin_amdgcn_readlane((int)size, (int)j);
    if (sz == 0u) continue;
    uint8_t* dst = dst0 + (uint32_t)__builtin_amdgcn_readlane((int)excl, (int)j);
    const uint64_t c = c0 + j;
    if (__builtin_amdgcn_readlane((int)raw, (int)j)) {
      copy_bytes16(dst, in + c * cs, sz, lane);
      continue;
    }
    const uint32_t a4 = (uint32_t)((4u - ((uintptr_t)dst & 3u)) & 3u);
    const uint32_t h = a4 > sz ? sz : a4;
    if ((sz - h) / 4u >= 63u) {
      const uint32_t done = h + 4u * 63u;
      copy_bytes16(dst + done, staging + c * cs + done, sz - done, lane);
    }
  }
}

// Split-mode assembly (codebase notes CN-GPULZ-1, split mode; GPULZStage page,
// split-mode paragraphs): one workgroup per tile of kCTile chunks.  A chunk
// contributes flag bytes to the meta port, literal bytes (its literal words,
// or all its bytes when raw) to the literals port and one byte per match to
// each of the lengths and offsets ports; three scans with decoupled look-back
// (one flag set each) place them.  Coded chunks' rows become {items,
// matches}; then every wave copies its raw chunks from the input and deals
// its coded chunks' items into the ports, each payload first brought from
// its staging slot into LDS with 16-byte loads.  The last tile writes the
// header and the port lengths.
__global__ __launch_bounds__(kBlock) void split_compact_kernel(
    const uint8_t* __restrict__ in, const uint8_t* __restrict__ staging, const uint2* __restrict__ km, uint32_t cs,
    uint32_t ws, uint64_t n,
    uint32_t num_chunks, uint32_t num_tiles, uint8_t* __restrict__ meta, uint8_t* __restrict__ lit,
    uint8_t* __restrict__ lens, uint8_t* __restrict__ offs, uint64_t* __restrict__ port_bytes,
    uint64_t* __restrict__ tile_flags, EncCtl* __restrict__ ctl) {
  __shared__ uint32_t s_kind[kCTile], s_f[kCTile], s_k[kCTile], s_m[kCTile], s_lb[kCTile];
  __shared__ uint32_t s_fo[kCTile], s_lo[kCTile], s_mo[kCTile];
  __shared__ uint64_t s_pre[3];
  __shared__ __attribute__((aligned(16))) uint8_t s_pay[kWaves][4096];  // one staged payload per wave
  const uint32_t tid = threadIdx.x, lane = lane_id(), wave = tid >> 6;
  uint8_t* table = meta + kHeaderBytes;
  uint8_t* mflags = table + (uint64_t)kEntryBytes * num_chunks;
  auto header = [&](uint64_t nflag) {
    put_le(meta + 0, kMagic, 4);
    meta[4] = (uint8_t)kSplitVersion;
    meta[5] = (uint8_t)ws;
    meta[6] = 0;
    meta[7] = 0;
    put_le(meta + 8, cs, 4);
    put_le(meta + 12, num_chunks, 4);
    put_le(meta + 16, n, 8);
    put_le(meta + 24, nflag, 8);
  };
  if (num_chunks == 0) {
    if (tid == 0) {
      header(0);
      port_bytes[0] = port_bytes[1] = port_bytes[2] = 0;
      port_bytes[3] = kHeaderBytes;
    }
    return;
  }
  const uint32_t t = blockIdx.x;
  const uint64_t c0 = (uint64_t)t * kCTile;
  const uint32_t E = cs / ws;
  if (wave == 0) {
    static_assert(kCTile == 64, "one chunk per lane of the first wave");
    const uint64_t c = c0 + lane;
    uint32_t kind = 0, f = 0, K = 0, M = 0, lb = 0;  // kind: 0 zero / none, 1 raw, 2 coded
    uint8_t* row = table + kEntryBytes * c;
    const bool al = (((uintptr_t)table) & 7u) == 0;
    if (c < num_chunks) {
      uint2 e;
      if (al) {
        e = *(const uint2*)row;
      } else {
        e.x = (uint32_t)row[0] | ((uint32_t)row[1] << 8) | ((uint32_t)row[2] << 16) | ((uint32_t)row[3] << 24);
        e.y = (uint32_t)row[4] | ((uint32_t)row[5] << 8) | ((uint32_t)row[6] << 16) | ((uint32_t)row[7] << 24);
      }
      const uint64_t start = c * cs;
      const uint32_t bc = (uint32_t)((n - start) < cs ? (n - start) : cs);
      // sizes never exceed the chunk's, so every write stays inside the ports
      // even if a row were wrong
      if (e.x != 0u) {
        const uint2 q = km[c];
        kind = 2;
        K = q.x < E ? q.x : E;
        M = q.y < K ? q.y : K;
        f = (K + 7u) / 8u;
        lb = ws * (K - M);
      } else if (e.y & kRawBit) {
        kind = 1;
        lb = bc;
      }
    }
    const uint32_t incf = wave_incl_add(f), incl = wave_incl_add(lb), incm = wave_incl_add(M);
    s_kind[lane] = kind;
    s_f[lane] = f;
    s_k[lane] = K;
    s_m[lane] = M;
    s_lb[lane] = lb;
    s_fo[lane] = incf - f;
    s_lo[lane] = incl - lb;
    s_mo[lane] = incm - M;
    const uint64_t tf = lane63(incf), tl = lane63(incl), tm = lane63(incm);
    const uint64_t pf = look_back(tile_flags, t, tf, &ctl->error);
    const uint64_t pl = look_back(tile_flags + num_tiles, t, tl, &ctl->error);
    const uint64_t pm = look_back(tile_flags + 2u * (uint64_t)num_tiles, t, tm, &ctl->error);
    if (kind == 2) {  // the row of a coded chunk becomes {items, matches}
      if (al) {
        *(uint2*)row = make_uint2(K, M);
      } else {
        put_le(row, K, 4);
        put_le(row + 4, M, 4);
      }
    }
    if (lane == 0) {
      s_pre[0] = pf;
      s_pre[1] = pl;
      s_pre[2] = pm;
      if (t == num_tiles - 1u) {
        const uint64_t nf = pf + tf;
        header(nf);
        const bool err = __hip_atomic_load(&ctl->error, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0u;
        port_bytes[0] = err ? 0ull : pl + tl;
        port_bytes[1] = err ? 0ull : pm + tm;
        port_bytes[2] = err ? 0ull : pm + tm;
        port_bytes[3] = err ? 0ull : (uint64_t)kHeaderBytes + (uint64_t)kEntryBytes * num_chunks + nf;
      }
    }
  }
  __syncthreads();
  const uint64_t pf = s_pre[0], pl = s_pre[1], pm = s_pre[2];
  constexpr uint32_t PW = kCTile / kWaves;
  uint8_t* buf = s_pay[wave];
  for (uint32_t u = 0; u < PW; ++u) {
    const uint32_t j = wave * PW + u;
    const uint64_t c = c0 + j;
    if (c >= num_chunks) break;
    const uint32_t kind = s_kind[j];
    const uint8_t* src = staging + c * cs;
    if (kind == 1u) {  // a raw chunk's bytes, straight from the input
      copy_bytes16(lit + pl + s_lo[j], in + c * cs, s_lb[j], lane);
    } else if (kind == 2u) {
      const uint32_t F = s_f[j], K = s_k[j];
      copy_bytes16(mflags + pf + s_fo[j], src, F, lane);
      // the payload (flags, then data) into LDS with 16-byte loads, the
      // items dealt out from there
      const uint32_t nbk = (F + ws * (K - s_m[j]) + 2u * s_m[j] + 15u) / 16u;
      for (uint32_t b0 = 0; b0 < nbk; b0 += 256u) {
        uint4 v[4];
#pragma unroll
        for (uint32_t r = 0; r < 4u; ++r) {
          const uint32_t b = b0 + lane + 64u * r;
          v[r] = b < nbk ? ((const uint4*)src)[b] : make_uint4(0u, 0u, 0u, 0u);
        }
#pragma unroll
        for (uint32_t r = 0; r < 4u; ++r) {
          const uint32_t b = b0 + lane + 64u * r;
          if (b < nbk) ((uint4*)buf)[b] = v[r];
        }
      }
      wave_sync();
      const uint8_t* flg = buf;
      const uint8_t* data = buf + F;
      uint8_t* L = lit + pl + s_lo[j];
      uint8_t* LN = lens + pm + s_mo[j];
      uint8_t* OF = offs + pm + s_mo[j];
      uint32_t mg = 0;  // matches before this group of 64 items
      for (uint32_t k0 = 0; k0 < K; k0 += 64u) {
        const uint32_t k = k0 + lane;
        const bool live = k < K;
        const bool mt = live && ((flg[k >> 3] >> (k & 7u)) & 1u);
        const uint64_t mw = __ballot(mt);
        const uint32_t mb = mg + mbcnt64(mw);  // matches before item k
        if (live) {
          const uint32_t tp = ws * (k - mb) + 2u * mb;  // item k's data offset
          if (mt) {
            LN[mb] = data[tp];
            OF[mb] = data[tp + 1u];
          } else {
            for (uint32_t b = 0; b < ws; ++b) L[ws * (k - mb) + b] = data[tp + b];
          }
        }
        mg += (uint32_t)__builtin_popcountll(mw);
      }
      wave_sync();  // every item read before the next payload lands
    }
  }
}

// Upstream-style baseline search (GPULZStage page, exact longest-match search
// paragraph, which describes upstream's search as one whose candidate pointer
// moves forward with each comparison, so that it ends up with shorter
// matches than the exact search).  Read as: the pointer w walks the
// 32 words before p, one comparison per step of x[w] against x[p + len], the
// word the partial match started at w - len needs next; equal grows it,
// unequal drops it and spends w; the longest partial match seen is the
// result, the first on ties.  Everything else is the level-0 stream.  One
// wave per chunk: each lane searches its positions, lane 0 walks the greedy
// parse and writes the payload into LDS, the wave copies it to the chunk's
// staging slot; compact_kernel then assembles the stream.  A baseline for
// the page's comparison, not a tuned path.
template <int WS, uint32_t CS>
__global__ __launch_bounds__(64) void advancing_encode_kernel(const uint8_t* __restrict__ in, uint64_t n,
                                                              uint32_t num_chunks, uint8_t* __restrict__ out,
                                                              uint8_t* __restrict__ staging,
                                                              uint64_t* __restrict__ tile_flags, uint32_t num_tiles,
                                                              EncCtl* __restrict__ ctl) {
  constexpr uint32_t E = CS / (uint32_t)WS;
  constexpr uint32_t MM = min_match<WS>();
  __shared__ uint32_t X[E];
  __shared__ uint32_t LO[E];
  __shared__ __attribute__((aligned(16))) uint8_t P[CS];  // a coded payload: F + D < CS bytes
  const uint32_t c = blockIdx.x, lane = lane_id();
  const uint64_t base = (uint64_t)c * CS;
  const uint32_t bc = (uint32_t)((n - base) < CS ? (n - base) : CS);
  const uint8_t* src = in + base;
  uint32_t any = 0;
  for (uint32_t i = lane; i < E; i += 64u) {
    uint32_t w = 0;
#pragma unroll
    for (int b = 0; b < WS; ++b) {
      const uint32_t j = i * (uint32_t)WS + (uint32_t)b;
      if (j < bc) w |= (uint32_t)src[j] << (8 * b);
    }
    X[i] = w;
    any |= w;
  }
  const bool nonzero = __ballot(any != 0u) != 0ull;
  wave_sync();
  uint32_t F = 0, D = 0;
  bool raw = false;
  if (nonzero) {
    for (uint32_t p = lane; p < E; p += 64u) {
      uint32_t best = 0, bo = 0, len = 0;
      for (uint32_t w = p < kWindow ? 0u : p - kWindow; w < p; ++w) {
        if (p + len < E && X[w] == X[p + len]) {
          ++len;
          if (len > best) {
            best = len;
            bo = p - (w + 1u - len);  // the match starts at w + 1 - len
          }
        } else {
          len = 0;
        }
      }
      LO[p] = best | (bo << 8);
    }
    wave_sync();
    uint32_t K = 0, M = 0;
    if (lane == 0u) {  // the greedy parse, counting items and matches
      for (uint32_t p = 0; p < E;) {
        const uint32_t L = LO[p] & 0xFFu;
        if (L >= MM) {
          ++M;
          p += L;
        } else {
          ++p;
        }
        ++K;
      }
    }
    K = (uint32_t)__builtin_amdgcn_readfirstlane((int)K);
    M = (uint32_t)__builtin_amdgcn_readfirstlane((int)M);
    F = (K + 7u) / 8u;
    D = (uint32_t)WS * (K - M) + 2u * M;
    raw = F + D >= bc;
    if (!raw) {
      for (uint32_t i = lane; i < (F + 3u) / 4u; i += 64u) ((uint32_t*)P)[i] = 0u;
      wave_sync();
      if (lane == 0u) {  // the same walk, writing flags and data
        uint8_t* d = P + F;
        uint32_t k = 0;
        for (uint32_t p = 0; p < E; ++k) {
          const uint32_t v = LO[p], L = v & 0xFFu;
          if (L >= MM) {
            P[k >> 3] |= (uint8_t)(1u << (k & 7u));
            d[0] = (uint8_t)L;
            d[1] = (uint8_t)(v >> 8);
            d += 2;
            p += L;
          } else {
            const uint32_t x = X[p];
#pragma unroll
            for (int b = 0; b < WS; ++b) d[b] = (uint8_t)(x >> (8 * b));
            d += WS;
            ++p;
          }
        }
      }
      wave_sync();
      uint32_t* slot = (uint32_t*)(staging + base);
      for (uint32_t i = lane; i < (F + D + 3u) / 4u; i += 64u) slot[i] = ((const uint32_t*)P)[i];
    }
  }
  if (lane == 0u) {
    const uint2 ent = !nonzero ? make_uint2(0u, 0u) : (raw ? make_uint2(0u, kRawBit | bc) : make_uint2(F, D));
    uint8_t* row = out + kHeaderBytes + kEntryBytes * (uint64_t)c;
    if ((((uintptr_t)row) & 7u) == 0) {
      *(uint2*)row = ent;
    } else {
      put_le(row, ent.x, 4);
      put_le(row + 4, ent.y, 4);
    }
    // tile flag c of the assembly kernel (never more tiles than chunks), and
    // the error flag
    if (c < num_tiles) tile_flags[c] = 0ull;
    if (c == 0u) ctl->error = 0u;
  }
}

template <int WS, uint32_t CS>
hipError_t launch_advancing(const EncodeArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL((advancing_encode_kernel<WS, CS>), dim3(a.num_chunks), dim3(64), 0, stream, a.in, a.n,
                     a.num_chunks, a.out, a.staging, a.tile_flags, num_tiles_of(a.num_chunks), (EncCtl*)a.ctl);
  return hipGetLastError();
}

template <int WS, int E, int LEVEL, int W>
hipError_t launch_one(const EncodeArgs& a, hipStream_t stream) {
  // waves per chunk: one up to 512 elements (four chunks per workgroup at
  // level 0, two at level 1, whose larger layout would leave fewer waves per
  // CU in four-chunk workgroups), then one per 512 elements, so LDS per wave
  // stays the same and occupancy holds
  constexpr int WPC = E <= 512 ? 1 : E / 512;
  constexpr int CPW = E <= 512 ? (LEVEL == 0 ? 4 : 2) : 1;
  constexpr uint32_t threads = 64u * WPC * CPW;
  const uint32_t grid = (a.num_chunks + CPW - 1) / CPW;  // one chunk per team
  hipLaunchKernelGGL((encode_kernel<WS, E, LEVEL, W, WPC, CPW>), dim3(grid), dim3(threads), 0, stream, a.in, a.n,
                     a.num_chunks, a.out, a.staging, a.tile_flags, num_tiles_of(a.num_chunks),
                     a.km ? 3u : 1u, a.km, (EncCtl*)a.ctl);
  return hipGetLastError();
}

template <int WS, int E, int W>
hipError_t launch_level(const EncodeArgs& a, hipStream_t stream) {
  return a.level ? launch_one<WS, E, 1, W>(a, stream) : launch_one<WS, E, 0, W>(a, stream);
}

template <int WS, int E>
hipError_t launch_window(const EncodeArgs& a, hipStream_t stream) {
  switch (a.window) {
    case 32u: return launch_level<WS, E, 32>(a, stream);
    case 48u: return launch_level<WS, E, 48>(a, stream);
    case 64u: return launch_level<WS, E, 64>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

uint64_t encode_ctl_bytes() { return sizeof(EncCtl); }
uint64_t encode_tiles(uint32_t num_chunks) { return num_tiles_of(num_chunks); }

hipError_t launch_compact(const EncodeArgs& a, hipStream_t stream) {
  // Few tiles (at most two per CU): 16 waves per tile, four chunks each, so
  // the per-chunk placement latency is spread over more waves; otherwise 8.
  const uint32_t tiles = num_tiles_of(a.num_chunks);
  if (tiles <= 512u)
    hipLaunchKernelGGL(compact_kernel<1024>, dim3(tiles ? tiles : 1u), dim3(1024), 0, stream, a.in, a.staging,
                       a.cs, a.ws, a.n, a.num_chunks, tiles, a.out, a.out_bytes, a.tile_flags, (EncCtl*)a.ctl);
  else
    hipLaunchKernelGGL(compact_kernel<512>, dim3(tiles), dim3(512), 0, stream, a.in, a.staging, a.cs, a.ws, a.n,
                       a.num_chunks, tiles, a.out, a.out_bytes, a.tile_flags, (EncCtl*)a.ctl);
  return hipGetLastError();
}

hipError_t launch_split_compact(const EncodeArgs& a, hipStream_t stream) {
  const uint32_t tiles = num_tiles_of(a.num_chunks);
  hipLaunchKernelGGL(split_compact_kernel, dim3(tiles ? tiles : 1u), dim3(kBlock), 0, stream, a.in, a.staging,
                     (const uint2*)a.km, a.cs, a.ws, a.n, a.num_chunks, tiles, a.out, a.lit, a.lens, a.offs,
                     a.port_bytes, a.tile_flags, (EncCtl*)a.ctl);
  return hipGetLastError();
}

hipError_t launch_encode_advancing(const EncodeArgs& a, hipStream_t stream) {
  if (a.num_chunks == 0) return hipSuccess;
  switch (a.cs * 8u + a.ws) {
    case 1024u * 8u + 1u: return launch_advancing<1, 1024>(a, stream);
    case 1024u * 8u + 2u: return launch_advancing<2, 1024>(a, stream);
    case 1024u * 8u + 4u: return launch_advancing<4, 1024>(a, stream);
    case 2048u * 8u + 1u: return launch_advancing<1, 2048>(a, stream);
    case 2048u * 8u + 2u: return launch_advancing<2, 2048>(a, stream);
    case 2048u * 8u + 4u: return launch_advancing<4, 2048>(a, stream);
    case 4096u * 8u + 1u: return launch_advancing<1, 4096>(a, stream);
    case 4096u * 8u + 2u: return launch_advancing<2, 4096>(a, stream);
    case 4096u * 8u + 4u: return launch_advancing<4, 4096>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_encode_chunks(const EncodeArgs& a, hipStream_t stream) {
  if (a.num_chunks == 0) return hipSuccess;
  switch (a.cs * 8u + a.ws) {
    case 1024u * 8u + 1u: return launch_window<1, 1024>(a, stream);
    case 1024u * 8u + 2u: return launch_window<2, 512>(a, stream);
    case 1024u * 8u + 4u: return launch_window<4, 256>(a, stream);
    case 2048u * 8u + 1u: return launch_window<1, 2048>(a, stream);
    case 2048u * 8u + 2u: return launch_window<2, 1024>(a, stream);
    case 2048u * 8u + 4u: return launch_window<4, 512>(a, stream);
    case 4096u * 8u + 1u: return launch_window<1, 4096>(a, stream);
    case 4096u * 8u + 2u: return launch_window<2, 2048>(a, stream);
    case 4096u * 8u + 4u: return launch_window<4, 1024>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace gpulz
