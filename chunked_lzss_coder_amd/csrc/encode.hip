// encode.hip -- chunked LZSS encode for gfx950, one fused pass.
//
// A "team" of WPC wave64s owns one chunk at a time (WPC = 1 for chunks of up
// to 1024 elements, so most of the work needs no workgroup barrier).  Teams
// take chunks in ticket order from an atomic counter and assemble the stream
// themselves: once a chunk's payload size is known it is published and the
// chunk's output offset is found by a decoupled look-back over its
// predecessors' published sizes, so flags and data go straight from LDS to
// their final place in the stream (no staging area, no second pass).
//
// Per chunk (GPULZStage page paragraphs in brackets):
//   1. load the chunk (zero padded past its real bytes) into LDS as E words;
//      all zero -> entry (0,0), no payload [zero-chunk paragraph];
//   2. omask[p], bit o-1 = (x[p] == x[p-o]), o = 1..32 [exact-search
//      paragraph]: each lane holds 8 consecutive positions and the 32 words
//      before them in registers, so the 256 comparisons per lane read LDS once;
//   3. doubling table S_k[p] = AND of omask over [p, p+k), k = 1..128, and a
//      binary descent per position giving the exact longest run L <= 255 of
//      any offset and the smallest offset reaching it [exact-search and
//      long-match paragraphs];
//   4. level 1: 2048-bucket table of position+1 per sub-block, lookups and
//      atomicMax inserts separated by barriers [hashed-table paragraphs];
//   5. greedy parse [provenance paragraph], in parallel: every 8-position
//      segment computes, for each entry position, where the parse leaves the
//      segment and which positions start items; a short chain of hops over
//      segments then fixes the real entry of each segment;
//   6. item counts from popcounts (two item sizes only) -> flag bytes F and
//      data bytes D; raw when F + D >= real bytes [raw-fallback paragraph];
//   7. look-back for the output offset, size-table row, payload bytes.
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

// Decoupled look-back over the chunks' published payload sizes (one wave).
// Each flag is one 64-bit word {state:2, value:62}, written with one atomic
// store, so a reader never sees a state without its value.  Returns the
// exclusive prefix (output offset of chunk c's payload).
__device__ uint64_t look_back(uint64_t* flags, uint32_t c, uint64_t agg, uint32_t* err) {
  const uint32_t lane = lane_id();
  if (c == 0) {
    if (lane == 0) __hip_atomic_store(&flags[0], kFlagIncl | agg, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
    return 0;
  }
  if (lane == 0) __hip_atomic_store(&flags[c], kFlagAgg | agg, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
  uint64_t prefix = 0;
  int64_t j = (int64_t)c - 1;
  uint32_t spins = 0;
  while (true) {
    const int64_t idx = j - (int64_t)lane;
    uint64_t f = kFlagIncl;  // before chunk 0: an inclusive prefix of 0
    if (idx >= 0) f = __hip_atomic_load(&flags[idx], __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_AGENT);
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
    __hip_atomic_store(&flags[c], kFlagIncl | (prefix + agg), __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
  return prefix;
}

// Copy n bytes from an LDS byte buffer (4-aligned) to global dst (any
// alignment): aligned dwords in the middle, single bytes at the two edges.
// `lane` runs over `nl` cooperating lanes.
__device__ __forceinline__ void lds_to_global(uint8_t* dst, const uint8_t* src, uint32_t n, uint32_t lane,
                                              uint32_t nl) {
  uint32_t head = (uint32_t)((4u - ((uintptr_t)dst & 3u)) & 3u);
  if (head > n) head = n;
  if (lane < head) dst[lane] = src[lane];
  const uint32_t nbody = (n - head) >> 2;
  const uint32_t* sw = (const uint32_t*)src;
  uint32_t* dw = (uint32_t*)(dst + head);
  for (uint32_t j = lane; j < nbody; j += nl) {
    const uint32_t s = head + 4u * j;
    const uint32_t lo = sw[s >> 2];
    const uint32_t hi = head ? sw[(s >> 2) + 1u] : 0u;
    dw[j] = __builtin_amdgcn_alignbyte(hi, lo, head);
  }
  const uint32_t t0 = head + 4u * nbody;
  if (t0 + lane < n) dst[t0 + lane] = src[t0 + lane];
}

__device__ __forceinline__ void put_le(uint8_t* p, uint64_t v, int nb) {
  for (int i = 0; i < nb; ++i) p[i] = (uint8_t)(v >> (8 * i));
}

struct EncCtl {
  uint32_t ticket;
  uint32_t error;
  uint32_t pad[62];
};

template <int WS, int E>
struct Lay {
  static constexpr uint32_t CS = (uint32_t)E * WS;
  static constexpr uint32_t NW64 = E / 64;  // 64-position words
  static constexpr uint32_t NSEG = E / 8;   // 8-position parse segments
  // word offsets inside the per-chunk region, after X[E]:
  //   phase A: LV = 8 doubling levels of E words
  //   phase B: LO (E) | XQ (E) | hash table (2048) or
  //            LO (E) | XQ (E) | ISB (E/32) | LMB (E/32) | FLG (E/32) | STG (CS/4 + 4)
  static constexpr uint32_t RB = 2u * E;
  static constexpr uint32_t R =
      (cmax(cmax(8u * E, RB + kHashSize), RB + 3u * (E / 32u) + CS / 4u + 8u) + 3u) & ~3u;
  static constexpr uint32_t MISC = 2u * (E / 64u + 1u) + 8u;
  static constexpr uint32_t TOTAL = (E + R + MISC + 3u) & ~3u;  // words per chunk, 16-byte multiple
};

template <int WS, int E, int LEVEL, int WPC, int CPW>
__global__ __launch_bounds__(64 * WPC * CPW) void encode_kernel(const uint8_t* __restrict__ in, uint64_t n,
                                                                 uint32_t num_chunks, uint8_t* __restrict__ out,
                                                                 uint64_t* __restrict__ out_bytes,
                                                                 uint64_t* __restrict__ flags,
                                                                 EncCtl* __restrict__ ctl) {
  using L = Lay<WS, E>;
  constexpr uint32_t CS = L::CS;
  constexpr uint32_t TL = 64u * WPC;          // lanes per team
  constexpr uint32_t PPL = E / TL;            // positions per lane (strided)
  constexpr uint32_t MM = min_match<WS>();
  static_assert(WPC == 1 || CPW == 1, "a team is one wave or the whole workgroup");
  static_assert(E % (8 * TL) == 0 || E == 256, "omask passes");
  __shared__ __attribute__((aligned(16))) uint32_t lds_all[CPW * L::TOTAL];
  const uint32_t team = threadIdx.x / TL;
  const uint32_t g = threadIdx.x % TL;        // lane within the team
  const uint32_t lane = lane_id();
  uint32_t* X = lds_all + team * L::TOTAL;
  uint32_t* LV = X + E;
  uint32_t* LO = LV;
  uint32_t* XQ = LV + E;
  uint32_t* T = LV + L::RB;
  uint32_t* ISB = LV + L::RB;
  uint32_t* LMB = ISB + E / 32u;
  uint32_t* FLG = LMB + E / 32u;
  uint8_t* STG = (uint8_t*)(FLG + E / 32u);
  uint32_t* MISC = LV + L::R;
  uint32_t* KB = MISC;                        // items before 64-position word w
  uint32_t* MB = MISC + (E / 64u + 1u);       // matches before word w
  uint32_t* SC = MB + (E / 64u + 1u);         // scalars
  const uint64_t* IS64 = (const uint64_t*)ISB;
  const uint64_t* LM64 = (const uint64_t*)LMB;
  uint8_t* table = out + kHeaderBytes;
  uint8_t* payload = table + (uint64_t)kEntryBytes * num_chunks;

  while (true) {
    // ---- ticket -------------------------------------------------------------------
    uint32_t c;
    if (WPC == 1) {
      uint32_t t = 0;
      if (lane == 0) t = atomicAdd(&ctl->ticket, 1u);
      c = __builtin_amdgcn_readfirstlane(t);
    } else {
      if (g == 0) SC[0] = atomicAdd(&ctl->ticket, 1u);
      __syncthreads();
      c = SC[0];
      __syncthreads();
    }
    if (c >= num_chunks) break;
    const uint64_t base = (uint64_t)c * CS;
    const uint32_t bc = (uint32_t)((n - base) < CS ? (n - base) : CS);
    const uint8_t* src = in + base;

    // ---- 1. load + zero vote ---------------------------------------------------------
    uint32_t any = 0;
    if (bc == CS && (((uintptr_t)src) & 15u) == 0) {
      const uint4* s4 = (const uint4*)src;
      for (uint32_t i = g; i < CS / 16u; i += TL) {
        const uint4 v = s4[i];
        any |= v.x | v.y | v.z | v.w;
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
    bool nonzero;
    if (WPC == 1) {
      nonzero = __ballot(any != 0u) != 0ull;
      wave_sync();
    } else {
      nonzero = __syncthreads_or(any != 0u);
    }
    uint32_t K = 0, M = 0;
    if (nonzero) {
    // ---- 2. omask: 8 consecutive positions per lane, window in registers -------------
    {
      constexpr uint32_t PPASS = (E == 256 ? 4u : 8u);  // positions per lane per pass
      constexpr uint32_t NPASS = E / (PPASS * TL);
#pragma unroll 1
      for (uint32_t ps = 0; ps < NPASS; ++ps) {
        const uint32_t p0 = (ps * TL + g) * PPASS;
        uint32_t w[32 + PPASS];
        if (p0 >= 32u) {
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
        uint32_t om[PPASS];
#pragma unroll
        for (uint32_t q = 0; q < PPASS; ++q) {
          const uint32_t v = w[32 + q];
          uint32_t m = 0;
#pragma unroll
          for (uint32_t o = 32; o >= 1; --o) m = m + m + (uint32_t)(w[32 + q - o] == v);
          const uint32_t p = p0 + q;
          om[q] = p >= 32u ? m : (m & ((1u << p) - 1u));
        }
#pragma unroll
        for (uint32_t i = 0; i < PPASS / 4; ++i)
          *(uint4*)(LV + p0 + 4 * i) = make_uint4(om[4 * i], om[4 * i + 1], om[4 * i + 2], om[4 * i + 3]);
      }
    }
    team_sync<WPC>();

    // ---- 3. doubling table + descent ---------------------------------------------------
#pragma unroll
    for (uint32_t lv = 1; lv < 8; ++lv) {
      const uint32_t half = 1u << (lv - 1);
      const uint32_t* prev = LV + (lv - 1) * E;
      uint32_t* cur = LV + lv * E;
#pragma unroll
      for (uint32_t i = 0; i < PPL; ++i) {
        const uint32_t p = g + i * TL;
        cur[p] = (p + half < (uint32_t)E) ? (prev[p] & prev[p + half]) : 0u;
      }
      team_sync<WPC>();
    }
    uint32_t lo[PPL];
#pragma unroll
    for (uint32_t i = 0; i < PPL; ++i) {
      const uint32_t p = g + i * TL;
      uint32_t surv = LV[7 * E + p], Ln = 0;
      if (surv) Ln = 128;
      else surv = ~0u;
#pragma unroll
      for (int lv = 6; lv >= 0; --lv) {
        const uint32_t k = 1u << lv;
        if (p + Ln + k <= (uint32_t)E) {
          const uint32_t t = surv & LV[(uint32_t)lv * E + p + Ln];
          if (t) {
            surv = t;
            Ln += k;
          }
        }
      }
      lo[i] = Ln ? (Ln | (((uint32_t)__builtin_ctz(surv) + 1u) << 8)) : 0u;
    }
    team_sync<WPC>();
#pragma unroll
    for (uint32_t i = 0; i < PPL; ++i) LO[g + i * TL] = lo[i];
    team_sync<WPC>();

    // ---- 4. level 1 ----------------------------------------------------------------------
    if (LEVEL == 1) {
      for (uint32_t i = g; i < kHashSize; i += TL) T[i] = 0u;
      team_sync<WPC>();  // T overlays dead doubling levels
      constexpr uint32_t SB = E / kSubBlocks;
#pragma unroll 1
      for (uint32_t s = 0; s < kSubBlocks; ++s) {
        for (uint32_t p = s * SB + g; p < (s + 1) * SB; p += TL) {
          if (p + 1 >= (uint32_t)E) continue;
          const uint32_t v = T[bucket_of(X[p], X[p + 1])];
          if (v == 0) continue;
          const uint32_t o = p - (v - 1u);  // entries come from earlier sub-blocks: o >= 1
          if (o > kMaxFar) continue;
          const uint32_t Lnear = LO[p] & 0xFFu;
          if (Lnear >= kMaxLen) continue;
          uint32_t r = 0;
          while (r < kMaxLen && p + r < (uint32_t)E && X[p + r] == X[p + r - o]) ++r;
          if (r > Lnear) LO[p] = r | (o << 8);
        }
        team_sync<WPC>();
        for (uint32_t p = s * SB + g; p < (s + 1) * SB; p += TL)
          if (p + 1 < (uint32_t)E) atomicMax(&T[bucket_of(X[p], X[p + 1])], p + 1u);
        team_sync<WPC>();
      }
    }

    // ---- 5. parallel greedy parse --------------------------------------------------------
    // (a) per segment of 8 positions: for every entry q, the exit position and
    //     the item-start mask of the parse walked from q.
    for (uint32_t sg = g; sg < L::NSEG; sg += TL) {
      const uint32_t p0 = sg * 8u;
      const uint4 a = *(const uint4*)(LO + p0);
      const uint4 b = *(const uint4*)(LO + p0 + 4);
      const uint32_t l8[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
      uint32_t ex[8], im[8], lmb = 0;
#pragma unroll
      for (int q = 7; q >= 0; --q) {
        const uint32_t len = l8[q] & 0xFFu;
        const bool mt = len >= MM;
        lmb |= (mt ? 1u : 0u) << q;
        const uint32_t nq = (uint32_t)q + (mt ? len : 1u);
        uint32_t e = p0 + nq, m = 1u << q;
#pragma unroll
        for (int r = q + 1; r < 8; ++r)
          if (nq == (uint32_t)r) {
            e = ex[r];
            m = (1u << q) | im[r];
          }
        ex[q] = e;
        im[q] = m;
      }
      *(uint4*)(XQ + p0) = make_uint4(ex[0] | (im[0] << 16), ex[1] | (im[1] << 16), ex[2] | (im[2] << 16),
                                      ex[3] | (im[3] << 16));
      *(uint4*)(XQ + p0 + 4) = make_uint4(ex[4] | (im[4] << 16), ex[5] | (im[5] << 16),
                                          ex[6] | (im[6] << 16), ex[7] | (im[7] << 16));
      ((uint8_t*)LMB)[sg] = (uint8_t)lmb;
      ((uint8_t*)ISB)[sg] = 0;
    }
    team_sync<WPC>();
    // (b) hop chain: the real entry of every segment the parse passes through
    if (g == 0) {
      uint32_t P = 0;
      while (P < (uint32_t)E) {
        const uint32_t xq = XQ[P];
        ((uint8_t*)ISB)[P >> 3] = (uint8_t)(xq >> 16);
        P = xq & 0xFFFFu;
      }
    }
    team_sync<WPC>();

    // ---- 6. counts, payload size ------------------------------------------------------------
    if (g < 64u) {
      uint32_t kc = 0, mc = 0;
      if (g < L::NW64) {
        const uint64_t is = IS64[g];
        kc = __builtin_popcountll(is);
        mc = __builtin_popcountll(is & LM64[g]);
      }
      uint32_t ki = kc, mi = mc;
#pragma unroll
      for (int d = 1; d < 64; d <<= 1) {
        const uint32_t a = __shfl_up(ki, d, 64), b = __shfl_up(mi, d, 64);
        if (lane >= (uint32_t)d) {
          ki += a;
          mi += b;
        }
      }
      if (g < L::NW64) {
        KB[g] = ki - kc;
        MB[g] = mi - mc;
      }
      if (g == L::NW64 - 1u) {
        SC[1] = ki;
        SC[2] = mi;
      }
    }
    team_sync<WPC>();
    K = SC[1];
    M = SC[2];
    }  // nonzero
    const uint32_t F = (K + 7u) / 8u;
    const uint32_t D = (uint32_t)WS * (K - M) + 2u * M;
    const bool raw = nonzero && F + D >= bc;
    const uint32_t size = !nonzero ? 0u : (raw ? bc : F + D);

    // ---- 7. offset, entry, payload ----------------------------------------------------------
    if (g < 64u) {
      const uint64_t pre = look_back(flags, c, size, &ctl->error);
      if (g == 0) {
        SC[4] = (uint32_t)pre;
        SC[5] = (uint32_t)(pre >> 32);
        const uint2 ent = !nonzero ? make_uint2(0u, 0u) : (raw ? make_uint2(0u, kRawBit | bc) : make_uint2(F, D));
        uint8_t* row = table + kEntryBytes * (uint64_t)c;
        if ((((uintptr_t)row) & 7u) == 0) {
          *(uint2*)row = ent;
        } else {
          put_le(row, ent.x, 4);
          put_le(row + 4, ent.y, 4);
        }
        if (c == num_chunks - 1u) {
          const uint64_t pb = pre + size;
          put_le(out + 0, kMagic, 4);
          out[4] = (uint8_t)kVersion;
          out[5] = (uint8_t)WS;
          out[6] = 0;
          out[7] = 0;
          put_le(out + 8, CS, 4);
          put_le(out + 12, num_chunks, 4);
          put_le(out + 16, n, 8);
          put_le(out + 24, pb, 8);
          *out_bytes = __hip_atomic_load(&ctl->error, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                           ? 0ull
                           : (uint64_t)kHeaderBytes + (uint64_t)kEntryBytes * num_chunks + pb;
        }
      }
    }
    if (nonzero && !raw) {
      for (uint32_t i = g; i < E / 32u; i += TL) FLG[i] = 0u;
    }
    team_sync<WPC>();
    const uint64_t pre = (uint64_t)SC[4] | ((uint64_t)SC[5] << 32);
    uint8_t* dst = payload + pre;
    if (raw) {
      // the real bytes, read back from the LDS copy of the chunk
      if (WS == 4) {
        lds_to_global(dst, (const uint8_t*)X, bc, g, TL);
      } else {
        uint8_t* xb = STG;  // repack the words as bytes first
        for (uint32_t i = g; i < CS / 4u; i += TL) {
          uint32_t v;
          if (WS == 2) v = X[2 * i] | (X[2 * i + 1] << 16);
          else v = X[4 * i] | (X[4 * i + 1] << 8) | (X[4 * i + 2] << 16) | (X[4 * i + 3] << 24);
          ((uint32_t*)xb)[i] = v;
        }
        team_sync<WPC>();
        lds_to_global(dst, xb, bc, g, TL);
      }
    } else if (nonzero) {
#pragma unroll
      for (uint32_t i = 0; i < PPL; ++i) {
        const uint32_t p = g + i * TL;
        const uint32_t wi = p >> 6;
        const uint64_t is = IS64[wi];
        const uint64_t ms = is & LM64[wi];
        const uint64_t bit = 1ull << (p & 63u);
        if (!(is & bit)) continue;
        const uint64_t below = bit - 1ull;
        const uint32_t k = KB[wi] + (uint32_t)__builtin_popcountll(is & below);
        const uint32_t m = MB[wi] + (uint32_t)__builtin_popcountll(ms & below);
        const uint32_t off = (uint32_t)WS * (k - m) + 2u * m;
        if (ms & bit) {
          const uint32_t v = LO[p];
          STG[off] = (uint8_t)v;
          STG[off + 1] = (uint8_t)(v >> 8);
          atomicOr(&FLG[k >> 5], 1u << (k & 31u));
        } else {
          const uint32_t v = X[p];
#pragma unroll
          for (int b = 0; b < WS; ++b) STG[off + b] = (uint8_t)(v >> (8 * b));
        }
      }
      team_sync<WPC>();
      lds_to_global(dst, (const uint8_t*)FLG, F, g, TL);
      lds_to_global(dst + F, STG, D, g, TL);
    }
    team_sync<WPC>();  // LDS is reused by the next chunk
  }
}

__global__ void encode_init_kernel(uint64_t* __restrict__ flags, uint32_t num_chunks, EncCtl* __restrict__ ctl,
                                   uint8_t* __restrict__ out, uint64_t* __restrict__ out_bytes, uint64_t n,
                                   uint32_t cs, uint32_t ws) {
  const uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < num_chunks) flags[i] = 0ull;
  if (i == 0) {
    ctl->ticket = 0u;
    ctl->error = 0u;
    if (num_chunks == 0) {  // empty input: the header is the whole stream
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
  }
}

template <int WS, int E, int LEVEL>
hipError_t launch_one(const EncodeArgs& a, hipStream_t stream) {
  constexpr int WPC = E <= 1024 ? 1 : E / 1024;
  constexpr int CPW = E <= 512 ? 4 : (E <= 1024 ? 2 : 1);
  constexpr uint32_t threads = 64u * WPC * CPW;
  const uint32_t want = (a.num_chunks + CPW - 1) / CPW;
  const uint32_t grid = want < kMaxGrid ? want : kMaxGrid;
  hipLaunchKernelGGL((encode_kernel<WS, E, LEVEL, WPC, CPW>), dim3(grid), dim3(threads), 0, stream, a.in, a.n,
                     a.num_chunks, a.out, a.out_bytes, a.flags, (EncCtl*)a.ctl);
  return hipGetLastError();
}

template <int WS, int E>
hipError_t launch_level(const EncodeArgs& a, hipStream_t stream) {
  return a.level ? launch_one<WS, E, 1>(a, stream) : launch_one<WS, E, 0>(a, stream);
}

}  // namespace

uint64_t encode_ctl_bytes() { return sizeof(EncCtl); }

hipError_t launch_encode_init(const EncodeArgs& a, hipStream_t stream) {
  const uint32_t per = 256;
  const uint32_t blocks = a.num_chunks == 0 ? 1u : (a.num_chunks + per - 1) / per;
  hipLaunchKernelGGL(encode_init_kernel, dim3(blocks), dim3(per), 0, stream, a.flags, a.num_chunks,
                     (EncCtl*)a.ctl, a.out, a.out_bytes, a.n, a.cs, a.ws);
  return hipGetLastError();
}

hipError_t launch_encode_chunks(const EncodeArgs& a, hipStream_t stream) {
  if (a.num_chunks == 0) return hipSuccess;
  switch (a.cs * 8u + a.ws) {
    case 1024u * 8u + 1u: return launch_level<1, 1024>(a, stream);
    case 1024u * 8u + 2u: return launch_level<2, 512>(a, stream);
    case 1024u * 8u + 4u: return launch_level<4, 256>(a, stream);
    case 2048u * 8u + 1u: return launch_level<1, 2048>(a, stream);
    case 2048u * 8u + 2u: return launch_level<2, 1024>(a, stream);
    case 2048u * 8u + 4u: return launch_level<4, 512>(a, stream);
    case 4096u * 8u + 1u: return launch_level<1, 4096>(a, stream);
    case 4096u * 8u + 2u: return launch_level<2, 2048>(a, stream);
    case 4096u * 8u + 4u: return launch_level<4, 1024>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace gpulz
