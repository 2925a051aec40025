// encode.hip -- per-chunk LZSS encode for gfx950.
//
// One workgroup (4 x wave64) encodes one chunk at a time; the chunk lives in
// LDS for the whole encode (GPULZStage page, chunk-residency paragraph).
// Steps, each separated by a workgroup barrier:
//   1. load cs bytes (zero padded past the real bytes) as E words; vote on
//      "all zero" (zero-chunk paragraph) -> entry (0,0), nothing else;
//   2. omask[p]: bit o-1 set iff x[p] == x[p-o], o = 1..32 (exact-search
//      paragraph);
//   3. a doubling table S_k[p] = AND of omask over [p, p+k), k = 1..128, and a
//      binary descent over it giving, at every p, the longest run L <= 255
//      (long-match paragraph) reached by any offset and the smallest offset
//      reaching it.  This is the page's "AND successive masks until empty",
//      done in 8 table steps per position instead of L+1 dependent steps;
//   4. level 1: 2048-bucket table of position+1 keyed on the two-word hash,
//      walked in 8 sub-blocks with lookups and atomicMax inserts separated by
//      barriers (hashed-table paragraphs); a verified candidate replaces the
//      near match only when strictly longer;
//   5. the sequential greedy parse (provenance paragraph: literal unless the
//      match pays for its token);
//   6. item byte offsets from popcounts of the item/match bitmaps (only two
//      item sizes exist, so the per-item scan reduces to two prefix counts);
//   7. flags + data staged in LDS, raw fallback when not smaller than the
//      real bytes (raw-fallback paragraph), coalesced dword stores to the
//      fixed-stride staging area and the chunk's size-table entry.
#include "common.h"

namespace gpulz {
namespace {

template <int WS>
constexpr uint32_t min_match() {
  // a match is taken only when it is shorter than the literals it replaces
  return WS >= 4 ? 1u : (WS == 2 ? 2u : 3u);
}

constexpr uint32_t cmax(uint32_t a, uint32_t b) { return a > b ? a : b; }

template <int WS, int E>
struct EncLayout {
  static constexpr uint32_t CS = (uint32_t)E * WS;
  static constexpr uint32_t W32 = E / 32;  // words of a per-position bitmap
  // region after x: doubling table (8E words) reused, in turn, for
  //   LO[E] + hash table[2048], then LO[E] + bitmaps + output staging (CS bytes)
  static constexpr uint32_t R =
      cmax(cmax(8u * E, (uint32_t)E + kHashSize), (uint32_t)E + 5u * W32 + CS / 4u + 4u);
  static constexpr uint32_t MISC = 8;
  static constexpr uint32_t TOTAL = E + R + MISC;
};

template <int WS, int E, int LEVEL>
__global__ __launch_bounds__(kBlock) void encode_chunks_kernel(const uint8_t* __restrict__ in, uint64_t n,
                                                               uint32_t num_chunks,
                                                               uint8_t* __restrict__ staging,
                                                               uint2* __restrict__ entries) {
  using Lay = EncLayout<WS, E>;
  constexpr uint32_t CS = Lay::CS;
  constexpr uint32_t W32 = Lay::W32;
  constexpr uint32_t PER = (E + kBlock - 1) / kBlock;  // positions per thread
  __shared__ uint32_t lds[Lay::TOTAL];
  uint32_t* X = lds;                   // chunk words
  uint32_t* LV = lds + E;              // doubling table / reuse
  uint32_t* MISC = lds + E + Lay::R;   // counters
  uint32_t* LO = LV;                   // after step 3: L | O<<8 per position
  const uint32_t tid = threadIdx.x;

  for (uint32_t c = blockIdx.x; c < num_chunks; c += gridDim.x) {
    const uint64_t base = (uint64_t)c * CS;
    const uint32_t bc = (uint32_t)((n - base) < CS ? (n - base) : CS);
    const uint8_t* src = in + base;

    // ---- 1. load + zero vote ------------------------------------------------
    uint32_t any = 0;
    if (bc == CS && (((uintptr_t)src) & 15u) == 0) {
      const uint4* s4 = (const uint4*)src;
      for (uint32_t i = tid; i < CS / 16u; i += kBlock) {
        uint4 v = s4[i];
        any |= v.x | v.y | v.z | v.w;
        uint32_t w[4] = {v.x, v.y, v.z, v.w};
        if (WS == 4) {
#pragma unroll
          for (int j = 0; j < 4; ++j) X[4 * i + j] = w[j];
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
      for (uint32_t i = tid; i < (uint32_t)E; i += kBlock) {
        uint32_t w = 0;
#pragma unroll
        for (int b = 0; b < WS; ++b) {
          uint32_t j = i * WS + b;
          if (j < bc) w |= (uint32_t)src[j] << (8 * b);
        }
        X[i] = w;
        any |= w;
      }
    }
    if (!__syncthreads_or(any != 0)) {
      if (tid == 0) entries[c] = make_uint2(0u, 0u);
      continue;  // nothing reads LDS after the vote barrier
    }

    // ---- 2. omask -------------------------------------------------------------
    for (uint32_t p = tid; p < (uint32_t)E; p += kBlock) {
      const uint32_t v = X[p];
      uint32_t m = 0;
      if (p >= kWindow) {
#pragma unroll
        for (uint32_t o = 1; o <= kWindow; ++o) m |= (X[p - o] == v ? 1u : 0u) << (o - 1);
      } else {
        for (uint32_t o = 1; o <= p; ++o) m |= (X[p - o] == v ? 1u : 0u) << (o - 1);
      }
      LV[p] = m;
    }
    __syncthreads();

    // ---- 3. doubling table and descent -------------------------------------------
#pragma unroll
    for (int lv = 1; lv < 8; ++lv) {
      const uint32_t half = 1u << (lv - 1);
      const uint32_t* prev = LV + (uint32_t)(lv - 1) * E;
      uint32_t* cur = LV + (uint32_t)lv * E;
      for (uint32_t p = tid; p < (uint32_t)E; p += kBlock)
        cur[p] = (p + half < (uint32_t)E) ? (prev[p] & prev[p + half]) : 0u;
      __syncthreads();
    }
    uint32_t lo[PER];
#pragma unroll
    for (uint32_t i = 0; i < PER; ++i) {
      const uint32_t p = tid + i * kBlock;
      uint32_t surv = ~0u, L = 0;
      if (p < (uint32_t)E) {
#pragma unroll
        for (int lv = 7; lv >= 0; --lv) {
          const uint32_t k = 1u << lv;
          if (p + L + k <= (uint32_t)E) {
            const uint32_t t = surv & LV[(uint32_t)lv * E + p + L];
            if (t) {
              surv = t;
              L += k;
            }
          }
        }
      }
      lo[i] = L ? (L | ((uint32_t)__builtin_ctz(surv) + 1u) << 8) : 0u;
    }
    __syncthreads();
#pragma unroll
    for (uint32_t i = 0; i < PER; ++i) {
      const uint32_t p = tid + i * kBlock;
      if (p < (uint32_t)E) LO[p] = lo[i];
    }

    // ---- 4. level-1 hashed long-range candidates ----------------------------------
    if (LEVEL == 1) {
      uint32_t* T = LV + E;
      for (uint32_t i = tid; i < kHashSize; i += kBlock) T[i] = 0u;
      __syncthreads();
      constexpr uint32_t SB = E / kSubBlocks;
      for (uint32_t s = 0; s < kSubBlocks; ++s) {
        for (uint32_t p = s * SB + tid; p < (s + 1) * SB; p += kBlock) {
          if (p + 1 >= (uint32_t)E) continue;
          const uint32_t v = T[bucket_of(X[p], X[p + 1])];
          if (v == 0) continue;
          const uint32_t o = p - (v - 1u);  // v-1 < s*SB <= p, so o >= 1
          if (o > kMaxFar) continue;
          const uint32_t Ln = LO[p] & 0xFFu;
          uint32_t r = 0;
          while (r < kMaxLen && p + r < (uint32_t)E && X[p + r] == X[p + r - o]) ++r;
          if (r > Ln) LO[p] = r | (o << 8);
        }
        __syncthreads();
        for (uint32_t p = s * SB + tid; p < (s + 1) * SB; p += kBlock)
          if (p + 1 < (uint32_t)E) atomicMax(&T[bucket_of(X[p], X[p + 1])], p + 1u);
        __syncthreads();
      }
    } else {
      __syncthreads();
    }

    // ---- 5. greedy parse ----------------------------------------------------------
    uint32_t* IS = LV + E;       // item starts
    uint32_t* MS = IS + W32;     // match starts
    uint32_t* LM = MS + W32;     // positions whose match pays
    uint32_t* PK = LM + W32;     // items before word w
    uint32_t* PM = PK + W32;     // matches before word w
    uint8_t* STG = (uint8_t*)(PM + W32);
    constexpr uint32_t MM = min_match<WS>();
#pragma unroll
    for (uint32_t i = 0; i < PER; ++i) {
      const uint32_t p = tid + i * kBlock;
      const bool lm = p < (uint32_t)E && (LO[p] & 0xFFu) >= MM;
      const uint64_t b = __ballot(lm);
      if ((tid & 63u) == 0 && p < (uint32_t)E) {
        LM[p >> 5] = (uint32_t)b;
        if ((p >> 5) + 1 < W32) LM[(p >> 5) + 1] = (uint32_t)(b >> 32);
      }
    }
    for (uint32_t w = tid; w < W32; w += kBlock) {
      IS[w] = 0u;
      MS[w] = 0u;
    }
    __syncthreads();
    if (tid == 0) {
      uint32_t p = 0, K = 0, M = 0;
      while (p < (uint32_t)E) {
        // next position q >= p where a match pays; [p, q) are literals
        uint32_t w = p >> 5;
        uint32_t bits = LM[w] & (~0u << (p & 31u));
        while (bits == 0u && ++w < W32) bits = LM[w];
        const uint32_t q = (w < W32) ? (w * 32u + (uint32_t)__builtin_ctz(bits)) : (uint32_t)E;
        for (uint32_t a = p; a < q;) {
          const uint32_t ww = a >> 5, lo_b = a & 31u;
          const uint32_t hi_b = (q - ww * 32u) < 32u ? (q - ww * 32u) : 32u;
          const uint32_t mask = (hi_b == 32u ? ~0u : ((1u << hi_b) - 1u)) & (~0u << lo_b);
          IS[ww] |= mask;
          a = ww * 32u + hi_b;
        }
        K += q - p;
        if (q >= (uint32_t)E) break;
        const uint32_t L = LO[q] & 0xFFu;
        IS[q >> 5] |= 1u << (q & 31u);
        MS[q >> 5] |= 1u << (q & 31u);
        ++K;
        ++M;
        p = q + L;
      }
      uint32_t ak = 0, am = 0;
      for (uint32_t ww = 0; ww < W32; ++ww) {
        PK[ww] = ak;
        PM[ww] = am;
        ak += __builtin_popcount(IS[ww]);
        am += __builtin_popcount(MS[ww]);
      }
      MISC[0] = K;
      MISC[1] = M;
    }
    __syncthreads();

    // ---- 6./7. serialize ------------------------------------------------------------
    const uint32_t K = MISC[0], M = MISC[1];
    const uint32_t F = (K + 7u) / 8u;
    const uint32_t D = (uint32_t)WS * (K - M) + 2u * M;
    uint32_t* gdst = (uint32_t*)(staging + (uint64_t)c * CS);
    if (F + D >= bc) {
      // raw fallback: the padded chunk as bytes (the compaction copies bc of them)
      for (uint32_t i = tid; i < CS / 4u; i += kBlock) {
        uint32_t v;
        if (WS == 4) v = X[i];
        else if (WS == 2) v = X[2 * i] | (X[2 * i + 1] << 16);
        else v = X[4 * i] | (X[4 * i + 1] << 8) | (X[4 * i + 2] << 16) | (X[4 * i + 3] << 24);
        gdst[i] = v;
      }
      if (tid == 0) entries[c] = make_uint2(0u, kRawBit | bc);
    } else {
      uint32_t* STG32 = (uint32_t*)STG;
      for (uint32_t i = tid; i < CS / 4u; i += kBlock) STG32[i] = 0u;
      __syncthreads();
      // flags first (bit k of the bitmap = item k is a match)
#pragma unroll
      for (uint32_t i = 0; i < PER; ++i) {
        const uint32_t p = tid + i * kBlock;
        if (p >= (uint32_t)E) continue;
        const uint32_t w = p >> 5, bit = 1u << (p & 31u), below = bit - 1u;
        if (MS[w] & bit) {
          const uint32_t k = PK[w] + (uint32_t)__builtin_popcount(IS[w] & below);
          atomicOr(&STG32[k >> 5], 1u << (k & 31u));
        }
      }
      __syncthreads();
#pragma unroll
      for (uint32_t i = 0; i < PER; ++i) {
        const uint32_t p = tid + i * kBlock;
        if (p >= (uint32_t)E) continue;
        const uint32_t w = p >> 5, bit = 1u << (p & 31u), below = bit - 1u;
        if (!(IS[w] & bit)) continue;
        const uint32_t k = PK[w] + (uint32_t)__builtin_popcount(IS[w] & below);
        const uint32_t m = PM[w] + (uint32_t)__builtin_popcount(MS[w] & below);
        const uint32_t off = F + (uint32_t)WS * (k - m) + 2u * m;
        if (MS[w] & bit) {
          const uint32_t v = LO[p];
          STG[off] = (uint8_t)(v & 0xFFu);
          STG[off + 1] = (uint8_t)(v >> 8);
        } else {
          const uint32_t v = X[p];
#pragma unroll
          for (int b = 0; b < WS; ++b) STG[off + b] = (uint8_t)(v >> (8 * b));
        }
      }
      __syncthreads();
      for (uint32_t i = tid; i < (F + D + 3u) / 4u; i += kBlock) gdst[i] = STG32[i];
      if (tid == 0) entries[c] = make_uint2(F, D);
    }
    __syncthreads();  // LDS is reused by the next chunk
  }
}

template <int WS, int E, int LEVEL>
hipError_t launch_one(const EncodeArgs& a, hipStream_t stream) {
  const uint32_t grid = a.num_chunks < kMaxGrid ? a.num_chunks : kMaxGrid;
  hipLaunchKernelGGL((encode_chunks_kernel<WS, E, LEVEL>), dim3(grid), dim3(kBlock), 0, stream, a.in, a.n,
                     a.num_chunks, a.staging, a.entries);
  return hipGetLastError();
}

template <int WS, int E>
hipError_t launch_level(const EncodeArgs& a, hipStream_t stream) {
  return a.level ? launch_one<WS, E, 1>(a, stream) : launch_one<WS, E, 0>(a, stream);
}

}  // namespace

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
