/*
 * gpulz_oracle.c -- plain, single-threaded CPU reference of the chunked LZSS
 * coder described on the FZGPUModules "fz::GPULZStage" page (stage_gpulz).
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the oracle that the HIP path is
 * checked against.  Only the test suite, the package smoke check and the
 * benchmark's CPU-baseline leg may load it.  It shares no code, header,
 * table or constant generator with the HIP library: every format constant
 * below is restated here from the stream-format rules, not included.
 *
 * It is written for obviousness, not speed: the match search is the plain
 * definition (a loop over every offset and every following element), the
 * level-1 table is the step-by-step sub-block walk, and the parse is the
 * sequential greedy walk.
 *
 * Citations name the GPULZStage page and the paragraph on it ("level table",
 * "exact longest-match search", ...) or the FZGPUModules codebase notes page
 * and its note id (CN-GPULZ-1).  Where the pages are silent the reading used
 * is stated in place and listed with the other readings in the design notes.
 *
 * Parity pins: every function here is pinned by the CPU tests (hand-worked
 * streams, brute-force longest match on tiny inputs, an independent
 * omask-AND search, round trips, an independent Python stream walker, an
 * independent level-1 table simulation, corrupted-stream rejection; the
 * upstream-style advancing search by hand-worked matches, a closed form on
 * constant chunks and a hand-built stream).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ---- stream-format constants (restated, not shared) ------------------- */
#define OR_MAGIC 0x315A4C47u /* bytes 'G','L','Z','1' little-endian        */
#define OR_VERSION 1u
#define OR_HEADER_BYTES 32u
#define OR_ENTRY_BYTES 8u
#define OR_RAW_BIT 0x80000000u
#define OR_WINDOW 32u       /* near window, fixed (page: window paragraph)  */
#define OR_MAX_LEN 255u     /* one-byte length field (page: long matches)   */
#define OR_MAX_FAR 255u     /* one-byte offset field, level-1 reach         */
#define OR_SUBBLOCKS 8u     /* level-1 sub-block walk (page: hashed table)  */
#define OR_HASH_BITS 11u
#define OR_HASH_SIZE (1u << OR_HASH_BITS)

/* Status codes, shared meaning with the library's but declared separately. */
#define OR_OK 0
#define OR_EINVAL -1
#define OR_ECAP -2
#define OR_ECORRUPT -3

static int cs_ok(uint32_t cs) { return cs == 1024u || cs == 2048u || cs == 4096u; }
static int ws_ok(uint32_t ws) { return ws == 1u || ws == 2u || ws == 4u; }

static void put_u32(uint8_t* p, uint32_t v) {
  p[0] = (uint8_t)v; p[1] = (uint8_t)(v >> 8); p[2] = (uint8_t)(v >> 16); p[3] = (uint8_t)(v >> 24);
}
static void put_u64(uint8_t* p, uint64_t v) {
  for (int i = 0; i < 8; ++i) p[i] = (uint8_t)(v >> (8 * i));
}
static uint32_t get_u32(const uint8_t* p) {
  return (uint32_t)p[0] | ((uint32_t)p[1] << 8) | ((uint32_t)p[2] << 16) | ((uint32_t)p[3] << 24);
}
static uint64_t get_u64(const uint8_t* p) {
  uint64_t v = 0;
  for (int i = 7; i >= 0; --i) v = (v << 8) | p[i];
  return v;
}

/* Little-endian word of ws bytes, zero-extended to 32 bits. */
static uint32_t load_word(const uint8_t* p, uint32_t ws) {
  uint32_t v = 0;
  for (uint32_t b = 0; b < ws; ++b) v |= (uint32_t)p[b] << (8 * b);
  return v;
}

/* Worst-case stream size: header + one entry per chunk + every input byte
 * (raw fallback bounds each chunk by its own size; page: raw-fallback
 * paragraph). */
uint64_t oracle_max_stream_size(uint64_t n, uint32_t cs) {
  if (!cs_ok(cs)) return 0;
  uint64_t chunks = (n + cs - 1) / cs;
  return OR_HEADER_BYTES + OR_ENTRY_BYTES * chunks + n;
}

/* Level-1 bucket of a two-word key (CN-GPULZ-1: hashed two-word key; the
 * pages give no hash, so a fixed Fibonacci multiplicative hash of the 64-bit
 * key w0 | w1<<32 is used, top 11 bits kept). */
uint32_t oracle_hash(uint32_t w0, uint32_t w1) {
  uint64_t key = (uint64_t)w0 | ((uint64_t)w1 << 32);
  return (uint32_t)((key * 0x9E3779B97F4A7C15ull) >> (64u - OR_HASH_BITS));
}

/* Length of the run of equal elements at distance o starting at p,
 * stopping at the chunk end and at the 255 cap (page: long matches). */
static uint32_t run_at(const uint32_t* x, uint32_t E, uint32_t p, uint32_t o) {
  uint32_t k = 0;
  while (k < OR_MAX_LEN && p + k < E && x[p + k] == x[p + k - o]) ++k;
  return k;
}

/* Near windows the encoder accepts: the fixed 32 of the stage, and the 48
 * and 64 the page measured (window-width paragraph: ratio 4.36x at 32,
 * 4.82x at 48, 5.13x at 64).  The window is an encode-side choice only:
 * offsets up to 64 fit the token's offset byte, the stream is unchanged. */
static int window_ok(uint32_t w) { return w == 32u || w == 48u || w == 64u; }

/* Exact longest match over a near window of `window` offsets at position p
 * (page: exact longest-match search; offsets 1..window, never before the
 * chunk start).  Ties on length go to the smallest offset.  L = 0 means no
 * offset matches. */
void oracle_near_match_w(const uint32_t* x, uint32_t E, uint32_t p, uint32_t window, uint32_t* L, uint32_t* O) {
  uint32_t bestL = 0, bestO = 0;
  uint32_t omax = p < window ? p : window;
  for (uint32_t o = 1; o <= omax; ++o) {
    uint32_t k = run_at(x, E, p, o);
    if (k > bestL) { bestL = k; bestO = o; }
  }
  *L = bestL;
  *O = bestO;
}

/* The stage's own near window: offsets 1..32 (page: window paragraph). */
void oracle_near_match(const uint32_t* x, uint32_t E, uint32_t p, uint32_t* L, uint32_t* O) {
  oracle_near_match_w(x, E, p, OR_WINDOW, L, O);
}

/* The upstream-style search the page contrasts with its own (exact
 * longest-match search paragraph): the window pointer advances on every
 * step, so a match being extended carries the pointer with it and the
 * candidate starts it passes over are never tried.  The page gives no more
 * than that; the reading here: the pointer w walks the 32 elements before p
 * (never before the chunk start), one comparison per step, of x[w] against
 * the element the current partial match needs next, x[p + len].  Equal:
 * the partial match (starting at w - len) grows by one; unequal: it is
 * dropped and this w is spent.  The longest partial match seen is the
 * result (the first one on ties); it never reaches past p - 1 as a source,
 * so L <= 32, and never past the chunk end.  L = 0: nothing matched. */
void oracle_advancing_match(const uint32_t* x, uint32_t E, uint32_t p, uint32_t* L, uint32_t* O) {
  uint32_t best = 0, bestO = 0, len = 0;
  uint32_t w = p < OR_WINDOW ? 0u : p - OR_WINDOW;
  for (; w < p; ++w) {
    if (p + len < E && x[w] == x[p + len]) {
      len += 1;
      if (len > best) {
        best = len;
        bestO = p - (w + 1u - len); /* the match starts at w + 1 - len */
      }
    } else {
      len = 0;
    }
  }
  *L = best;
  *O = bestO;
}

/* Level-1 candidates for every position of one chunk (page: hashed
 * long-range paragraph; sub-block walk and atomicMax(position+1) insert).
 * Table entries hold position+1, 0 = empty.  For sub-block s, every
 * position p <= E-2 in it first looks its key up in the table as it stood
 * after sub-blocks 0..s-1, then every such position inserts p+1 with max.
 * cand[p] = p - (entry-1) when that distance is 1..255, else 0.
 * If table_out is not NULL the final table is copied there. */
void oracle_level1_candidates(const uint32_t* x, uint32_t E, uint32_t* cand, uint32_t* table_out) {
  uint32_t* T = (uint32_t*)calloc(OR_HASH_SIZE, sizeof(uint32_t));
  uint32_t sub = E / OR_SUBBLOCKS;
  for (uint32_t p = 0; p < E; ++p) cand[p] = 0;
  for (uint32_t s = 0; s < OR_SUBBLOCKS; ++s) {
    uint32_t lo = s * sub, hi = lo + sub;
    /* lookups: see only earlier sub-blocks */
    for (uint32_t p = lo; p < hi; ++p) {
      if (p + 1 >= E) continue; /* last element has no two-word key */
      uint32_t v = T[oracle_hash(x[p], x[p + 1])];
      if (v == 0) continue;
      uint32_t c = v - 1;
      uint32_t o = p - c;
      if (o >= 1 && o <= OR_MAX_FAR) cand[p] = o;
    }
    /* barrier, then inserts: keep the largest position+1.  The inserts of
     * one sub-block may land in any order; walking them backwards here makes
     * the max (not the arrival order) decide what a bucket keeps. */
    for (uint32_t p = hi; p-- > lo;) {
      if (p + 1 >= E) continue;
      uint32_t h = oracle_hash(x[p], x[p + 1]);
      if (p + 1 > T[h]) T[h] = p + 1;
    }
  }
  if (table_out) memcpy(table_out, T, OR_HASH_SIZE * sizeof(uint32_t));
  free(T);
}

/* Minimum match length that pays for its 2-byte token: a match is taken
 * only when L * ws > 2 (reading: the page fixes the token at 2 bytes and a
 * literal at ws bytes, and is silent on the threshold). */
static uint32_t min_match(uint32_t ws) { return ws >= 4u ? 1u : (ws == 2u ? 2u : 3u); }

/* Encode one chunk.  bytes points at its b_c real bytes; the rest of the
 * cs-byte chunk is zero padding (page: alignment paragraph).  On return
 * *flag_size / *data_size hold the 8-byte size-table entry and payload[]
 * (capacity >= cs) holds *payload_bytes bytes.
 * Returns OR_OK or OR_EINVAL. */
static int encode_chunk_search(const uint8_t* bytes, uint32_t bc, uint32_t cs, uint32_t ws, uint32_t level,
                               uint32_t window, int advancing, uint32_t* flag_size, uint32_t* data_size,
                               uint8_t* payload, uint32_t* payload_bytes) {
  if (!cs_ok(cs) || !ws_ok(ws) || level > 1u || !window_ok(window) || bc == 0 || bc > cs) return OR_EINVAL;
  if (advancing && level != 0u) return OR_EINVAL;
  uint32_t E = cs / ws;
  uint8_t* padded = (uint8_t*)calloc(cs, 1);
  memcpy(padded, bytes, bc);
  uint32_t* x = (uint32_t*)malloc(sizeof(uint32_t) * E);
  for (uint32_t i = 0; i < E; ++i) x[i] = load_word(padded + (size_t)i * ws, ws);

  /* 1. all-zero chunk: sentinel entry (0, 0), no payload (page: zero-chunk
   *    fast path paragraph). */
  int all_zero = 1;
  for (uint32_t i = 0; i < E; ++i)
    if (x[i] != 0) { all_zero = 0; break; }
  if (all_zero) {
    *flag_size = 0; *data_size = 0; *payload_bytes = 0;
    free(x); free(padded);
    return OR_OK;
  }

  /* 2. level-1 candidate offsets (before the parse). */
  uint32_t* cand = NULL;
  if (level == 1u) {
    cand = (uint32_t*)malloc(sizeof(uint32_t) * E);
    oracle_level1_candidates(x, E, cand, NULL);
  }

  /* 3. sequential greedy parse (page: provenance paragraph, parse follows
   *    the upstream compressKernelI). Items are recorded as (is_match, a, b):
   *    literal -> a = element index; match -> a = L, b = O. */
  uint8_t* is_match = (uint8_t*)malloc(E);
  uint32_t* ia = (uint32_t*)malloc(sizeof(uint32_t) * E);
  uint32_t* ib = (uint32_t*)malloc(sizeof(uint32_t) * E);
  uint32_t items = 0, mm = min_match(ws);
  uint32_t p = 0;
  while (p < E) {
    uint32_t L, O;
    if (advancing) oracle_advancing_match(x, E, p, &L, &O);
    else oracle_near_match_w(x, E, p, window, &L, &O);
    if (cand && cand[p] != 0) {
      uint32_t r = run_at(x, E, p, cand[p]);
      if (r > L) { L = r; O = cand[p]; } /* hash wins only when strictly longer */
    }
    if (L >= mm) {
      is_match[items] = 1; ia[items] = L; ib[items] = O;
      p += L;
    } else {
      is_match[items] = 0; ia[items] = p; ib[items] = 0;
      p += 1;
    }
    ++items;
  }

  /* 4. serialize: flag bitmap (bit k of item k, LSB first, 1 = match, unused
   *    bits 0) then the data bytes (literal = ws bytes little-endian, match =
   *    length byte then offset byte; page: intro paragraph on item forms). */
  uint32_t F = (items + 7u) / 8u;
  uint32_t D = 0;
  for (uint32_t k = 0; k < items; ++k) D += is_match[k] ? 2u : ws;

  if ((uint64_t)F + D >= bc) {
    /* raw fallback: the real bytes verbatim, high bit on the entry (page:
     * raw-fallback paragraph). */
    *flag_size = 0;
    *data_size = OR_RAW_BIT | bc;
    memcpy(payload, bytes, bc);
    *payload_bytes = bc;
  } else {
    memset(payload, 0, F);
    uint8_t* d = payload + F;
    for (uint32_t k = 0; k < items; ++k) {
      if (is_match[k]) {
        payload[k >> 3] |= (uint8_t)(1u << (k & 7u));
        d[0] = (uint8_t)ia[k];
        d[1] = (uint8_t)ib[k];
        d += 2;
      } else {
        memcpy(d, padded + (size_t)ia[k] * ws, ws);
        d += ws;
      }
    }
    *flag_size = F;
    *data_size = D;
    *payload_bytes = F + D;
  }
  free(ib); free(ia); free(is_match); free(cand); free(x); free(padded);
  return OR_OK;
}

int oracle_encode_chunk_w(const uint8_t* bytes, uint32_t bc, uint32_t cs, uint32_t ws, uint32_t level,
                          uint32_t window, uint32_t* flag_size, uint32_t* data_size, uint8_t* payload,
                          uint32_t* payload_bytes) {
  return encode_chunk_search(bytes, bc, cs, ws, level, window, 0, flag_size, data_size, payload, payload_bytes);
}

int oracle_encode_chunk(const uint8_t* bytes, uint32_t bc, uint32_t cs, uint32_t ws, uint32_t level,
                        uint32_t* flag_size, uint32_t* data_size, uint8_t* payload, uint32_t* payload_bytes) {
  return oracle_encode_chunk_w(bytes, bc, cs, ws, level, OR_WINDOW, flag_size, data_size, payload, payload_bytes);
}

/* Encode a whole buffer into one stream:
 *   32-byte header | num_chunks x {u32 flag_size, u32 data_size} | payloads
 * Payloads are packed back to back in chunk order; chunk offsets are not
 * stored (page: CUDA-graph paragraph, the inverse derives them from sizes).
 * Returns the stream length, or a negative status. */
static int64_t encode_search(const uint8_t* in, uint64_t n, uint32_t cs, uint32_t ws, uint32_t level,
                             uint32_t window, int advancing, uint8_t* out, uint64_t cap) {
  if (!cs_ok(cs) || !ws_ok(ws) || level > 1u || !window_ok(window)) return OR_EINVAL;
  if (advancing && level != 0u) return OR_EINVAL;
  if (n > 0 && in == NULL) return OR_EINVAL;
  uint64_t chunks = (n + cs - 1) / cs;
  if (chunks > 0xFFFFFFFFull) return OR_EINVAL;
  if (out == NULL || cap < oracle_max_stream_size(n, cs)) return OR_ECAP;

  uint8_t* table = out + OR_HEADER_BYTES;
  uint8_t* pay = table + OR_ENTRY_BYTES * chunks;
  uint64_t total = 0;
  for (uint64_t c = 0; c < chunks; ++c) {
    uint64_t start = c * cs;
    uint32_t bc = (uint32_t)((n - start) < cs ? (n - start) : cs);
    uint32_t f, d, pb;
    int st = encode_chunk_search(in + start, bc, cs, ws, level, window, advancing, &f, &d, pay + total, &pb);
    if (st != OR_OK) return st;
    put_u32(table + OR_ENTRY_BYTES * c, f);
    put_u32(table + OR_ENTRY_BYTES * c + 4, d);
    total += pb;
  }
  put_u32(out + 0, OR_MAGIC);
  out[4] = (uint8_t)OR_VERSION;
  out[5] = (uint8_t)ws;
  out[6] = 0;
  out[7] = 0;
  put_u32(out + 8, cs);
  put_u32(out + 12, (uint32_t)chunks);
  put_u64(out + 16, n);
  put_u64(out + 24, total);
  return (int64_t)(OR_HEADER_BYTES + OR_ENTRY_BYTES * chunks + total);
}

int64_t oracle_encode_w(const uint8_t* in, uint64_t n, uint32_t cs, uint32_t ws, uint32_t level, uint32_t window,
                        uint8_t* out, uint64_t cap) {
  return encode_search(in, n, cs, ws, level, window, 0, out, cap);
}

int64_t oracle_encode(const uint8_t* in, uint64_t n, uint32_t cs, uint32_t ws, uint32_t level, uint8_t* out,
                      uint64_t cap) {
  return oracle_encode_w(in, n, cs, ws, level, OR_WINDOW, out, cap);
}

/* The same stream with the upstream-style advancing search in place of the
 * exact one (level 0 only: the greedy parse, the item forms and the raw
 * fallback are unchanged, so the stream decodes with the same decoder). */
int64_t oracle_encode_advancing(const uint8_t* in, uint64_t n, uint32_t cs, uint32_t ws, uint8_t* out, uint64_t cap) {
  return encode_search(in, n, cs, ws, 0u, OR_WINDOW, 1, out, cap);
}

/* Read the header.  Returns OR_OK or OR_ECORRUPT. */
int oracle_stream_info(const uint8_t* s, uint64_t in_bytes, uint64_t* original_size,
                       uint64_t* stream_bytes, uint32_t* cs_out, uint32_t* ws_out) {
  if (in_bytes < OR_HEADER_BYTES) return OR_ECORRUPT;
  if (get_u32(s) != OR_MAGIC || s[4] != OR_VERSION || s[6] != 0 || s[7] != 0) return OR_ECORRUPT;
  uint32_t ws = s[5], cs = get_u32(s + 8), chunks = get_u32(s + 12);
  uint64_t n = get_u64(s + 16), pb = get_u64(s + 24);
  if (!ws_ok(ws) || !cs_ok(cs)) return OR_ECORRUPT;
  if ((n + cs - 1) / cs != chunks) return OR_ECORRUPT;
  if (pb > n) return OR_ECORRUPT;
  *original_size = n;
  *stream_bytes = OR_HEADER_BYTES + (uint64_t)OR_ENTRY_BYTES * chunks + pb;
  *cs_out = cs;
  *ws_out = ws;
  return OR_OK;
}

/* Decode one compressed (not zero, not raw) chunk into out[cs].  Walks the
 * items in order; every check failure returns OR_ECORRUPT. */
static int decode_items(const uint8_t* flags, uint32_t F, const uint8_t* data, uint32_t D,
                        uint32_t cs, uint32_t ws, uint8_t* out) {
  uint32_t E = cs / ws;
  uint32_t* x = (uint32_t*)malloc(sizeof(uint32_t) * E);
  uint32_t q = 0, d = 0, k = 0;
  int st = OR_OK;
  while (q < E) {
    if (k >= 8u * F) { st = OR_ECORRUPT; break; }
    int m = (flags[k >> 3] >> (k & 7u)) & 1;
    if (m) {
      if (d + 2u > D) { st = OR_ECORRUPT; break; }
      uint32_t L = data[d], O = data[d + 1];
      d += 2;
      if (L == 0 || O == 0 || O > q || q + L > E) { st = OR_ECORRUPT; break; }
      for (uint32_t j = 0; j < L; ++j) { x[q] = x[q - O]; ++q; } /* overlap allowed */
    } else {
      if (d + ws > D) { st = OR_ECORRUPT; break; }
      x[q++] = load_word(data + d, ws);
      d += ws;
    }
    ++k;
  }
  if (st == OR_OK) {
    if (d != D) st = OR_ECORRUPT;
    for (uint32_t b = k; b < 8u * F && st == OR_OK; ++b)
      if ((flags[b >> 3] >> (b & 7u)) & 1) st = OR_ECORRUPT; /* pad bits must be 0 */
    if ((k + 7u) / 8u != F) st = OR_ECORRUPT;
  }
  if (st == OR_OK)
    for (uint32_t i = 0; i < E; ++i)
      for (uint32_t b = 0; b < ws; ++b) out[(size_t)i * ws + b] = (uint8_t)(x[i] >> (8 * b));
  free(x);
  return st;
}

/* Decode a whole stream into out (capacity cap).  Returns original_size or
 * a negative status; never reads past in_bytes or writes past cap. */
int64_t oracle_decode(const uint8_t* s, uint64_t in_bytes, uint8_t* out, uint64_t cap) {
  uint64_t n, total;
  uint32_t cs, ws;
  if (s == NULL) return OR_EINVAL;
  int st = oracle_stream_info(s, in_bytes, &n, &total, &cs, &ws);
  if (st != OR_OK) return st;
  if (in_bytes < total) return OR_ECORRUPT;
  if (cap < n || (n > 0 && out == NULL)) return OR_ECAP;
  uint64_t chunks = (n + cs - 1) / cs;
  const uint8_t* table = s + OR_HEADER_BYTES;
  const uint8_t* pay = table + OR_ENTRY_BYTES * chunks;
  uint64_t pb = get_u64(s + 24);
  uint64_t off = 0;
  uint8_t* tmp = (uint8_t*)malloc(cs);
  for (uint64_t c = 0; c < chunks && st == OR_OK; ++c) {
    uint64_t start = c * cs;
    uint32_t bc = (uint32_t)((n - start) < cs ? (n - start) : cs);
    uint32_t f = get_u32(table + OR_ENTRY_BYTES * c), d = get_u32(table + OR_ENTRY_BYTES * c + 4);
    if (f == 0 && d == 0) { /* zero chunk */
      memset(out + start, 0, bc);
      continue;
    }
    if (f == 0 && (d & OR_RAW_BIT)) { /* raw chunk */
      if ((d & ~OR_RAW_BIT) != bc || off + bc > pb) { st = OR_ECORRUPT; break; }
      memcpy(out + start, pay + off, bc);
      off += bc;
      continue;
    }
    if (f == 0 || (d & OR_RAW_BIT) || (uint64_t)f + d >= bc || off + f + d > pb) { st = OR_ECORRUPT; break; }
    st = decode_items(pay + off, f, pay + off + f, d, cs, ws, tmp);
    if (st != OR_OK) break;
    /* the padded tail must decode to zeros: the encoder only pads with 0 */
    for (uint32_t b = bc; b < cs; ++b)
      if (tmp[b] != 0) { st = OR_ECORRUPT; break; }
    memcpy(out + start, tmp, bc);
    off += (uint64_t)f + d;
  }
  free(tmp);
  if (st != OR_OK) return st;
  if (off != pb) return OR_ECORRUPT;
  return (int64_t)n;
}

/* ---- split mode --------------------------------------------------------
 * The same items in four ports instead of one interleaved stream (codebase
 * notes CN-GPULZ-1, split mode; GPULZStage page, split-mode paragraphs):
 *   literals  literal words of coded chunks in item order, and the real
 *             bytes of raw chunks (they are all literal);
 *   lengths   one length byte per match item;
 *   offsets   one offset byte per match item;
 *   meta      the 32-byte header (version byte 2), one entry per chunk, then
 *             the flag bitmaps of the coded chunks back to back.
 * Readings (the pages give the ports, not their byte layout): ports follow
 * chunk order; a coded chunk's entry is {u32 items K, u32 matches M}; zero
 * and raw chunks keep their entries (0,0) and (0, 0x80000000 | real bytes);
 * a chunk is raw exactly when its single-stream form would be; the header's
 * last field holds the total flag bytes. */
#define OR_SPLIT_VERSION 2u

/* Port capacities that always suffice. */
void oracle_split_bounds(uint64_t n, uint32_t cs, uint32_t ws, uint64_t* lit, uint64_t* tok, uint64_t* meta) {
  uint64_t chunks = (n + cs - 1) / cs;
  *lit = n;           /* a coded chunk's literals are fewer than its bytes */
  *tok = n / 2 + 1;   /* two data bytes per match, and fewer than the chunk */
  *meta = OR_HEADER_BYTES + OR_ENTRY_BYTES * chunks + chunks * ((cs / ws + 7u) / 8u);
}

/* Encode into the four ports.  sizes[0..3] = bytes written to literals,
 * lengths, offsets, meta.  Returns OR_OK or a negative status. */
int oracle_encode_split(const uint8_t* in, uint64_t n, uint32_t cs, uint32_t ws, uint32_t level,
                        uint8_t* lit, uint64_t lit_cap, uint8_t* lens, uint8_t* offs, uint64_t tok_cap,
                        uint8_t* meta, uint64_t meta_cap, uint64_t* sizes) {
  if (!cs_ok(cs) || !ws_ok(ws) || level > 1u) return OR_EINVAL;
  if (n > 0 && in == NULL) return OR_EINVAL;
  uint64_t chunks = (n + cs - 1) / cs;
  if (chunks > 0xFFFFFFFFull) return OR_EINVAL;
  uint64_t blit, btok, bmeta;
  oracle_split_bounds(n, cs, ws, &blit, &btok, &bmeta);
  if (meta == NULL || lit_cap < blit || tok_cap < btok || meta_cap < bmeta) return OR_ECAP;
  if (n > 0 && (lit == NULL || lens == NULL || offs == NULL)) return OR_ECAP;

  uint8_t* table = meta + OR_HEADER_BYTES;
  uint8_t* flags_out = table + OR_ENTRY_BYTES * chunks;
  uint8_t* payload = (uint8_t*)malloc(cs + 8);
  uint64_t nl = 0, nt = 0, nf = 0;
  for (uint64_t c = 0; c < chunks; ++c) {
    uint64_t start = c * cs;
    uint32_t bc = (uint32_t)((n - start) < cs ? (n - start) : cs);
    uint32_t f, d, pb;
    int st = oracle_encode_chunk(in + start, bc, cs, ws, level, &f, &d, payload, &pb);
    if (st != OR_OK) { free(payload); return st; }
    if (f == 0) { /* zero or raw: the entry as in one stream; raw bytes to literals */
      put_u32(table + OR_ENTRY_BYTES * c, 0);
      put_u32(table + OR_ENTRY_BYTES * c + 4, d);
      memcpy(lit + nl, payload, pb);
      nl += pb;
      continue;
    }
    /* coded: walk the single-stream items in order and deal them out */
    const uint8_t* fl = payload;
    const uint8_t* dp = payload + f;
    uint32_t used = 0, K = 0, M = 0;
    while (used < d) {
      if ((fl[K >> 3] >> (K & 7u)) & 1u) {
        lens[nt + M] = dp[used];
        offs[nt + M] = dp[used + 1];
        used += 2;
        ++M;
      } else {
        memcpy(lit + nl, dp + used, ws);
        nl += ws;
        used += ws;
      }
      ++K;
    }
    put_u32(table + OR_ENTRY_BYTES * c, K);
    put_u32(table + OR_ENTRY_BYTES * c + 4, M);
    memcpy(flags_out + nf, fl, f); /* f = ceil(K / 8), unused bits 0 */
    nf += f;
    nt += M;
  }
  free(payload);
  put_u32(meta + 0, OR_MAGIC);
  meta[4] = (uint8_t)OR_SPLIT_VERSION;
  meta[5] = (uint8_t)ws;
  meta[6] = 0;
  meta[7] = 0;
  put_u32(meta + 8, cs);
  put_u32(meta + 12, (uint32_t)chunks);
  put_u64(meta + 16, n);
  put_u64(meta + 24, nf);
  sizes[0] = nl;
  sizes[1] = nt;
  sizes[2] = nt;
  sizes[3] = OR_HEADER_BYTES + OR_ENTRY_BYTES * chunks + nf;
  return OR_OK;
}

/* Decode from the four ports (each at least as long as the table implies;
 * extra bytes are ignored).  Returns original_size or a negative status;
 * never reads past a port's given length or writes past cap. */
int64_t oracle_decode_split(const uint8_t* lit, uint64_t lit_n, const uint8_t* lens, const uint8_t* offs,
                            uint64_t tok_n, const uint8_t* meta, uint64_t meta_n, uint8_t* out, uint64_t cap) {
  if (meta == NULL) return OR_EINVAL;
  if (meta_n < OR_HEADER_BYTES) return OR_ECORRUPT;
  if (get_u32(meta) != OR_MAGIC || meta[4] != OR_SPLIT_VERSION || meta[6] != 0 || meta[7] != 0) return OR_ECORRUPT;
  uint32_t ws = meta[5], cs = get_u32(meta + 8), chunks = get_u32(meta + 12);
  uint64_t n = get_u64(meta + 16), nf_total = get_u64(meta + 24);
  if (!ws_ok(ws) || !cs_ok(cs) || (n + cs - 1) / cs != chunks) return OR_ECORRUPT;
  if ((uint64_t)OR_HEADER_BYTES + (uint64_t)OR_ENTRY_BYTES * chunks > meta_n) return OR_ECORRUPT;
  if (nf_total > meta_n - OR_HEADER_BYTES - (uint64_t)OR_ENTRY_BYTES * chunks) return OR_ECORRUPT;
  if (cap < n || (n > 0 && out == NULL)) return OR_ECAP;
  const uint8_t* table = meta + OR_HEADER_BYTES;
  const uint8_t* flags = table + OR_ENTRY_BYTES * chunks;
  uint32_t E = cs / ws;
  uint32_t* x = (uint32_t*)malloc(sizeof(uint32_t) * E);
  uint64_t nl = 0, nt = 0, nf = 0;
  int st = OR_OK;
  for (uint64_t c = 0; c < chunks && st == OR_OK; ++c) {
    uint64_t start = c * cs;
    uint32_t bc = (uint32_t)((n - start) < cs ? (n - start) : cs);
    uint32_t K = get_u32(table + OR_ENTRY_BYTES * c), M = get_u32(table + OR_ENTRY_BYTES * c + 4);
    if (K == 0 && M == 0) { memset(out + start, 0, bc); continue; }
    if (K == 0 && (M & OR_RAW_BIT)) {
      if ((M & ~OR_RAW_BIT) != bc || nl + bc > lit_n) { st = OR_ECORRUPT; break; }
      memcpy(out + start, lit + nl, bc);
      nl += bc;
      continue;
    }
    /* coded: K items, M of them matches; its single-stream form must have
     * been smaller than the chunk (else it would be raw) */
    uint32_t F = (uint32_t)(((uint64_t)K + 7u) / 8u);
    if (K == 0 || M > K || K > E) { st = OR_ECORRUPT; break; }
    if ((uint64_t)F + (uint64_t)ws * (K - M) + 2ull * M >= bc) { st = OR_ECORRUPT; break; }
    if (nf + F > nf_total || nl + (uint64_t)ws * (K - M) > lit_n || nt + M > tok_n) { st = OR_ECORRUPT; break; }
    const uint8_t* fl = flags + nf;
    uint32_t q = 0, m = 0;
    for (uint32_t k = 0; k < K && st == OR_OK; ++k) {
      if (q >= E) { st = OR_ECORRUPT; break; } /* more items than elements */
      if ((fl[k >> 3] >> (k & 7u)) & 1u) {
        if (m >= M) { st = OR_ECORRUPT; break; }
        uint32_t L = lens[nt + m], O = offs[nt + m];
        ++m;
        if (L == 0 || O == 0 || O > q || q + L > E) { st = OR_ECORRUPT; break; }
        for (uint32_t j = 0; j < L; ++j) { x[q] = x[q - O]; ++q; }
      } else {
        if ((uint64_t)(k - m) >= (uint64_t)(K - M)) { st = OR_ECORRUPT; break; }
        x[q++] = load_word(lit + nl + (uint64_t)ws * (k - m), ws);
      }
    }
    if (st != OR_OK) break;
    if (q != E || m != M) { st = OR_ECORRUPT; break; }
    for (uint32_t b = K; b < 8u * F; ++b)
      if ((fl[b >> 3] >> (b & 7u)) & 1u) { st = OR_ECORRUPT; break; } /* unused flag bits are 0 */
    if (st != OR_OK) break;
    for (uint32_t i = 0; i < E && st == OR_OK; ++i)
      for (uint32_t b = 0; b < ws; ++b) {
        uint64_t pos = (uint64_t)i * ws + b;
        uint8_t v = (uint8_t)(x[i] >> (8 * b));
        if (pos < bc) out[start + pos] = v;
        else if (v != 0) { st = OR_ECORRUPT; break; } /* padding decodes to zeros */
      }
    nl += (uint64_t)ws * (K - M);
    nt += M;
    nf += F;
  }
  free(x);
  if (st != OR_OK) return st;
  if (nf != nf_total) return OR_ECORRUPT;
  return (int64_t)n;
}

/* ---- Lorenzo-quantizer front end ------------------------------------------
 * The coder's measured input is Lorenzo-quantized residuals of a float field
 * (GPULZStage page, results paragraph); LorenzoQuant turns float32 values
 * into integer codes (its alignment paragraph).  The pages give no formula;
 * this is the plainest reading, written out cell by cell:
 *   q(z,y,x) = round-half-even(f(z,y,x) / (2 eb)), in double precision;
 *   delta    = sum over the corners (dz,dy,dx) in {0,1}^3 of
 *              (-1)^(dz+dy+dx) q(z-dz, y-dy, x-dx), cells outside the grid 0;
 *   code     = delta + 32768, clamped to [0, 65535].
 * Field and codes are x fastest, then y, then z.  Returns the number of
 * clamped cells.  Parity pins: closed forms (constant and ramp fields), the
 * inverse (prefix sums of code - 32768 give back q), the error bound
 * |f - 2 eb q| <= eb, round-half-even ties, clamping. */
uint64_t oracle_lorenzo_quant(const float* f, uint32_t nx, uint32_t ny, uint32_t nz, double eb, uint32_t* codes) {
  uint64_t clamped = 0;
  for (uint32_t z = 0; z < nz; ++z)
    for (uint32_t y = 0; y < ny; ++y)
      for (uint32_t x = 0; x < nx; ++x) {
        int64_t delta = 0;
        for (uint32_t dz = 0; dz < 2; ++dz)
          for (uint32_t dy = 0; dy < 2; ++dy)
            for (uint32_t dx = 0; dx < 2; ++dx) {
              if (z < dz || y < dy || x < dx) continue; /* outside the grid: 0 */
              uint64_t at = ((uint64_t)(z - dz) * ny + (y - dy)) * nx + (x - dx);
              int64_t q = (int64_t)rint((double)f[at] / (2.0 * eb));
              delta += ((dz + dy + dx) & 1u) ? -q : q;
            }
        int64_t code = delta + 32768;
        if (code < 0 || code > 65535) {
          ++clamped;
          code = code < 0 ? 0 : 65535;
        }
        codes[((uint64_t)z * ny + y) * nx + x] = (uint32_t)code;
      }
  return clamped;
}
