// abi.hip -- the extern "C" entry points declared in include/gpulz.h.
// Host-side argument checks happen before anything is enqueued; the rest is
// workspace carving and kernel launches on the caller's stream.
#include "gpulz.h"
#include "gpulz_timing.h"
#include "gpulz_split.h"
#include "gpulz_baseline.h"
#include "gpulz_window.h"

#include <mutex>

#include "common.h"
#include "scan_tiles.h"

using namespace gpulz;

namespace {

constexpr uint64_t kAlign = 256;
constexpr uint64_t kStagingSlack = 256;  // realigning copies read a few bytes past a slot
inline uint64_t round_up(uint64_t v) { return (v + kAlign - 1) / kAlign * kAlign; }
// The workspace may start at any address: every layout reserves kAlign more
// bytes and is carved from the first kAlign-aligned address inside it.
inline uint8_t* align_up(void* p) { return (uint8_t*)(((uintptr_t)p + kAlign - 1) & ~(uintptr_t)(kAlign - 1)); }
inline uint64_t num_chunks_of(uint64_t n, uint32_t cs) { return n / cs + ((n % cs) != 0); }

struct EncLayoutHost {
  uint64_t ctl, tiles, staging, total;
};

// control block | compaction tile flags | one cs-byte payload slot per chunk
EncLayoutHost enc_layout(uint64_t chunks, uint32_t cs) {
  EncLayoutHost L;
  L.ctl = 0;
  L.tiles = round_up(encode_ctl_bytes());
  L.staging = L.tiles + round_up((encode_tiles((uint32_t)chunks) + 1u) * 8u);
  L.total = L.staging + round_up(chunks * cs + kStagingSlack) + kAlign;
  return L;
}

struct DecLayoutHost {
  uint64_t params, loc, tile_sums, tile_err, total;
};

// parameters | per-chunk offsets within scan tiles (u32) | tile totals | tile error flags
DecLayoutHost dec_layout(uint64_t chunks_cap) {
  DecLayoutHost L;
  L.params = 0;
  L.loc = round_up(decode_params_bytes());
  L.tile_sums = L.loc + round_up((chunks_cap ? chunks_cap : 1) * 4u);
  // a stream of at most chunks_cap chunks has at most this many scan tiles
  // (scan_tiles.h); the launch clamps the bound to 2^32 - 1 chunks
  const uint64_t tiles = workspace_tiles(chunks_cap > 0xFFFFFFFFull ? 0xFFFFFFFFull : chunks_cap);
  L.tile_err = L.tile_sums + round_up(tiles * 8u);
  L.total = L.tile_err + round_up(tiles * 4u) + kAlign;
  return L;
}

// split encode: control block | three sets of tile flags | {items, matches}
// per chunk | one cs-byte payload slot per chunk
struct EncSplitLayoutHost {
  uint64_t ctl, tiles, km, staging, total;
};
EncSplitLayoutHost enc_split_layout(uint64_t chunks, uint32_t cs) {
  EncSplitLayoutHost L;
  L.ctl = 0;
  L.tiles = round_up(encode_ctl_bytes());
  L.km = L.tiles + round_up((3u * encode_tiles((uint32_t)chunks) + 1u) * 8u);
  L.staging = L.km + round_up((chunks ? chunks : 1) * 8u);
  L.total = L.staging + round_up(chunks * cs + kStagingSlack) + kAlign;
  return L;
}

// split decode: parameters | 3 x chunk offsets in tiles | 3 x 4096 tile totals | tile errors
constexpr uint64_t kSplitTiles = 4096;
struct DecSplitLayoutHost {
  uint64_t params, loc, tile_sums, tile_err, total;
};
DecSplitLayoutHost dec_split_layout(uint64_t chunks_cap) {
  DecSplitLayoutHost L;
  L.params = 0;
  L.loc = round_up(decode_params_bytes());
  L.tile_sums = L.loc + round_up(3u * (chunks_cap ? chunks_cap : 1) * 4u);
  L.tile_err = L.tile_sums + round_up(3u * kSplitTiles * 8u);
  L.total = L.tile_err + round_up(kSplitTiles * 4u) + kAlign;
  return L;
}

uint64_t dec_chunks_bound(uint64_t in_bytes) { return in_bytes >= kHeaderBytes ? (in_bytes - kHeaderBytes) / 8u : 0u; }

}  // namespace

extern "C" {

uint64_t gpulz_max_compressed_size(uint64_t n_bytes, uint32_t chunk_size) {
  if (!chunk_size_ok(chunk_size)) return 0;
  return (uint64_t)kHeaderBytes + (uint64_t)kEntryBytes * num_chunks_of(n_bytes, chunk_size) + n_bytes;
}

uint64_t gpulz_encode_workspace_size(uint64_t n_bytes, uint32_t chunk_size) {
  if (!chunk_size_ok(chunk_size)) return 0;
  return enc_layout(num_chunks_of(n_bytes, chunk_size), chunk_size).total;
}

uint64_t gpulz_decode_workspace_size(uint64_t in_bytes) { return dec_layout(dec_chunks_bound(in_bytes)).total; }

}  // extern "C"

namespace {
int encode_common(const void* d_in, uint64_t n_bytes, uint32_t chunk_size, uint32_t word_size, uint32_t match_level,
                  uint32_t window, void* d_out, uint64_t out_capacity, uint64_t* d_out_bytes, void* d_workspace,
                  uint64_t workspace_bytes, hipStream_t stream, hipEvent_t ev_start, hipEvent_t ev_stop,
                  bool advancing = false) {
  if (!chunk_size_ok(chunk_size) || !word_size_ok(word_size) || match_level > 1u) return GPULZ_ERR_INVALID_ARG;
  if (window != 32u && window != 48u && window != 64u) return GPULZ_ERR_INVALID_ARG;
  if ((n_bytes > 0 && d_in == nullptr) || d_out == nullptr || d_out_bytes == nullptr || d_workspace == nullptr)
    return GPULZ_ERR_INVALID_ARG;
  const uint64_t chunks = num_chunks_of(n_bytes, chunk_size);
  if (chunks > 0xFFFFFFFFull) return GPULZ_ERR_INVALID_ARG;
  if (out_capacity < gpulz_max_compressed_size(n_bytes, chunk_size)) return GPULZ_ERR_CAPACITY;
  if (chunks > 0xFFFFFFFFull - 1024u) return GPULZ_ERR_INVALID_ARG;
  const EncLayoutHost L = enc_layout(chunks, chunk_size);
  if (workspace_bytes < L.total) return GPULZ_ERR_CAPACITY;
  uint8_t* ws = align_up(d_workspace);

  EncodeArgs ea;
  ea.in = (const uint8_t*)d_in;
  ea.n = n_bytes;
  ea.cs = chunk_size;
  ea.ws = word_size;
  ea.level = match_level;
  ea.window = window;
  ea.num_chunks = (uint32_t)chunks;
  ea.out = (uint8_t*)d_out;
  ea.out_bytes = d_out_bytes;
  ea.staging = ws + L.staging;
  ea.tile_flags = (uint64_t*)(ws + L.tiles);
  ea.ctl = ws + L.ctl;
  if (ev_start && hipEventRecord(ev_start, stream) != hipSuccess) return GPULZ_ERR_HIP;
  if ((advancing ? launch_encode_advancing(ea, stream) : launch_encode_chunks(ea, stream)) != hipSuccess)
    return GPULZ_ERR_HIP;
  if (ev_stop && hipEventRecord(ev_stop, stream) != hipSuccess) return GPULZ_ERR_HIP;
  if (launch_compact(ea, stream) != hipSuccess) return GPULZ_ERR_HIP;
  return GPULZ_OK;
}
}  // namespace

extern "C" {

int gpulz_encode_timed(const void* d_in, uint64_t n_bytes, uint32_t chunk_size, uint32_t word_size,
                       uint32_t match_level, void* d_out, uint64_t out_capacity, uint64_t* d_out_bytes,
                       void* d_workspace, uint64_t workspace_bytes, hipStream_t stream, hipEvent_t ev_start,
                       hipEvent_t ev_stop) {
  return encode_common(d_in, n_bytes, chunk_size, word_size, match_level, kWindow, d_out, out_capacity,
                       d_out_bytes, d_workspace, workspace_bytes, stream, ev_start, ev_stop);
}

int gpulz_encode_advancing_search(const void* d_in, uint64_t n_bytes, uint32_t chunk_size, uint32_t word_size,
                                  void* d_out, uint64_t out_capacity, uint64_t* d_out_bytes, void* d_workspace,
                                  uint64_t workspace_bytes, hipStream_t stream, hipEvent_t ev_start,
                                  hipEvent_t ev_stop) {
  return encode_common(d_in, n_bytes, chunk_size, word_size, 0u, kWindow, d_out, out_capacity, d_out_bytes,
                       d_workspace, workspace_bytes, stream, ev_start, ev_stop, true);
}

int gpulz_encode_window(const void* d_in, uint64_t n_bytes, uint32_t chunk_size, uint32_t word_size,
                        uint32_t match_level, uint32_t window, void* d_out, uint64_t out_capacity,
                        uint64_t* d_out_bytes, void* d_workspace, uint64_t workspace_bytes, hipStream_t stream) {
  return encode_common(d_in, n_bytes, chunk_size, word_size, match_level, window, d_out, out_capacity, d_out_bytes,
                       d_workspace, workspace_bytes, stream, nullptr, nullptr);
}

int gpulz_encode(const void* d_in, uint64_t n_bytes, uint32_t chunk_size, uint32_t word_size, uint32_t match_level,
                 void* d_out, uint64_t out_capacity, uint64_t* d_out_bytes, void* d_workspace,
                 uint64_t workspace_bytes, hipStream_t stream) {
  return gpulz_encode_timed(d_in, n_bytes, chunk_size, word_size, match_level, d_out, out_capacity, d_out_bytes,
                            d_workspace, workspace_bytes, stream, nullptr, nullptr);
}

namespace {
int decode_common(const void* d_in, uint64_t in_bytes, void* d_out, uint64_t out_capacity, uint64_t* d_out_bytes,
                  uint32_t* d_status, void* d_workspace, uint64_t workspace_bytes, hipStream_t stream,
                  hipEvent_t ev_start, hipEvent_t ev_stop, bool serial);
}  // namespace

int gpulz_decode_timed(const void* d_in, uint64_t in_bytes, void* d_out, uint64_t out_capacity,
                       uint64_t* d_out_bytes, uint32_t* d_status, void* d_workspace, uint64_t workspace_bytes,
                       hipStream_t stream, hipEvent_t ev_start, hipEvent_t ev_stop) {
  return decode_common(d_in, in_bytes, d_out, out_capacity, d_out_bytes, d_status, d_workspace, workspace_bytes,
                       stream, ev_start, ev_stop, false);
}

int gpulz_decode_one_thread_per_chunk(const void* d_in, uint64_t in_bytes, void* d_out, uint64_t out_capacity,
                                      uint64_t* d_out_bytes, uint32_t* d_status, void* d_workspace,
                                      uint64_t workspace_bytes, hipStream_t stream, hipEvent_t ev_start,
                                      hipEvent_t ev_stop) {
  return decode_common(d_in, in_bytes, d_out, out_capacity, d_out_bytes, d_status, d_workspace, workspace_bytes,
                       stream, ev_start, ev_stop, true);
}

}  // extern "C"

namespace {
// Chunk bound of a decode call: the stream's table cannot hold more rows than
// (in_bytes - 32) / 8, and the output no more chunks than one per 1024 bytes
// (the smallest chunk size).
uint64_t dec_call_chunks(uint64_t in_bytes, uint64_t out_capacity) {
  uint64_t cap = dec_chunks_bound(in_bytes);
  const uint64_t by_out = num_chunks_of(out_capacity, 1024u);
  if (by_out < cap) cap = by_out;
  if (cap > 0xFFFFFFFFull) cap = 0xFFFFFFFFull;
  return cap;
}

// Enqueue the decode kernels with the workspace laid out by L from ws (a
// kAlign-aligned address with L.total - kAlign bytes behind it).
int decode_launch(const void* d_in, uint64_t in_bytes, void* d_out, uint64_t out_capacity, uint64_t* d_out_bytes,
                  uint32_t* d_status, uint8_t* ws, const DecLayoutHost& L, uint64_t cap, hipStream_t stream,
                  hipEvent_t ev_start, hipEvent_t ev_stop, bool serial) {
  DecodeArgs da;
  da.in = (const uint8_t*)d_in;
  da.in_bytes = in_bytes;
  da.out = (uint8_t*)d_out;
  da.out_capacity = out_capacity;
  da.out_bytes = d_out_bytes;
  da.status = d_status;
  da.params = ws + L.params;
  da.loc = (uint32_t*)(ws + L.loc);
  da.tile_sums = (uint64_t*)(ws + L.tile_sums);
  da.tile_err = (uint32_t*)(ws + L.tile_err);
  da.chunks_cap = (uint32_t)cap;
  da.ev_start = ev_start;
  da.ev_stop = ev_stop;
  if ((serial ? launch_decode_serial(da, stream) : launch_decode(da, stream)) != hipSuccess) return GPULZ_ERR_HIP;
  return GPULZ_OK;
}

int decode_common(const void* d_in, uint64_t in_bytes, void* d_out, uint64_t out_capacity, uint64_t* d_out_bytes,
                  uint32_t* d_status, void* d_workspace, uint64_t workspace_bytes, hipStream_t stream,
                  hipEvent_t ev_start, hipEvent_t ev_stop, bool serial) {
  if (d_in == nullptr || d_out_bytes == nullptr || d_status == nullptr || d_workspace == nullptr)
    return GPULZ_ERR_INVALID_ARG;
  if (out_capacity > 0 && d_out == nullptr) return GPULZ_ERR_INVALID_ARG;
  if (in_bytes < kHeaderBytes) return GPULZ_ERR_CORRUPT;
  const uint64_t cap = dec_call_chunks(in_bytes, out_capacity);
  // sized by the stream bound alone, as gpulz_decode_workspace_size is
  const DecLayoutHost L = dec_layout(dec_chunks_bound(in_bytes));
  if (workspace_bytes < L.total) return GPULZ_ERR_CAPACITY;
  return decode_launch(d_in, in_bytes, d_out, out_capacity, d_out_bytes, d_status, align_up(d_workspace), L, cap,
                       stream, ev_start, ev_stop, serial);
}

// ---- decode without allocation: the workspace in a static device array ----
// The decode workspace (stream parameters, per-chunk offsets within scan
// tiles, tile totals and error flags) lives in `scratch`, one copy per GPU,
// held from the library's first use on that GPU to the end of the process.
// Every part of it is written by the scan kernel before the chunk kernel
// reads it, so nothing needs clearing between calls.  In host code `scratch`
// only names the symbol: its device address comes from hipGetSymbolAddress,
// taken once per device with that device current and kept in scratch_ptr.
constexpr uint64_t kNoAllocMaxChunks = GPULZ_DECODE_NOALLOC_MAX_CHUNKS;
constexpr uint64_t kScratchBytes = kNoAllocMaxChunks * 4u + (64u << 10);
static __device__ __align__(256) uint8_t scratch[kScratchBytes];
constexpr int kMaxDevices = 64;
std::mutex scratch_mu;
void* scratch_ptr[kMaxDevices] = {};

int scratch_of_current_device(uint8_t** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return GPULZ_ERR_HIP;
  std::lock_guard<std::mutex> lock(scratch_mu);
  if (scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return GPULZ_ERR_HIP;
    scratch_ptr[dev] = p;
  }
  *out = (uint8_t*)scratch_ptr[dev];
  return GPULZ_OK;
}
}  // namespace

extern "C" {

int gpulz_decode(const void* d_in, uint64_t in_bytes, void* d_out, uint64_t out_capacity, uint64_t* d_out_bytes,
                 uint32_t* d_status, void* d_workspace, uint64_t workspace_bytes, hipStream_t stream) {
  return gpulz_decode_timed(d_in, in_bytes, d_out, out_capacity, d_out_bytes, d_status, d_workspace,
                            workspace_bytes, stream, nullptr, nullptr);
}

int gpulz_decode_noalloc(const void* d_in, uint64_t in_bytes, void* d_out, uint64_t out_capacity,
                         uint64_t* d_out_bytes, uint32_t* d_status, hipStream_t stream) {
  if (d_in == nullptr || d_out_bytes == nullptr || d_status == nullptr) return GPULZ_ERR_INVALID_ARG;
  if (out_capacity > 0 && d_out == nullptr) return GPULZ_ERR_INVALID_ARG;
  if (in_bytes < kHeaderBytes) return GPULZ_ERR_CORRUPT;
  const uint64_t cap = dec_call_chunks(in_bytes, out_capacity);
  if (cap > kNoAllocMaxChunks) return GPULZ_ERR_CAPACITY;
  // the scan and chunk kernels never index past chunk `cap - 1` (a stream
  // declaring more chunks is rejected on the device), so the layout of the
  // call's own bound suffices
  const DecLayoutHost L = dec_layout(cap);
  if (L.total > kScratchBytes) return GPULZ_ERR_CAPACITY;
  uint8_t* ws = nullptr;
  const int rc = scratch_of_current_device(&ws);
  if (rc != GPULZ_OK) return rc;
  return decode_launch(d_in, in_bytes, d_out, out_capacity, d_out_bytes, d_status, align_up(ws), L, cap, stream,
                       nullptr, nullptr, false);
}

int gpulz_split_bounds(uint64_t n_bytes, uint32_t chunk_size, uint32_t word_size, uint64_t* lit_cap,
                       uint64_t* tok_cap, uint64_t* meta_cap) {
  if (!chunk_size_ok(chunk_size) || !word_size_ok(word_size) || !lit_cap || !tok_cap || !meta_cap)
    return GPULZ_ERR_INVALID_ARG;
  const uint64_t chunks = num_chunks_of(n_bytes, chunk_size);
  *lit_cap = n_bytes;
  *tok_cap = n_bytes / 2u + 1u;
  *meta_cap = (uint64_t)kHeaderBytes + (uint64_t)kEntryBytes * chunks + chunks * ((chunk_size / word_size + 7u) / 8u);
  return GPULZ_OK;
}

uint64_t gpulz_encode_split_workspace_size(uint64_t n_bytes, uint32_t chunk_size) {
  if (!chunk_size_ok(chunk_size)) return 0;
  return enc_split_layout(num_chunks_of(n_bytes, chunk_size), chunk_size).total;
}

int gpulz_encode_split(const void* d_in, uint64_t n_bytes, uint32_t chunk_size, uint32_t word_size,
                       uint32_t match_level, void* d_lit, uint64_t lit_cap, void* d_lens, void* d_offs,
                       uint64_t tok_cap, void* d_meta, uint64_t meta_cap, uint64_t* d_port_bytes, void* d_workspace,
                       uint64_t workspace_bytes, hipStream_t stream) {
  if (!chunk_size_ok(chunk_size) || !word_size_ok(word_size) || match_level > 1u) return GPULZ_ERR_INVALID_ARG;
  if ((n_bytes > 0 && (d_in == nullptr || d_lit == nullptr || d_lens == nullptr || d_offs == nullptr)) ||
      d_meta == nullptr || d_port_bytes == nullptr || d_workspace == nullptr)
    return GPULZ_ERR_INVALID_ARG;
  const uint64_t chunks = num_chunks_of(n_bytes, chunk_size);
  if (chunks > 0xFFFFFFFFull - 1024u) return GPULZ_ERR_INVALID_ARG;
  uint64_t bl, bt, bm;
  gpulz_split_bounds(n_bytes, chunk_size, word_size, &bl, &bt, &bm);
  if (lit_cap < bl || tok_cap < bt || meta_cap < bm) return GPULZ_ERR_CAPACITY;
  const EncSplitLayoutHost L = enc_split_layout(chunks, chunk_size);
  if (workspace_bytes < L.total) return GPULZ_ERR_CAPACITY;
  uint8_t* ws = align_up(d_workspace);
  EncodeArgs ea;
  ea.in = (const uint8_t*)d_in;
  ea.n = n_bytes;
  ea.cs = chunk_size;
  ea.ws = word_size;
  ea.level = match_level;
  ea.num_chunks = (uint32_t)chunks;
  ea.out = (uint8_t*)d_meta;
  ea.out_bytes = nullptr;
  ea.staging = ws + L.staging;
  ea.tile_flags = (uint64_t*)(ws + L.tiles);
  ea.ctl = ws + L.ctl;
  ea.km = (uint2*)(ws + L.km);
  ea.lit = (uint8_t*)d_lit;
  ea.lens = (uint8_t*)d_lens;
  ea.offs = (uint8_t*)d_offs;
  ea.port_bytes = d_port_bytes;
  if (launch_encode_chunks(ea, stream) != hipSuccess) return GPULZ_ERR_HIP;
  if (launch_split_compact(ea, stream) != hipSuccess) return GPULZ_ERR_HIP;
  return GPULZ_OK;
}

uint64_t gpulz_decode_split_workspace_size(uint64_t meta_bytes) {
  return dec_split_layout(dec_chunks_bound(meta_bytes)).total;
}

int gpulz_decode_split(const void* d_lit, uint64_t lit_bytes, const void* d_lens, const void* d_offs,
                       uint64_t tok_bytes, const void* d_meta, uint64_t meta_bytes, void* d_out, uint64_t out_capacity,
                       uint64_t* d_out_bytes, uint32_t* d_status, void* d_workspace, uint64_t workspace_bytes,
                       hipStream_t stream) {
  if (d_meta == nullptr || d_out_bytes == nullptr || d_status == nullptr || d_workspace == nullptr)
    return GPULZ_ERR_INVALID_ARG;
  if ((lit_bytes > 0 && d_lit == nullptr) || (tok_bytes > 0 && (d_lens == nullptr || d_offs == nullptr)) ||
      (out_capacity > 0 && d_out == nullptr))
    return GPULZ_ERR_INVALID_ARG;
  if (meta_bytes < kHeaderBytes) return GPULZ_ERR_CORRUPT;
  uint64_t cap = dec_chunks_bound(meta_bytes);
  const uint64_t by_out = num_chunks_of(out_capacity, 1024u);
  if (by_out < cap) cap = by_out;
  if (cap > 0xFFFFFFFFull) cap = 0xFFFFFFFFull;
  const DecSplitLayoutHost L = dec_split_layout(dec_chunks_bound(meta_bytes));
  if (workspace_bytes < L.total) return GPULZ_ERR_CAPACITY;
  uint8_t* ws = align_up(d_workspace);
  SplitDecodeArgs da;
  da.meta = (const uint8_t*)d_meta;
  da.meta_bytes = meta_bytes;
  da.lit = (const uint8_t*)d_lit;
  da.lit_bytes = lit_bytes;
  da.lens = (const uint8_t*)d_lens;
  da.offs = (const uint8_t*)d_offs;
  da.tok_bytes = tok_bytes;
  da.out = (uint8_t*)d_out;
  da.out_capacity = out_capacity;
  da.out_bytes = d_out_bytes;
  da.status = d_status;
  da.params = ws + L.params;
  da.loc = (uint32_t*)(ws + L.loc);
  da.tile_sums = (uint64_t*)(ws + L.tile_sums);
  da.tile_err = (uint32_t*)(ws + L.tile_err);
  da.chunks_cap = (uint32_t)cap;
  if (launch_decode_split(da, stream) != hipSuccess) return GPULZ_ERR_HIP;
  return GPULZ_OK;
}

namespace {
// Fields of a 32-byte header in host memory; kind = version byte wanted.
int header_fields(const void* h_prefix, uint64_t bytes, uint32_t version, uint64_t* n_out, uint64_t* last_out,
                  uint32_t* nc_out, uint32_t* cs_out, uint32_t* ws_out) {
  if (h_prefix == nullptr || bytes < kHeaderBytes) return GPULZ_ERR_CORRUPT;
  const uint8_t* s = (const uint8_t*)h_prefix;
  auto u32 = [&](int o) {
    return (uint32_t)s[o] | ((uint32_t)s[o + 1] << 8) | ((uint32_t)s[o + 2] << 16) | ((uint32_t)s[o + 3] << 24);
  };
  auto u64 = [&](int o) { return (uint64_t)u32(o) | ((uint64_t)u32(o + 4) << 32); };
  const uint32_t ws = s[5], cs = u32(8), nc = u32(12);
  const uint64_t n = u64(16);
  if (u32(0) != kMagic || s[4] != version || s[6] != 0 || s[7] != 0) return GPULZ_ERR_CORRUPT;
  if (!word_size_ok(ws) || !chunk_size_ok(cs)) return GPULZ_ERR_CORRUPT;
  if (num_chunks_of(n, cs) != nc) return GPULZ_ERR_CORRUPT;
  *n_out = n;
  *last_out = u64(24);
  *nc_out = nc;
  *cs_out = cs;
  *ws_out = ws;
  return GPULZ_OK;
}
}  // namespace

int gpulz_split_info(const void* h_prefix, uint64_t bytes, uint64_t* original_size, uint64_t* meta_bytes,
                     uint32_t* chunk_size, uint32_t* word_size) {
  uint64_t n, nflag;
  uint32_t nc, cs, ws;
  const int rc = header_fields(h_prefix, bytes, kSplitVersion, &n, &nflag, &nc, &cs, &ws);
  if (rc != GPULZ_OK) return rc;
  // at most one flag byte per 8 items, at most chunk_size / word_size items per chunk
  if (nflag > (uint64_t)nc * ((cs / ws + 7u) / 8u)) return GPULZ_ERR_CORRUPT;
  if (original_size) *original_size = n;
  if (meta_bytes) *meta_bytes = (uint64_t)kHeaderBytes + (uint64_t)kEntryBytes * nc + nflag;
  if (chunk_size) *chunk_size = cs;
  if (word_size) *word_size = ws;
  return GPULZ_OK;
}

int gpulz_stream_info(const void* h_prefix, uint64_t bytes, uint64_t* original_size, uint64_t* stream_bytes,
                      uint32_t* chunk_size, uint32_t* word_size) {
  uint64_t n, pb;
  uint32_t nc, cs, ws;
  const int rc = header_fields(h_prefix, bytes, kVersion, &n, &pb, &nc, &cs, &ws);
  if (rc != GPULZ_OK) return rc;
  if (pb > n) return GPULZ_ERR_CORRUPT;
  if (original_size) *original_size = n;
  if (stream_bytes) *stream_bytes = (uint64_t)kHeaderBytes + (uint64_t)kEntryBytes * nc + pb;
  if (chunk_size) *chunk_size = cs;
  if (word_size) *word_size = ws;
  return GPULZ_OK;
}

}  // extern "C"
