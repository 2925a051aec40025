/* gpulz_split.h -- split mode of the chunked LZSS coder (gfx950).
 *
 * The same items as the one-stream form of gpulz.h (the same search, parse
 * and raw / zero decisions at the given match level), written to four ports
 * instead of one interleaved stream (FZGPUModules codebase notes CN-GPULZ-1,
 * split mode; GPULZStage page, split-mode paragraphs: literals / lengths /
 * offsets / meta, raw-fallback chunks folded into literals, size table and
 * flag bitmaps into meta, decode straight out of the ports).
 *
 * Port layout (the pages give the ports, not their bytes; this is the
 * library's reading), all in chunk order, items in item order:
 *   literals  each coded chunk's literal words (word_size bytes, little
 *             endian), and each raw chunk's real bytes;
 *   lengths   one length byte per match item;
 *   offsets   one offset byte per match item;
 *   meta      32-byte header as in gpulz.h but version byte 2 and, in the last
 *             u64, the total flag bytes | one u32 pair per chunk: coded
 *             {items K, matches M}, zero (0,0), raw (0, 0x80000000 | real
 *             bytes) | the coded chunks' flag bitmaps ((K + 7) / 8 bytes each,
 *             bit k = item k is a match, unused bits 0) back to back.
 * A chunk is raw exactly when its one-stream form would be.
 *
 * Conventions as in gpulz.h: device pointers, caller-provided workspace of
 * any alignment, all work on `stream`, no host synchronization, host-visible
 * argument errors returned before anything is enqueued.
 */
#ifndef GPULZ_SPLIT_H
#define GPULZ_SPLIT_H

#include "gpulz.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Port capacities that always suffice for n_bytes at chunk_size/word_size:
 * literals n_bytes, lengths and offsets n_bytes / 2 + 1 each, meta
 * 32 + 8 * chunks + chunks * ceil(chunk_size / word_size / 8).
 * Returns GPULZ_OK, or GPULZ_ERR_INVALID_ARG for an unsupported size or a
 * null output pointer. */
GPULZ_API int gpulz_split_bounds(uint64_t n_bytes, uint32_t chunk_size, uint32_t word_size, uint64_t* lit_cap,
                                 uint64_t* tok_cap, uint64_t* meta_cap);

/* Device workspace bytes gpulz_encode_split needs (0 if chunk_size is unsupported). */
GPULZ_API uint64_t gpulz_encode_split_workspace_size(uint64_t n_bytes, uint32_t chunk_size);

/* Encode d_in[0, n_bytes) into the four ports.
 *   d_lit / lit_cap, d_lens and d_offs / tok_cap (each), d_meta / meta_cap:
 *     device buffers of at least the gpulz_split_bounds capacities
 *     (GPULZ_ERR_CAPACITY otherwise, nothing enqueued);
 *   d_port_bytes: device u64[4], receives the bytes written to literals,
 *     lengths, offsets, meta (all 0 if the kernels report an internal stall);
 *   other arguments as gpulz_encode.
 * Port bytes are identical across runs, streams and workspace contents. */
GPULZ_API int gpulz_encode_split(const void* d_in, uint64_t n_bytes, uint32_t chunk_size, uint32_t word_size,
                                 uint32_t match_level, void* d_lit, uint64_t lit_cap, void* d_lens, void* d_offs,
                                 uint64_t tok_cap, void* d_meta, uint64_t meta_cap, uint64_t* d_port_bytes,
                                 void* d_workspace, uint64_t workspace_bytes, hipStream_t stream);

/* Device workspace bytes gpulz_decode_split needs for a meta port of meta_bytes. */
GPULZ_API uint64_t gpulz_decode_split_workspace_size(uint64_t meta_bytes);

/* Decode four ports into d_out.  lit_bytes, tok_bytes (each of lengths and
 * offsets) and meta_bytes are the readable bytes of the ports; the entries
 * must fit in them (extra bytes are ignored).  Results as gpulz_decode:
 * *d_status 0 / 2 (out_capacity below the original size, nothing written) /
 * 3 (corrupt: a rule of the format is broken), *d_out_bytes the original size
 * or 0.  Never reads outside the ports or writes outside d_out[0, out_capacity).
 * Host-side errors: GPULZ_ERR_INVALID_ARG (null pointer), GPULZ_ERR_CORRUPT
 * (meta_bytes < 32), GPULZ_ERR_CAPACITY (workspace too small), GPULZ_ERR_HIP. */
GPULZ_API int gpulz_decode_split(const void* d_lit, uint64_t lit_bytes, const void* d_lens, const void* d_offs,
                                 uint64_t tok_bytes, const void* d_meta, uint64_t meta_bytes, void* d_out,
                                 uint64_t out_capacity, uint64_t* d_out_bytes, uint32_t* d_status, void* d_workspace,
                                 uint64_t workspace_bytes, hipStream_t stream);

/* Host-side read of a meta port's header (no device access): from the first
 * `bytes` (>= 32) bytes of a meta port in host memory, return its original
 * size, the meta port's length (header, rows and flag bytes), chunk_size and
 * word_size.  GPULZ_ERR_CORRUPT if they are not a valid split-mode header
 * (magic, version 2, reserved bytes, supported sizes, chunk count matching
 * the original size); any output pointer may be NULL. */
GPULZ_API int gpulz_split_info(const void* h_prefix, uint64_t bytes, uint64_t* original_size,
                               uint64_t* meta_bytes, uint32_t* chunk_size, uint32_t* word_size);

#ifdef __cplusplus
}
#endif

#endif /* GPULZ_SPLIT_H */
