/*
 * gpulz.h -- C ABI of the MI355X (gfx950) chunked LZSS coder.
 *
 * The method is the GPU LZSS stage described on the FZGPUModules
 * "fz::GPULZStage" page: the input is cut into independent chunk_size-byte
 * chunks of word_size-byte elements (introduction paragraph); each chunk is
 * coded as LZ77 items -- a literal (word_size bytes) or a [length, offset]
 * match token (2 bytes) -- with one literal/match flag bit per item.  The
 * match search is the exact longest match over offsets 1..32 (exact-search
 * paragraph), lengths capped at 255 (long-match paragraph); match_level 1
 * adds the hashed long-range candidates with offsets up to 255 (level table
 * and hashed-table paragraphs; codebook notes CN-GPULZ-1).  All-zero chunks
 * cost only their size-table entry (zero-chunk paragraph) and chunks that do
 * not shrink are stored raw (raw-fallback paragraph).
 *
 * Stream layout (all little-endian, no padding, byte-addressed):
 *   [0,32)   header: u32 magic 0x315A4C47 ("GLZ1"), u8 version 1,
 *            u8 word_size, u16 reserved 0, u32 chunk_size, u32 num_chunks,
 *            u64 original_size, u64 payload_bytes
 *   [32, 32+8*num_chunks)  size table: per chunk {u32 flag_size, u32 data_size}
 *            (0,0) = all-zero chunk, no payload;
 *            (0, 0x80000000|b) = raw chunk, payload = its b real bytes;
 *            (F, D), F >= 1 = coded chunk, payload = F flag bytes then D data bytes
 *   then the payloads of all chunks back to back in chunk order.
 * Chunk offsets are not stored: they are the exclusive scan of the payload
 * sizes.  match_level is not stored; a stream decodes the same at any level.
 *
 * Conventions for every entry point:
 *   - Pointers named d_* are device pointers (hipMalloc / torch CUDA tensors)
 *     on the current HIP device; h_* are host pointers.  The caller owns every
 *     buffer.  Apart from the workspace argument the library allocates no
 *     memory and keeps no state between calls.
 *   - All work is enqueued on `stream` (0 = the null stream).  No call
 *     synchronizes the host; launch shapes depend only on the host-visible
 *     arguments, never on data, so calls may be captured into a HIP graph.
 *   - Any byte alignment is accepted for d_in and d_out.
 *   - d_in, d_out and d_workspace must not overlap.
 *   - Host-detectable argument errors return a negative code before anything
 *     is enqueued.  GPULZ_ERR_HIP means a HIP launch failed; the contents of
 *     the output buffers are then undefined.
 */
#ifndef GPULZ_H
#define GPULZ_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#if defined(__GNUC__) || defined(__clang__)
#define GPULZ_API __attribute__((visibility("default")))
#else
#define GPULZ_API
#endif

#define GPULZ_OK 0
#define GPULZ_ERR_INVALID_ARG (-1) /* null pointer, unsupported size, level */
#define GPULZ_ERR_CAPACITY (-2)    /* output or workspace smaller than required */
#define GPULZ_ERR_CORRUPT (-3)     /* host-side header check failed */
#define GPULZ_ERR_HIP (-4)         /* a HIP launch or runtime call failed */

/* Device status codes written to *d_status by gpulz_decode. */
#define GPULZ_STATUS_OK 0u
#define GPULZ_STATUS_CAPACITY 2u /* out_capacity < original_size: nothing decoded */
#define GPULZ_STATUS_CORRUPT 3u  /* malformed stream: output undefined */

/* Supported parameters: chunk_size in {1024, 2048, 4096} (the page lists
 * three sizes, two of which, 2048 and 4096, survive in its text), word_size
 * in {1, 2, 4}, match_level in {0, 1}.  A file written by one supported
 * combination decodes with no parameters. */

/* Worst-case stream size for n_bytes of input: 32 + 8*ceil(n/cs) + n.
 * (The raw fallback bounds each chunk's payload by its own size.)
 * Returns 0 for an unsupported chunk_size. */
GPULZ_API uint64_t gpulz_max_compressed_size(uint64_t n_bytes, uint32_t chunk_size);

/* Device workspace bytes gpulz_encode needs for n_bytes at chunk_size
 * (0 for an unsupported chunk_size).  Independent of word_size and level. */
GPULZ_API uint64_t gpulz_encode_workspace_size(uint64_t n_bytes, uint32_t chunk_size);

/* Device workspace bytes gpulz_decode needs for a stream of in_bytes bytes. */
GPULZ_API uint64_t gpulz_decode_workspace_size(uint64_t in_bytes);

/* Encode n_bytes at d_in into one stream at d_out.
 *   chunk_size, word_size, match_level: see above.  n_bytes may be 0 and
 *     need not be a multiple of word_size or chunk_size: the last chunk is
 *     zero-padded for the search and its real bytes are what round-trips.
 *   d_out / out_capacity: must hold gpulz_max_compressed_size(n, cs) bytes,
 *     else GPULZ_ERR_CAPACITY and nothing is enqueued.  Bytes of d_out past
 *     the stream's length are left untouched.
 *   d_out_bytes: device u64 that receives the stream length once the stream
 *     reaches the end of this call's work.  0 means the call failed on the
 *     device (the assembly's bounded wait for an earlier tile's offset gave
 *     up; never expected): the contents of d_out are then undefined.  A
 *     valid stream is at least 32 bytes long.
 *   d_workspace / workspace_bytes: at least gpulz_encode_workspace_size();
 *     any alignment; its contents on entry do not matter and are clobbered.
 * Output bytes do not depend on workspace contents, stream, or run. */
GPULZ_API int gpulz_encode(const void* d_in, uint64_t n_bytes, uint32_t chunk_size, uint32_t word_size,
                 uint32_t match_level, void* d_out, uint64_t out_capacity, uint64_t* d_out_bytes,
                 void* d_workspace, uint64_t workspace_bytes, hipStream_t stream);

/* Decode the stream of in_bytes bytes at d_in into d_out.
 *   in_bytes: bytes available at d_in (at least the stream's length).
 *   d_out / out_capacity: receives original_size bytes.  If the header asks
 *     for more than out_capacity, *d_status = GPULZ_STATUS_CAPACITY and
 *     nothing is written.
 *   d_out_bytes: device u64, receives original_size, or 0 on any error.
 *   d_status: device u32, receives GPULZ_STATUS_OK / _CAPACITY / _CORRUPT.
 *     On _CORRUPT the output is undefined, but no access ever falls outside
 *     [d_in, d_in+in_bytes) or [d_out, d_out+out_capacity).
 *   d_workspace: at least gpulz_decode_workspace_size(in_bytes) bytes, any
 *     alignment.
 * The stream header is read on the device; nothing waits on the host. */
GPULZ_API int gpulz_decode(const void* d_in, uint64_t in_bytes, void* d_out, uint64_t out_capacity,
                 uint64_t* d_out_bytes, uint32_t* d_status, void* d_workspace,
                 uint64_t workspace_bytes, hipStream_t stream);

/* Largest chunk bound gpulz_decode_noalloc accepts (see there). */
#define GPULZ_DECODE_NOALLOC_MAX_CHUNKS (1ull << 22)

/* gpulz_decode without a workspace argument and without any allocation, for
 * callers that cannot allocate device memory: code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc.  Same arguments and
 * results as gpulz_decode minus d_workspace / workspace_bytes; the
 * workspace is a static device array of the library (about 16 MiB, one per
 * GPU, held from the first call on that GPU until the process ends).
 *   Size limit: the call's chunk bound, min((in_bytes - 32) / 8,
 *     ceil(out_capacity / 1024)), must not exceed
 *     GPULZ_DECODE_NOALLOC_MAX_CHUNKS (4,194,304: e.g. any output of up to
 *     4 GiB), else GPULZ_ERR_CAPACITY and nothing is enqueued.  Pass
 *     out_capacity = the stream's original size (gpulz_stream_info) to keep
 *     the bound tight.
 *   Concurrency: every call on one GPU uses that GPU's one array, so calls
 *     whose work overlaps on one GPU (on different streams, or from several
 *     host threads without ordering) race and give undefined results; calls
 *     ordered on one stream are safe.  Nothing in the array needs to survive
 *     from one call to the next.
 *   Errors: as gpulz_decode; GPULZ_ERR_HIP also if the array's device
 *     address cannot be obtained. */
GPULZ_API int gpulz_decode_noalloc(const void* d_in, uint64_t in_bytes, void* d_out, uint64_t out_capacity,
                                   uint64_t* d_out_bytes, uint32_t* d_status, hipStream_t stream);

/* Host-side header read (no device access): from the first `bytes` (>= 32)
 * bytes of a stream in host memory, return its original size, total stream
 * length, chunk_size and word_size.  GPULZ_ERR_CORRUPT if the header is not
 * a valid stream header; any output pointer may be NULL. */
GPULZ_API int gpulz_stream_info(const void* h_prefix, uint64_t bytes, uint64_t* original_size,
                      uint64_t* stream_bytes, uint32_t* chunk_size, uint32_t* word_size);

#ifdef __cplusplus
}
#endif

#endif /* GPULZ_H */
