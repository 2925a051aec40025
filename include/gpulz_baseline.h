/* gpulz_baseline.h -- measured baselines of the chunked LZSS coder: the
 * upstream shapes the GPULZStage page compares its own design against.
 * Baselines, not faster paths.
 *
 * Decode: the page says upstream GPULZ decodes a whole chunk on a single
 * thread, replaying its items in order, and that a block-parallel decode is
 * ~2.4x faster at chunk_size 2048 / word_size 4 and ~4x at 4096 / 4 (its
 * block-parallel decode paragraph).  gpulz_decode_one_thread_per_chunk is
 * that decode, built the same way as gpulz_decode otherwise (device-side
 * header and size-table scan), so the two can be timed side by side.
 *
 * Encode: per the page, upstream's match search moves its candidate pointer
 * forward with each comparison, so starts passed while a match is extended
 * are never tried; the exact search costs less and compresses better (exact
 * longest-match search paragraph).
 * gpulz_encode_advancing_search is the level-0 coder with that search in
 * place of the exact one, read as: for position p the pointer w walks the 32
 * elements before p (not before the chunk start), one comparison per step of
 * x[w] against x[p + len], the element the partial match started at w - len
 * needs next; equal grows the partial match, unequal drops it and spends w;
 * the longest partial match seen is taken, the first on ties (so L <= 32).
 * The greedy parse, item forms, raw and zero chunks are unchanged, so
 * gpulz_decode reads its streams.
 */
#ifndef GPULZ_BASELINE_H
#define GPULZ_BASELINE_H

#include "gpulz.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Same arguments, results, errors and workspace (gpulz_decode_workspace_size)
 * as gpulz_decode; identical output and status for every stream.
 * ev_start / ev_stop: optional HIP events (may be null) recorded on `stream`
 * around the per-chunk decode kernel only. */
GPULZ_API int gpulz_decode_one_thread_per_chunk(const void* d_in, uint64_t in_bytes, void* d_out,
                                                uint64_t out_capacity, uint64_t* d_out_bytes, uint32_t* d_status,
                                                void* d_workspace, uint64_t workspace_bytes, hipStream_t stream,
                                                hipEvent_t ev_start, hipEvent_t ev_stop);

/* Same arguments, results, errors and workspace (gpulz_encode_workspace_size)
 * as gpulz_encode at match_level 0, with the search above: the stream the
 * oracle's advancing-search encoder gives, byte for byte.
 * ev_start / ev_stop: optional HIP events (may be null) recorded on `stream`
 * around the per-chunk search-and-parse kernel only (not the assembly). */
GPULZ_API int gpulz_encode_advancing_search(const void* d_in, uint64_t n_bytes, uint32_t chunk_size,
                                            uint32_t word_size, void* d_out, uint64_t out_capacity,
                                            uint64_t* d_out_bytes, void* d_workspace, uint64_t workspace_bytes,
                                            hipStream_t stream, hipEvent_t ev_start, hipEvent_t ev_stop);

#ifdef __cplusplus
}
#endif

#endif /* GPULZ_BASELINE_H */
