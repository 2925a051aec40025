/* gpulz_baseline.h -- a measured baseline decoder of the chunked LZSS coder.
 *
 * The GPULZStage page says upstream GPULZ decodes a whole chunk on a single
 * thread, replaying its items in order, and that a block-parallel decode is
 * ~2.4x faster at chunk_size 2048 / word_size 4 and ~4x at 4096 / 4 (its
 * block-parallel decode paragraph).  This entry point is that one-thread-per-
 * chunk decode, built the same way as gpulz_decode otherwise (device-side
 * header and size-table scan), so the two can be timed side by side.  It is a
 * baseline, not a faster path.
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

#ifdef __cplusplus
}
#endif

#endif /* GPULZ_BASELINE_H */
