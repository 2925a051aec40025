/*
 * gpulz_timing.h -- instrumented variants of the gfx950 LZSS coder entry
 * points, for benchmarks and profilers.
 *
 * Each does exactly the work of its counterpart in gpulz.h (same arguments,
 * same results, same errors) and in addition records ev_start on `stream`
 * immediately before the per-chunk kernel is enqueued and ev_stop
 * immediately after it:
 *   gpulz_encode_timed: around the chunk encode kernel (search, parse,
 *                       size-table rows, payloads into staging slots),
 *                       excluding the compaction kernel that scans the sizes
 *                       and moves the payloads to their stream offsets;
 *   gpulz_decode_timed: around the chunk decode kernel, excluding the kernel
 *                       that checks the header and scans the size table.
 * The caller creates both events (hipEventCreate) and reads them with
 * hipEventElapsedTime after the stream has reached them.  Null events are
 * allowed and are not recorded.
 */
#ifndef GPULZ_TIMING_H
#define GPULZ_TIMING_H

#include "gpulz.h"

#ifdef __cplusplus
extern "C" {
#endif

GPULZ_API int gpulz_encode_timed(const void* d_in, uint64_t n_bytes, uint32_t chunk_size, uint32_t word_size,
                                 uint32_t match_level, void* d_out, uint64_t out_capacity, uint64_t* d_out_bytes,
                                 void* d_workspace, uint64_t workspace_bytes, hipStream_t stream,
                                 hipEvent_t ev_start, hipEvent_t ev_stop);

GPULZ_API int gpulz_decode_timed(const void* d_in, uint64_t in_bytes, void* d_out, uint64_t out_capacity,
                                 uint64_t* d_out_bytes, uint32_t* d_status, void* d_workspace,
                                 uint64_t workspace_bytes, hipStream_t stream, hipEvent_t ev_start,
                                 hipEvent_t ev_stop);

#ifdef __cplusplus
}
#endif

#endif /* GPULZ_TIMING_H */
