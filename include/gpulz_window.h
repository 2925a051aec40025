/* gpulz_window.h -- wider near windows, an encode-side option of the
 * chunked LZSS coder.
 *
 * The stage's exact search covers offsets 1..32.  The GPULZStage page notes
 * that one comparison per element per offset keeps the window from growing
 * far, and that its measured ratio still rose with the window (4.36x at 32,
 * 4.82x at 48, 5.13x at 64; window-width paragraph), which is what led to the
 * hashed level-1 candidates instead.  This entry point runs the same exact
 * search over 48 or 64 offsets so that trade can be measured.  Like
 * match_level it only changes how hard the encoder looks: offsets up to 64
 * fit the token's offset byte, the stream format is unchanged and
 * gpulz_decode reads it as any other stream.
 */
#ifndef GPULZ_WINDOW_H
#define GPULZ_WINDOW_H

#include "gpulz.h"

#ifdef __cplusplus
extern "C" {
#endif

/* gpulz_encode with the near window as a parameter: window in {32, 48, 64}
 * (32 gives exactly gpulz_encode's stream).  Every other argument, buffer
 * size, workspace size (gpulz_encode_workspace_size) and error is as for
 * gpulz_encode; another window returns GPULZ_ERR_INVALID_ARG before
 * anything is enqueued.  The search tables double in size past 32 offsets
 * (64-bit offset masks), so wider windows run at lower occupancy. */
GPULZ_API int gpulz_encode_window(const void* d_in, uint64_t n_bytes, uint32_t chunk_size, uint32_t word_size,
                                  uint32_t match_level, uint32_t window, void* d_out, uint64_t out_capacity,
                                  uint64_t* d_out_bytes, void* d_workspace, uint64_t workspace_bytes,
                                  hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* GPULZ_WINDOW_H */
