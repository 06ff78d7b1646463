/*
 * lowram_timing.h — a measurement entry point of the LowRAM library (not
 * part of the method).
 *
 * lowram_decode_attn_timed is lowram_decode_attn (include/lowram.h; same
 * arguments, checks, results and errors) that also records two caller
 * events on `hip_stream`: `before_event` right before the call's body-row
 * kernel (the rebuild, rotation, scores and predictor hidden layer of the
 * attended body rows) and `after_event` right after it, so the caller can
 * time that one kernel with hipEventElapsedTime while the rest of the call
 * runs as usual.  Both are hipEvent_t handles created by the caller with
 * timing enabled and kept alive until the stream has passed them; both are
 * required (LOWRAM_E_ARG otherwise).  Nothing is kept between calls.  A
 * failed event record returns LOWRAM_E_HIP.
 */
#ifndef LOWRAM_TIMING_H
#define LOWRAM_TIMING_H

#include "lowram.h"

#ifdef __cplusplus
extern "C" {
#endif

int32_t lowram_decode_attn_timed(const lowram_shape *shape, int32_t layer,
                                 const void *q, const lowram_cache *cache,
                                 const int32_t *subset_off, const int32_t *subset_idx,
                                 void *out, float *lse_out,
                                 void *workspace, size_t workspace_bytes,
                                 void *hip_stream, void *before_event,
                                 void *after_event);

#ifdef __cplusplus
}
#endif
#endif /* LOWRAM_TIMING_H */
