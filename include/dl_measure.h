/*
 * dl_measure.h — measurement aids of libdl.so, not part of the decode layer step.
 *
 * These calls exist to time the step and to bound what its kernels can reach on the device; no step
 * entry point needs them.  Conventions as in dl.h (device pointers, enqueue only on `stream`, negative
 * dl_status on error, dl_last_error()).
 */
#ifndef DL_MEASURE_H
#define DL_MEASURE_H

#include "dl.h"

#ifdef __cplusplus
extern "C" {
#endif

/* ---------------------------------------------------------------- measurement
 * When enabled, every dl_layer_step records a HIP event on its stream at each phase boundary:
 *   0 indexer + top-k   1 attention   2 W_UV + W_O (+ activation split)   3 router
 *   4 dispatch plan + split of h   5 expert gate/up (one kernel)   6 split of Z
 *   7 expert down (one kernel)   8 combine
 * When the expert FFN runs as one kernel (dl_profile_ffn_fused), phase 5 holds all of it (gate/up, split
 * of Z and down) and phases 6 and 7 hold no work.
 * dl_profile_read waits for the recorded steps, adds each phase's elapsed milliseconds into
 * ms_sum[DL_N_PHASES], stores the number of steps in *steps and forgets them.  Measurement only:
 * single host thread, events are created on first use and kept until dl_profile_enable(0). */
#define DL_N_PHASES 9
int dl_profile_enable(int on);
int dl_profile_read(double *ms_sum, int64_t *steps);
/* How the most recent expert FFN (of any entry point, in this process) ran: 1 as one kernel (gate/up, the split
 * of Z and down in a single launch: FP8 weights in DL_LAYOUT_TILES), 0 as three kernels, -1 before the first. */
int dl_profile_ffn_fused(void);

/* Measurement aid, not part of the step: enqueue one streaming read of the first *bytes_read bytes of
 * the device buffer buf (16-byte non-temporal loads, each wave of a full-device grid reading its own
 * contiguous range, as the expert GEMV streams its weights); *bytes_read (host) receives the count,
 * which rounds `bytes` down to whole rounds of the grid.  Timing it with events on `stream` gives the
 * HBM read rate reachable for the buffer's contents.  DL_ERR_SHAPE if bytes is below one round. */
int dl_probe_read(const void *buf, size_t bytes, size_t *bytes_read, void *stream);

/* Measurement aid, not part of the step (Kiln's "null" kernel, which does no work and so exposes fixed costs:
 * "What moved the number from 19.4 to 122.9 tokens a second?"): enqueue n_kernels launches, one after
 * another on `stream`, of a kernel with `blocks` workgroups of 256 threads that do nothing.  Timing them
 * with events gives the fixed cost of a dependent launch, the floor under every phase of the step.
 * Limits 1 <= n_kernels <= 1024, 1 <= blocks <= 65536 (else DL_ERR_SHAPE). */
int dl_probe_null(int32_t n_kernels, int32_t blocks, void *stream);

#ifdef __cplusplus
}
#endif
#endif /* DL_MEASURE_H */
