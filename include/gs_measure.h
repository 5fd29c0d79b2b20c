/*
 * gs_measure.h -- measurement hooks of libgsraster (gs_raster.h holds the method's calls).
 */
#ifndef GS_MEASURE_H
#define GS_MEASURE_H

#include <stdint.h>

#include "gs_raster.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Device time of one of the library's kernels, for comparing a kernel's rate with its
 * roofline.  Not part of the method, and the one piece of process-wide state of the
 * library's measured kernels: while the timer is armed, every launch of the named kernel,
 * from any thread and on any stream, records two events, so it is for single-threaded
 * measurement runs; while it is not armed a launch pays one atomic load.
 *
 * gs_kernel_timer_start arms the timer for `kernel`, one of "k_project", "k_render_fwd",
 * "k_render_bwd", "k_project_bwd", "k_densify_emit", "k_adam_q16" (the single kernel behind
 * gs_project, gs_render_fwd, the two halves of gs_render_bwd, the writing pass of gs_densify
 * and gs_adam_q16).  From then on each launch of that kernel is bracketed
 * by two HIP events recorded on the caller's stream; the events are created on first use
 * and kept by the library until the process ends.
 * gs_kernel_timer_stop disarms the timer, waits for the last recorded event and writes the
 * number of timed launches and the sum of their durations in milliseconds.
 * One timer per process; arming it while it is armed is an error.
 * Errors: INVALID_ARG (unknown kernel name, already armed / not armed, NULL outputs),
 * HIP (an event could not be created, recorded or read).
 */
gs_status gs_kernel_timer_start(const char* kernel);
gs_status gs_kernel_timer_stop(int64_t* launches, double* total_ms);

#ifdef __cplusplus
}
#endif

#endif /* GS_MEASURE_H */
