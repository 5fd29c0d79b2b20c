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
 * and gs_adam_q16) or "k_onesweep_u64" (each digit pass of gs_sort_keys, gs_sort_ids and
 * gs_sort_keys_noalloc).  From then on each launch of that kernel is bracketed
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

/*
 * Memory ceilings: kernels that perform only the loads and stores of a kernel of the
 * method, in its layout, so that their time bounds the kernel's from below.  They compute
 * nothing of the method; their outputs hold no result.
 *
 * gs_measure_project_io: the loads and stores of gs_project's kernel for n Gaussians
 * (inputs and `out` as for gs_project: the same arrays, read and written with the same
 * widths, strides and grid), with none of its arithmetic.  Every array of `out` is
 * overwritten with unspecified values.  Errors: INVALID_ARG (n < 0, sh_degree outside
 * 0..3, a NULL pointer), OVERFLOW (n >= 2^32), HIP.
 *
 * gs_measure_scatter_io: for i < n, reads keys[i], vals[i] and dest[i] (device arrays of
 * n elements, 1024 consecutive elements per workgroup, four per lane, as a digit pass of the
 * pair sort reads its partition) and writes vals[i] + (uint32_t)keys[i] to out[dest[i]]
 * (out: n device words); a dest[i] >= n is skipped.  With the elements arranged in the
 * order in which a digit pass writes them and dest the sorted positions, its time bounds
 * that pass's (which moves 4 fewer bytes per element: it computes the destinations).
 * Errors: INVALID_ARG (n < 0, a NULL pointer), OVERFLOW (n > 2^32 - 1), HIP.
 */
gs_status gs_measure_project_io(int64_t n, const float* means, const float* scales, const float* quats,
                                const float* opacities, const float* sh, int32_t sh_degree, gs_projected out,
                                void* stream);
gs_status gs_measure_scatter_io(int64_t n, const uint64_t* keys, const uint32_t* vals, const uint32_t* dest,
                                uint32_t* out, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* GS_MEASURE_H */
