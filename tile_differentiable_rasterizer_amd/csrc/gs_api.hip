// gs_api.hip -- the extern "C" boundary of libgsraster: argument validation (before any
// HIP call), the workspace layout, and kernel launches on the caller's stream.  Every
// buffer belongs to the caller; nothing here allocates.
#include <math.h>
#include <string.h>

#include <atomic>
#include <mutex>
#include <vector>

#include "gs_device.h"
#include "../../include/gs_measure.h"

namespace gs {
hipError_t launch_project(int64_t n, const float* means, const float* scales, const float* quats,
                          const float* opac, const float* sh, int L, const DevCamera& cam,
                          const gs_projected& out, hipStream_t s);
hipError_t launch_project_bwd(int64_t n, const float* means, const float* scales, const float* quats,
                              const float* sh, int L, const DevCamera& cam, const gs_projected& proj,
                              const gs_grads& gr, float* accum, int32_t* denom, hipStream_t s);
size_t bin_workspace_bytes(int64_t n, int64_t n_pairs);
hipError_t launch_bin_count(int64_t n, const uint32_t* n_tiles, const uint32_t* rows, void* ws, hipStream_t s);
uint64_t* bin_report_ptr(int64_t n, void* ws);
bool bin_report(uint64_t report, int64_t* P, bool* large);
hipError_t launch_bin_depth(int64_t n, const gs_projected& proj, uint64_t* digit_counts, void* ws, hipStream_t s);
hipError_t launch_bin_emit(int64_t n, int64_t P, bool large, const gs_projected& proj, int tiles_x, int tile_bits,
                           uint64_t* digit_counts, void* ws, uint64_t* keys, uint32_t* vals, hipStream_t s);
size_t sort_workspace_bytes(int64_t n_pairs, int64_t num_tiles, int sorted_low_bits);
int sort_significant_bits(int64_t num_tiles);
hipError_t launch_sort(int64_t P, int64_t num_tiles, uint64_t* keys, uint32_t* vals, uint64_t* keys_tmp,
                       uint32_t* vals_tmp, int64_t* ranges, int32_t* order, int sorted_low_bits,
                       const uint64_t* digit_counts, int32_t* result_in_tmp, void* ws, hipStream_t s,
                       bool ids_only);
hipError_t launch_fill_u32(void* p, int64_t count, uint32_t v, hipStream_t s);
hipError_t launch_project_io(int64_t n, const float* means, const float* scales, const float* quats,
                             const float* opac, const float* sh, int L, const gs_projected& out, hipStream_t s);
hipError_t launch_scatter_io(int64_t n, const uint64_t* keys, const uint32_t* vals, const uint32_t* dest,
                             uint32_t* out, hipStream_t s);
size_t densify_workspace_bytes(int64_t n);
hipError_t launch_quantize_sh(int64_t U, const float* sh, int bits, void* codes, float* bounds, hipStream_t s);
hipError_t launch_project_qsh(int64_t n, const float* means, const float* scales, const float* quats,
                              const float* opac, const void* shq, const float* shb, int bits, int L,
                              const DevCamera& cam, const gs_projected& out, hipStream_t s);
hipError_t launch_adam_q16(int64_t U, float* params, const float* grads, uint32_t* state, float* bounds,
                           const gs_adam_params& p, hipStream_t s);
hipError_t launch_fpbo_pack(int64_t U, const float* params, uint16_t* state, float* bounds, hipStream_t s);
hipError_t launch_adam_fpbo(int64_t U, uint16_t* state, float* bounds, const float* grads, float* params_out,
                            const gs_adam_params& p, hipStream_t s);
hipError_t launch_densify_count(int64_t n, const float* scales, const float* opac, const float* accum,
                                const int32_t* denom, const gs_densify_params& q, void* ws, uint64_t** total,
                                hipStream_t s);
hipError_t launch_densify_emit(int64_t n, const float* means, const float* scales, const float* quats,
                               const float* opac, const float* sh, int L, const float* accum, const int32_t* denom,
                               const float* normals, const gs_densify_params& q, const void* ws, float* om,
                               float* os, float* oq, float* oo, float* osh, uint32_t* osrc, hipStream_t s);
hipError_t launch_render_fwd(const gs_projected& proj, const uint32_t* vals, uint32_t id_max, const int64_t* ranges,
                             const int32_t* order, const DevCamera& cam, const float bg[3], float* image,
                             float* final_T, uint32_t* n_contrib, hipStream_t s);
hipError_t launch_render_bwd(const gs_projected& proj, const uint32_t* vals, uint32_t id_max, const int64_t* ranges,
                             const int32_t* order, const DevCamera& cam, const float bg[3], const float* final_T,
                             const uint32_t* n_contrib, const float* dL, float* gscreen, hipStream_t s);
}  // namespace gs

using namespace gs;

namespace {

constexpr int64_t kMaxGaussians = (int64_t)1 << 32;  // ids are uint32

bool camera_ok(const gs_camera* c) {
  if (!c) return false;
  if (!(c->fx > 0.0f) || !(c->fy > 0.0f) || !(c->near_z > 0.0f)) return false;
  if (c->width <= 0 || c->height <= 0) return false;
  return true;
}

bool camera_fits(const gs_camera* c) { return c->width <= 65535 && c->height <= 65535; }

DevCamera dev_camera(const gs_camera* c) {
  DevCamera d;
  for (int i = 0; i < 9; ++i) d.R[i] = c->R[i];
  for (int i = 0; i < 3; ++i) d.t[i] = c->t[i];
  d.fx = c->fx; d.fy = c->fy; d.cx = c->cx; d.cy = c->cy; d.near_z = c->near_z;
  for (int i = 0; i < 3; ++i) d.campos[i] = -(d.R[i] * d.t[0] + d.R[3 + i] * d.t[1] + d.R[6 + i] * d.t[2]);
  d.width = c->width; d.height = c->height;
  d.tiles_x = (c->width + kTile - 1) / kTile;
  d.tiles_y = (c->height + kTile - 1) / kTile;
  return d;
}

bool projected_ok(const gs_projected& p) {
  return p.rec && p.depth && p.rect && p.n_tiles && p.clamp && p.runs && p.rows;
}

gs_status hip_status(hipError_t e) { return e == hipSuccess ? GS_OK : GS_ERR_HIP; }

// Kernel timer: while armed for one kernel, every launch of that kernel is bracketed by
// two HIP events recorded on its launch stream.  The events are created on first use and
// kept for the life of the process (they are reused by later arming).
enum TimedKernel { kNone = 0, kProject, kRenderFwd, kRenderBwd, kProjectBwd, kDensifyEmit, kAdamQ16, kSortPass, kAdamFpbo };

struct KernelTimer {
  std::mutex mu;
  std::atomic<int> armed_any{0};  // read without the lock on every launch
  TimedKernel armed = kNone;
  std::vector<hipEvent_t> events;  // pairs: start, stop
  size_t used = 0;                 // events recorded since arming
  bool failed = false;
};

KernelTimer& timer() {
  static KernelTimer t;
  return t;
}

TimedKernel timed_kernel_id(const char* name) {
  if (!name) return kNone;
  if (!strcmp(name, "k_project")) return kProject;
  if (!strcmp(name, "k_render_fwd")) return kRenderFwd;
  if (!strcmp(name, "k_render_bwd")) return kRenderBwd;
  if (!strcmp(name, "k_project_bwd")) return kProjectBwd;
  if (!strcmp(name, "k_densify_emit")) return kDensifyEmit;
  if (!strcmp(name, "k_adam_q16")) return kAdamQ16;
  if (!strcmp(name, "k_adam_fpbo")) return kAdamFpbo;
  if (!strcmp(name, "k_onesweep_u64")) return kSortPass;
  return kNone;
}

// Records one event of the pair for kernel k when the timer is armed for it.  While it is
// not armed a launch pays one relaxed atomic load and takes no lock.
void timer_mark(TimedKernel k, hipStream_t s) {
  KernelTimer& t = timer();
  if (!t.armed_any.load(std::memory_order_acquire)) return;
  std::lock_guard<std::mutex> g(t.mu);
  if (t.armed != k || t.failed) return;
  if (t.used == t.events.size()) {
    hipEvent_t e;
    if (hipEventCreate(&e) != hipSuccess) { t.failed = true; return; }
    t.events.push_back(e);
  }
  if (hipEventRecord(t.events[t.used], s) != hipSuccess) { t.failed = true; return; }
  ++t.used;
}

// Launches through f with the timer's events around it.
template <class F>
hipError_t timed(TimedKernel k, hipStream_t s, F&& f) {
  timer_mark(k, s);
  const hipError_t e = f();
  timer_mark(k, s);
  return e;
}

}  // namespace

namespace gs {
void mark_sort_pass(hipStream_t s) { timer_mark(kSortPass, s); }
}  // namespace gs

extern "C" {

size_t gs_densify_workspace_bytes(int64_t n) { return n < 0 ? 0 : densify_workspace_bytes(n); }

gs_status gs_densify(int64_t n, const float* means, const float* scales, const float* quats, const float* opacities,
                     const float* sh, int32_t sh_degree, const float* densify_accum, const int32_t* densify_denom,
                     const float* normals, const gs_densify_params* params, float* out_means, float* out_scales,
                     float* out_quats, float* out_opacities, float* out_sh, uint32_t* out_src, int64_t capacity,
                     int64_t* n_out, void* workspace, size_t workspace_bytes, void* stream) {
  if (n < 0 || capacity < 0 || !params || !n_out || sh_degree < 0 || sh_degree > 3) return GS_ERR_INVALID_ARG;
  const gs_densify_params q = *params;
  if (q.split_n < 2 || q.split_n > 4 || !(q.split_shrink > 0.0f)) return GS_ERR_INVALID_ARG;
  if (n >= kMaxGaussians) return GS_ERR_OVERFLOW;
  if (n > 0 && (!means || !scales || !quats || !opacities || !sh || !densify_accum || !densify_denom || !normals))
    return GS_ERR_INVALID_ARG;
  if (out_means && (!out_scales || !out_quats || !out_opacities || !out_sh || !out_src)) return GS_ERR_INVALID_ARG;
  if (!workspace || workspace_bytes < densify_workspace_bytes(n)) return GS_ERR_WORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  uint64_t* dtotal = nullptr;
  if (launch_densify_count(n, scales, opacities, densify_accum, densify_denom, q, workspace, &dtotal, s) !=
      hipSuccess)
    return GS_ERR_HIP;
  uint64_t total = 0;
  if (hipMemcpyAsync(&total, dtotal, sizeof total, hipMemcpyDeviceToHost, s) != hipSuccess) return GS_ERR_HIP;
  if (hipStreamSynchronize(s) != hipSuccess) return GS_ERR_HIP;
  if (total >= (uint64_t)kMaxGaussians) return GS_ERR_OVERFLOW;
  *n_out = (int64_t)total;
  if (!out_means) return GS_OK;
  if ((int64_t)total > capacity) return GS_ERR_CAPACITY;
  return hip_status(timed(kDensifyEmit, s, [&] {
    return launch_densify_emit(n, means, scales, quats, opacities, sh, sh_degree, densify_accum, densify_denom,
                               normals, q, workspace, out_means, out_scales, out_quats, out_opacities, out_sh,
                               out_src, s);
  }));
}

gs_status gs_adam_q16(int64_t n, float* params, const float* grads, uint32_t* state, float* bounds,
                      const gs_adam_params* hyper, void* stream) {
  if (n < 0 || !hyper) return GS_ERR_INVALID_ARG;
  const gs_adam_params p = *hyper;
  if (p.step < 1 || !(p.beta1 >= 0.0f && p.beta1 < 1.0f) || !(p.beta2 >= 0.0f && p.beta2 < 1.0f))
    return GS_ERR_INVALID_ARG;
  if (n > 0 && (!params || !grads || !state || !bounds)) return GS_ERR_INVALID_ARG;
  if (n >= ((int64_t)1 << 40)) return GS_ERR_OVERFLOW;
  hipStream_t s = static_cast<hipStream_t>(stream);
  return hip_status(timed(kAdamQ16, s, [&] { return launch_adam_q16(n, params, grads, state, bounds, p, s); }));
}

namespace {
bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }
}  // namespace

gs_status gs_fpbo_pack(int64_t n, const float* params, uint16_t* state, float* bounds, void* stream) {
  if (n < 0) return GS_ERR_INVALID_ARG;
  if (n > 0 && (!params || !state || !bounds)) return GS_ERR_INVALID_ARG;
  if (!aligned(params, 16) || !aligned(state, 8) || !aligned(bounds, 8)) return GS_ERR_INVALID_ARG;
  if (n >= ((int64_t)1 << 40)) return GS_ERR_OVERFLOW;
  return hip_status(launch_fpbo_pack(n, params, state, bounds, static_cast<hipStream_t>(stream)));
}

gs_status gs_adam_fpbo(int64_t n, uint16_t* state, float* bounds, const float* grads, float* params_out,
                       const gs_adam_params* hyper, void* stream) {
  if (n < 0 || !hyper) return GS_ERR_INVALID_ARG;
  const gs_adam_params p = *hyper;
  if (p.step < 1 || !(p.beta1 >= 0.0f && p.beta1 < 1.0f) || !(p.beta2 >= 0.0f && p.beta2 < 1.0f))
    return GS_ERR_INVALID_ARG;
  if (n > 0 && (!state || !bounds || !grads)) return GS_ERR_INVALID_ARG;
  if (!aligned(grads, 16) || !aligned(params_out, 16) || !aligned(state, 8) || !aligned(bounds, 8))
    return GS_ERR_INVALID_ARG;
  if (n >= ((int64_t)1 << 40)) return GS_ERR_OVERFLOW;
  hipStream_t s = static_cast<hipStream_t>(stream);
  return hip_status(
      timed(kAdamFpbo, s, [&] { return launch_adam_fpbo(n, state, bounds, grads, params_out, p, s); }));
}

const char* gs_status_string(gs_status s) {
  switch (s) {
    case GS_OK: return "ok";
    case GS_ERR_INVALID_ARG: return "invalid argument";
    case GS_ERR_CAPACITY: return "pair buffer too small";
    case GS_ERR_OVERFLOW: return "size overflow";
    case GS_ERR_HIP: return "HIP error";
    case GS_ERR_WORKSPACE: return "workspace too small";
    default: return "unknown status";
  }
}

size_t gs_workspace_bytes(int64_t n, int64_t pair_capacity, int32_t num_tiles) {
  if (n < 0 || pair_capacity < 0 || num_tiles < 1) return 0;
  const size_t a = bin_workspace_bytes(n, pair_capacity);
  const size_t b = sort_workspace_bytes(pair_capacity, num_tiles, 0);
  return a > b ? a : b;
}

gs_status gs_project(int64_t n, const float* means, const float* scales, const float* quats,
                     const float* opacities, const float* sh, int32_t sh_degree, const gs_camera* cam,
                     gs_projected out, void* stream) {
  if (n < 0 || sh_degree < 0 || sh_degree > 3 || !camera_ok(cam)) return GS_ERR_INVALID_ARG;
  if (n >= kMaxGaussians || !camera_fits(cam)) return GS_ERR_OVERFLOW;
  if (n == 0) return GS_OK;
  if (!means || !scales || !quats || !opacities || !sh || !projected_ok(out)) return GS_ERR_INVALID_ARG;
  const DevCamera d = dev_camera(cam);
  hipStream_t s = static_cast<hipStream_t>(stream);
  return hip_status(timed(kProject, s, [&] {
    return launch_project(n, means, scales, quats, opacities, sh, sh_degree, d, out, s);
  }));
}

gs_status gs_quantize_sh(int64_t n, const float* sh, int32_t sh_degree, int32_t bits, void* codes, float* bounds,
                         void* stream) {
  if (n < 0 || sh_degree < 0 || sh_degree > 3 || (bits != 8 && bits != 16)) return GS_ERR_INVALID_ARG;
  if (n >= kMaxGaussians) return GS_ERR_OVERFLOW;
  if (n == 0) return GS_OK;
  if (!sh || !codes || !bounds) return GS_ERR_INVALID_ARG;
  const int64_t units = n * 3 * (int64_t)(sh_degree + 1) * (sh_degree + 1);
  return hip_status(launch_quantize_sh(units, sh, bits, codes, bounds, static_cast<hipStream_t>(stream)));
}

gs_status gs_project_qsh(int64_t n, const float* means, const float* scales, const float* quats,
                         const float* opacities, const void* sh_codes, const float* sh_bounds, int32_t sh_bits,
                         int32_t sh_degree, const gs_camera* cam, gs_projected out, void* stream) {
  if (n < 0 || sh_degree < 0 || sh_degree > 3 || (sh_bits != 8 && sh_bits != 16) || !camera_ok(cam))
    return GS_ERR_INVALID_ARG;
  if (n >= kMaxGaussians || !camera_fits(cam)) return GS_ERR_OVERFLOW;
  if (n == 0) return GS_OK;
  if (!means || !scales || !quats || !opacities || !sh_codes || !sh_bounds || !projected_ok(out))
    return GS_ERR_INVALID_ARG;
  const DevCamera d = dev_camera(cam);
  hipStream_t s = static_cast<hipStream_t>(stream);
  return hip_status(timed(kProject, s, [&] {
    return launch_project_qsh(n, means, scales, quats, opacities, sh_codes, sh_bounds, sh_bits, sh_degree, d, out,
                              s);
  }));
}

// The event gs_bin_tiles waits on for its pair-count copy: one per host thread and GPU,
// created on the thread's first binning call on that GPU and kept, so a frame creates
// nothing.
hipError_t count_event(hipStream_t s, hipEvent_t* ev) {
  constexpr int kMaxDevices = 64;
  thread_local hipEvent_t events[kMaxDevices] = {};
  int dev = 0;
  hipError_t e = hipStreamGetDevice(s, &dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  if (!events[dev]) {
    int cur = 0;
    if ((e = hipGetDevice(&cur)) != hipSuccess) return e;
    if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return e;
    hipEvent_t created = nullptr;
    e = hipEventCreateWithFlags(&created, hipEventDisableTiming);
    const hipError_t r = cur != dev ? hipSetDevice(cur) : hipSuccess;
    if (e != hipSuccess) return e;
    if (r != hipSuccess) return r;
    events[dev] = created;
  }
  *ev = events[dev];
  return hipSuccess;
}

gs_status gs_bin_tiles(int64_t n, gs_projected proj, const gs_camera* cam, uint64_t* keys, uint32_t* vals,
                       int64_t capacity, int64_t* n_pairs, uint64_t* tile_digit_counts, void* workspace,
                       size_t workspace_bytes, void* stream) {
  if (n < 0 || capacity < 0 || !n_pairs || !camera_ok(cam)) return GS_ERR_INVALID_ARG;
  if (n >= kMaxGaussians || !camera_fits(cam)) return GS_ERR_OVERFLOW;
  if (n > 0 && !projected_ok(proj)) return GS_ERR_INVALID_ARG;
  if (keys && !vals) return GS_ERR_INVALID_ARG;
  if (!workspace || workspace_bytes < bin_workspace_bytes(n, 0)) return GS_ERR_WORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const DevCamera d = dev_camera(cam);
  const int tile_bits = sort_significant_bits((int64_t)d.tiles_x * d.tiles_y) - 32;
  uint64_t* dc = keys ? tile_digit_counts : nullptr;
  if (launch_bin_count(n, proj.n_tiles, proj.rows, workspace, s) != hipSuccess) return GS_ERR_HIP;
  // the report word: P, with a flag bit that the call strips (bin_report)
  const uint64_t* dP = bin_report_ptr(n, workspace);
  int64_t P = 0;
  bool large = false;
  if (keys) {
    // the count lands in the caller's word and the depth phase, which needs no host value,
    // is queued behind the copy: with page-locked memory the GPU runs the depth phase while
    // the host waits for the copy alone; into pageable memory the copy completes before
    // hipMemcpyAsync returns (HIP performs it synchronously), so the same results follow
    // without the overlap
    hipEvent_t ev;
    hipError_t e = count_event(s, &ev);
    if (e == hipSuccess) e = hipMemcpyAsync(n_pairs, dP, sizeof(int64_t), hipMemcpyDeviceToHost, s);
    if (e == hipSuccess) e = hipEventRecord(ev, s);
    if (e == hipSuccess) e = launch_bin_depth(n, proj, dc, workspace, s);
    if (e == hipSuccess) e = hipEventSynchronize(ev);
    if (e != hipSuccess) return GS_ERR_HIP;
    if (!bin_report((uint64_t)*n_pairs, &P, &large)) return GS_ERR_OVERFLOW;  // a count past 2^62
    *n_pairs = P;
  } else {
    uint64_t report = 0;
    if (hipMemcpyAsync(&report, dP, sizeof report, hipMemcpyDeviceToHost, s) != hipSuccess) return GS_ERR_HIP;
    if (hipStreamSynchronize(s) != hipSuccess) return GS_ERR_HIP;
    if (!bin_report(report, &P, &large)) return GS_ERR_OVERFLOW;
    *n_pairs = P;
    return GS_OK;
  }
  if (P > capacity) return GS_ERR_CAPACITY;
  if (workspace_bytes < bin_workspace_bytes(n, P)) return GS_ERR_WORKSPACE;
  return hip_status(launch_bin_emit(n, P, large, proj, d.tiles_x, tile_bits, dc, workspace, keys, vals, s));
}

gs_status gs_sort_keys(int64_t n_pairs, int32_t num_tiles, int32_t sorted_low_bits, uint64_t* keys, uint32_t* vals,
                       uint64_t* keys_tmp, uint32_t* vals_tmp, int64_t* tile_ranges, int32_t* tile_order,
                       const uint64_t* digit_counts, int32_t* result_in_tmp, void* workspace, size_t workspace_bytes,
                       void* stream) {
  if (n_pairs < 0 || num_tiles < 1 || !tile_ranges || sorted_low_bits < 0 || sorted_low_bits > 64)
    return GS_ERR_INVALID_ARG;
  if (n_pairs > 0 && (!keys || !vals || !keys_tmp || !vals_tmp)) return GS_ERR_INVALID_ARG;
  if (n_pairs >= ((int64_t)1 << 62)) return GS_ERR_OVERFLOW;
  if (!workspace || workspace_bytes < sort_workspace_bytes(n_pairs, num_tiles, sorted_low_bits))
    return GS_ERR_WORKSPACE;
  return hip_status(launch_sort(n_pairs, num_tiles, keys, vals, keys_tmp, vals_tmp, tile_ranges, tile_order,
                                sorted_low_bits, digit_counts, result_in_tmp, workspace,
                                static_cast<hipStream_t>(stream), false));
}

gs_status gs_sort_ids(int64_t n_pairs, int32_t num_tiles, int32_t sorted_low_bits, uint64_t* keys, uint32_t* vals,
                      uint64_t* keys_tmp, uint32_t* vals_tmp, int64_t* tile_ranges, int32_t* tile_order,
                      const uint64_t* digit_counts, int32_t* result_in_tmp, void* workspace, size_t workspace_bytes,
                      void* stream) {
  if (n_pairs < 0 || num_tiles < 1 || !tile_ranges || sorted_low_bits < 0 || sorted_low_bits > 64 || !result_in_tmp)
    return GS_ERR_INVALID_ARG;
  if (n_pairs > 0 && (!keys || !vals || !keys_tmp || !vals_tmp)) return GS_ERR_INVALID_ARG;
  if (n_pairs >= ((int64_t)1 << 62)) return GS_ERR_OVERFLOW;
  if (!workspace || workspace_bytes < sort_workspace_bytes(n_pairs, num_tiles, sorted_low_bits))
    return GS_ERR_WORKSPACE;
  return hip_status(launch_sort(n_pairs, num_tiles, keys, vals, keys_tmp, vals_tmp, tile_ranges, tile_order,
                                sorted_low_bits, digit_counts, result_in_tmp, workspace,
                                static_cast<hipStream_t>(stream), true));
}

}  // extern "C"

namespace {

// Scratch of gs_sort_keys_noalloc: a fixed device array, one copy per GPU, held until the
// process ends.  Host code never passes `scratch` itself (its host-side name is not a
// device address): sort_scratch() looks up this GPU's address once, with the GPU current.
static __device__ __align__(256) unsigned char scratch[GS_SORT_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;

// Device address of `scratch` on the GPU that `stream` belongs to (looked up on the first
// call on that GPU, with it current, and kept).
hipError_t sort_scratch(hipStream_t stream, void** out) {
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = 0;
  hipError_t e = hipStreamGetDevice(stream, &dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> g(mu);
  if (!addr[dev]) {
    int cur = 0;
    e = hipGetDevice(&cur);
    if (e != hipSuccess) return e;
    if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return e;
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    const hipError_t r = cur != dev ? hipSetDevice(cur) : hipSuccess;
    if (e != hipSuccess) return e;
    if (r != hipSuccess) return r;
    if (!p) return hipErrorInvalidSymbol;
    addr[dev] = p;
  }
  *out = addr[dev];
  return hipSuccess;
}

}  // namespace

extern "C" {

gs_status gs_sort_keys_noalloc(int64_t n_pairs, int32_t num_tiles, int32_t sorted_low_bits, uint64_t* keys,
                               uint32_t* vals, uint64_t* keys_tmp, uint32_t* vals_tmp, int64_t* tile_ranges,
                               int32_t* tile_order, const uint64_t* digit_counts, int32_t* result_in_tmp,
                               void* stream) {
  if (n_pairs < 0 || num_tiles < 1 || !tile_ranges || sorted_low_bits < 0 || sorted_low_bits > 64)
    return GS_ERR_INVALID_ARG;
  if (n_pairs > 0 && (!keys || !vals || !keys_tmp || !vals_tmp)) return GS_ERR_INVALID_ARG;
  if (n_pairs >= ((int64_t)1 << 62)) return GS_ERR_OVERFLOW;
  if (sort_workspace_bytes(n_pairs, num_tiles, sorted_low_bits) > (size_t)GS_SORT_NOALLOC_SCRATCH_BYTES)
    return GS_ERR_WORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  void* ws = nullptr;
  if (sort_scratch(s, &ws) != hipSuccess) return GS_ERR_HIP;
  return hip_status(launch_sort(n_pairs, num_tiles, keys, vals, keys_tmp, vals_tmp, tile_ranges, tile_order,
                                sorted_low_bits, digit_counts, result_in_tmp, ws, s, false));
}

gs_status gs_render_fwd(int64_t n, gs_projected proj, const uint32_t* sorted_vals, const int64_t* tile_ranges,
                        const int32_t* tile_order, const gs_camera* cam, const float bg[3], float* image,
                        float* final_T, uint32_t* n_contrib, void* stream) {
  if (n < 0 || !camera_ok(cam) || !bg || !image || !final_T || !n_contrib || !tile_ranges) return GS_ERR_INVALID_ARG;
  if (n >= kMaxGaussians || !camera_fits(cam)) return GS_ERR_OVERFLOW;
  if (n > 0 && (!projected_ok(proj) || !sorted_vals)) return GS_ERR_INVALID_ARG;
  const DevCamera d = dev_camera(cam);
  hipStream_t s = static_cast<hipStream_t>(stream);
  return hip_status(timed(kRenderFwd, s, [&] {
    return launch_render_fwd(proj, sorted_vals, (uint32_t)(n - 1), tile_ranges, tile_order, d, bg, image, final_T,
                             n_contrib, s);
  }));
}

gs_status gs_render_bwd(int64_t n, const float* means, const float* scales, const float* quats,
                        const float* opacities, const float* sh, int32_t sh_degree, const gs_camera* cam,
                        gs_projected proj, const uint32_t* sorted_vals, const int64_t* tile_ranges,
                        const int32_t* tile_order, const float bg[3], const float* final_T,
                        const uint32_t* n_contrib, const float* dL_dimage, gs_grads out, float* densify_accum,
                        int32_t* densify_denom, void* stream) {
  (void)opacities;
  if (n < 0 || sh_degree < 0 || sh_degree > 3 || !camera_ok(cam) || !bg || !final_T || !n_contrib ||
      !dL_dimage || !tile_ranges)
    return GS_ERR_INVALID_ARG;
  if (n >= kMaxGaussians || !camera_fits(cam)) return GS_ERR_OVERFLOW;
  if (n == 0) return GS_OK;
  if (!means || !scales || !quats || !sh || !projected_ok(proj) || !sorted_vals) return GS_ERR_INVALID_ARG;
  if (!out.grad_screen || !out.dmeans || !out.dscales || !out.dquats || !out.dsh) return GS_ERR_INVALID_ARG;
  const DevCamera d = dev_camera(cam);
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = launch_fill_u32(out.grad_screen, n * GS_GRAD_SCREEN, 0u, s);
  if (e == hipSuccess)
    e = timed(kRenderBwd, s, [&] {
      return launch_render_bwd(proj, sorted_vals, (uint32_t)(n - 1), tile_ranges, tile_order, d, bg, final_T, n_contrib,
                               dL_dimage, out.grad_screen, s);
    });
  if (e == hipSuccess)
    e = timed(kProjectBwd, s, [&] {
      return launch_project_bwd(n, means, scales, quats, sh, sh_degree, d, proj, out, densify_accum, densify_denom,
                                s);
    });
  return hip_status(e);
}

gs_status gs_measure_project_io(int64_t n, const float* means, const float* scales, const float* quats,
                                const float* opacities, const float* sh, int32_t sh_degree, gs_projected out,
                                void* stream) {
  if (n < 0 || sh_degree < 0 || sh_degree > 3) return GS_ERR_INVALID_ARG;
  if (n >= kMaxGaussians) return GS_ERR_OVERFLOW;
  if (n == 0) return GS_OK;
  if (!means || !scales || !quats || !opacities || !sh || !projected_ok(out)) return GS_ERR_INVALID_ARG;
  return hip_status(
      launch_project_io(n, means, scales, quats, opacities, sh, sh_degree, out, static_cast<hipStream_t>(stream)));
}

gs_status gs_measure_scatter_io(int64_t n, const uint64_t* keys, const uint32_t* vals, const uint32_t* dest,
                                uint32_t* out, void* stream) {
  if (n < 0) return GS_ERR_INVALID_ARG;
  if (n > (int64_t)UINT32_MAX) return GS_ERR_OVERFLOW;
  if (n == 0) return GS_OK;
  if (!keys || !vals || !dest || !out) return GS_ERR_INVALID_ARG;
  return hip_status(launch_scatter_io(n, keys, vals, dest, out, static_cast<hipStream_t>(stream)));
}

gs_status gs_kernel_timer_start(const char* kernel) {
  const TimedKernel k = timed_kernel_id(kernel);
  if (k == kNone) return GS_ERR_INVALID_ARG;
  KernelTimer& t = timer();
  std::lock_guard<std::mutex> g(t.mu);
  if (t.armed != kNone) return GS_ERR_INVALID_ARG;
  t.armed = k;
  t.used = 0;
  t.failed = false;
  t.armed_any.store(1, std::memory_order_release);
  return GS_OK;
}

gs_status gs_kernel_timer_stop(int64_t* launches, double* total_ms) {
  if (!launches || !total_ms) return GS_ERR_INVALID_ARG;
  KernelTimer& t = timer();
  std::lock_guard<std::mutex> g(t.mu);
  if (t.armed == kNone) return GS_ERR_INVALID_ARG;
  t.armed = kNone;
  t.armed_any.store(0, std::memory_order_release);
  *launches = 0;
  *total_ms = 0.0;
  if (t.failed) return GS_ERR_HIP;
  double sum = 0.0;
  for (size_t i = 0; i + 1 < t.used; i += 2) {
    if (hipEventSynchronize(t.events[i + 1]) != hipSuccess) return GS_ERR_HIP;
    float ms = 0.0f;
    if (hipEventElapsedTime(&ms, t.events[i], t.events[i + 1]) != hipSuccess) return GS_ERR_HIP;
    sum += ms;
  }
  *launches = (int64_t)(t.used / 2);
  *total_ms = sum;
  return GS_OK;
}

}  // extern "C"
