/*
 * gs_raster.h -- C ABI of the MI355X (gfx950) tile rasteriser for 3D Gaussian splatting.
 *
 * The five calls follow the pipeline the pages describe: project every Gaussian to a 2D
 * Gaussian, assign it to 16x16 tiles, sort each tile's list by depth, composite every
 * pixel front to back with transmittance, and run the reverse pass that feeds the
 * densification statistics.
 *   - "Implementing Better Gaussian Splatting in Julia" (pwwt.cn): s1.1 pipeline, s3.1
 *     the Gaussian record (position, scale, quaternion rotation, opacity, colour), s3.2
 *     projection through the Jacobian, s3.3 front-to-back compositing, s4.3 16x16 tiles
 *     and the influence radius, s5.1/s5.3 preallocated buffers and data resident on GPU.
 *   - "Better Gaussian Splatting in Julia" (lshu.cn): s3.1 parameter table (mean,
 *     covariance, SH coefficients by degree, opacity), s3.2 the rasterize pipeline
 *     (project_gaussians, assign_to_tiles, sort_by_depth!, blend), s7.2 buffers passed in.
 *   - "Enabling the absolute-gradient strategy in 3D Gaussian Splatting" (jsqmd.com):
 *     s1-s3 the view-space and absolute gradient accumulators and their visibility mask.
 *   - "Training 10M Gaussians in 8 GB: Spirula Studio's VRAM efficiency" (mhpq.cn): the
 *     32-bit index wrap section (64-bit addressing, overflow is an error, never a wrap).
 *
 * Conventions
 *  - Pointers are DEVICE pointers owned by the caller unless marked [host].  The library
 *    never allocates memory; scratch space comes from one caller workspace sized by
 *    gs_workspace_bytes().  Arrays are dense, row major, naturally aligned (16 bytes for
 *    float arrays read as vectors: means/scales/quats/sh/rec).
 *  - `stream` is a hipStream_t (NULL = the null stream).  Work is enqueued on it; only
 *    gs_bin_tiles waits on it, once, to read the pair count back.
 *  - Every call validates its arguments before touching the GPU and returns a gs_status.
 *  - Calls keep no global state and may run concurrently on different streams with
 *    different buffers; the exceptions are gs_sort_keys_noalloc (its fixed scratch is per
 *    GPU) and the one HIP event per host thread and GPU that gs_bin_tiles creates once and
 *    keeps.  The kernel timer of gs_measure.h is measurement state, outside the method.
 *  - Numbers: fp32 storage; the projection evaluates the binning-critical geometry
 *    (camera-space mean, 2D covariance, support, pixel box) in float64 and rounds once.
 *  - Gaussians with NaN/Inf inputs are culled (every visibility test fails on NaN).
 */
#ifndef GS_RASTER_H
#define GS_RASTER_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t gs_status;
enum {
  GS_OK = 0,
  GS_ERR_INVALID_ARG = 1, /* null pointer with n > 0, sh_degree not in 0..3, bad camera   */
  GS_ERR_CAPACITY = 2,    /* pair buffer too small; *n_pairs holds the required count     */
  GS_ERR_OVERFLOW = 3,    /* n >= 2^32, width/height > 65535, or a count past int64        */
  GS_ERR_HIP = 4,         /* a HIP launch or runtime call failed                          */
  GS_ERR_WORKSPACE = 5    /* workspace NULL or smaller than gs_workspace_bytes()          */
};

#define GS_TILE 16       /* tiles are 16x16 pixels                                          */
#define GS_REC_FLOATS 12 /* floats per projected render record                            */
#define GS_GRAD_SCREEN 10 /* floats per Gaussian in the screen-space gradient block        */
#define GS_TILE_DIGIT_COUNTS 512 /* uint64 words of gs_bin_tiles' tile-digit counts (2 x 256) */
#define GS_ROW_BLOCK 256     /* Gaussians per region of gs_projected.rows                       */
#define GS_ROWS_PER_BLOCK 128 /* entries (uint32 pairs) per region of gs_projected.rows          */

/* Pinhole camera, OpenCV frame: x right, y down, z forward.  x_cam = R x_world + t with
 * R row major.  Pixel (i, j) has its centre at (i + 0.5, j + 0.5).  Gaussians with
 * z_cam <= near_z are culled.  The camera centre used for view-dependent colour is
 * -R^T t.  width, height in 1..65535; fx, fy, near_z > 0. */
typedef struct gs_camera {
  float R[9];
  float t[3];
  float fx, fy, cx, cy;
  int32_t width, height;
  float near_z;
} gs_camera;

/* Output of gs_project, N rows each (device pointers, caller-owned).
 *  rec[n][12]: u, v (2D mean, pixels); A, B, C (conic = inverse 2D covariance
 *              [[A, B], [B, C]]); opacity; r, g, b (colour, clamped at 0);
 *              word 9 = px0 | px1 << 16 and word 10 = py0 | py1 << 16 (the pixel-centre
 *              bounding box of the support ellipse, clamped to the image, as uint32
 *              bit patterns); word 11 = 0.  All zero for a culled Gaussian.
 *  depth[n]:   camera-space z rounded once to fp32 (sort keys use its bit pattern).
 *  rect[n][4]: tile rectangle tx0, tx1, ty0, ty1 (inclusive); zero when culled.
 *  n_tiles[n]: tiles of the rectangle whose pixel-centre box (inside the pixel box) meets
 *              the record's support ellipse q <= tau ("Training 10M Gaussians in 8 GB:
 *              Spirula Studio's VRAM efficiency", 16-bit AABB section: an ellipse test
 *              after the box), for every rectangle whatever its size.  0 when culled or no
 *              tile passes.
 *  clamp[n]:   bit c set when colour channel c was negative before the clamp at 0.
 *  runs[n][8]: the tile record gs_bin_tiles expands, 32 bytes per Gaussian: words 0-3
 *              the kept tiles of each tile row of a rectangle of at most 8 tile rows and
 *              255 tile columns, two bytes per row (first kept column - tx0, kept count),
 *              rows in order from ty0; for a larger rectangle word 0 = 0xFFFFFFFE and word
 *              1 = the index of its first entry in `rows`, or, when its block's region of
 *              `rows` is full, all bytes 0xFF (gs_bin_tiles then recomputes its kept tiles
 *              from rec by the same test); word 4 = tx0 | tx1 << 16; word 5 = ty0 | ty1 << 16;
 *              word 6 = n_tiles; word 7 = 0.
 *  rows[ceil(n / GS_ROW_BLOCK) * GS_ROWS_PER_BLOCK][2]: the larger rectangles' kept tiles,
 *              one entry per tile row from ty0: (first kept column | kept count << 16,
 *              kept tiles of the rectangle's earlier rows).  Block b of GS_ROW_BLOCK
 *              Gaussians owns entries [GS_ROWS_PER_BLOCK b, GS_ROWS_PER_BLOCK (b + 1)), a
 *              quarter of them for each 64 consecutive Gaussians: its first 31 entries
 *              filled in id order, its last one's first word 1 when one of the 64 has a
 *              rectangle that did not fit (then left to the float64 path), else 0. */
typedef struct gs_projected {
  float* rec;
  float* depth;
  uint16_t* rect;
  uint32_t* n_tiles;
  uint8_t* clamp;
  uint32_t* runs;
  uint32_t* rows;
} gs_projected;

/* Gradients written by gs_render_bwd (all overwritten, N rows each).
 *  grad_screen[n][10]: dL/du, dL/dv, dL/dA, dL/dB, dL/dC, dL/dopacity, dL/dr, dL/dg,
 *                      dL/db, and sum over pixels of ||dL_p/d(u, v)||_2 (the absolute
 *                      view-space gradient).  B is the off-diagonal conic entry, which
 *                      enters the exponent as 2 B dx dy.
 *  dmeans[n][3], dscales[n][3], dquats[n][4] (w, x, y, z), dsh[n][K][3]: gradients with
 *                      respect to the inputs of gs_project.  The opacity gradient is
 *                      grad_screen column 5. */
typedef struct gs_grads {
  float* grad_screen;
  float* dmeans;
  float* dscales;
  float* dquats;
  float* dsh;
} gs_grads;

/*
 * gs_project -- project N Gaussians ("Implementing Better Gaussian Splatting in Julia"
 * s3.1-3.2; "Better Gaussian Splatting in Julia" s3.1-3.2).
 *  means[n][3]      world-space centres
 *  scales[n][3]     linear standard deviations along the local axes
 *  quats[n][4]      rotation quaternion (w, x, y, z); normalised inside
 *  opacities[n]     opacity in (0, 1) (already activated)
 *  sh[n][K][3]      SH coefficients, K = (sh_degree + 1)^2, real basis with the
 *                   Condon-Shortley phase; colour = max(0, 0.5 + sum_k Y_k(d) sh_k)
 *                   with d the unit direction from the camera centre to the mean
 *  cam [host]       camera
 * The 2D covariance is J W Sigma W^T J^T (first-order perspective Jacobian J at the
 * camera-space mean, no low-pass dilation).  A Gaussian is kept when z > near_z, its 2D
 * covariance [[a, b], [b, c]] is not a line to working precision (det = a c - b^2 >
 * 1e-9 (a + c)^2, a screen-space axis ratio above ~3e-5: a zero scale otherwise leaves det
 * as rounding noise), opacity >= 1/255 and its support {q <= 2 ln(255 opacity)} covers at
 * least one pixel centre; the tile rect is the support's pixel-centre bounding box >> 4.
 * Errors: INVALID_ARG, OVERFLOW (n >= 2^32), HIP.
 */
gs_status gs_project(int64_t n, const float* means, const float* scales, const float* quats,
                     const float* opacities, const float* sh, int32_t sh_degree,
                     const gs_camera* cam, gs_projected out, void* stream);

/*
 * gs_quantize_sh -- q8 / q16 codes of SH coefficients ("Training 10M Gaussians in 8 GB:
 * Spirula Studio's VRAM efficiency", quantised training section: 8/16-bit fixed-point SH with a
 * (min, max) table, one pair per 256 units).  Units are the coefficients of sh[n][K][3] in
 * that order; block b = units [256 b, 256 b + 256).
 *  codes[n][K][3]  uint8 (bits 8) or uint16 (bits 16): rint((x - lo) * (qmax / (hi - lo)))
 *                  evaluated in float64, clamped to [0, qmax] (0 when hi == lo), qmax = 2^bits - 1
 *  bounds[ceil(3 K n / 256)][2]  float32 (lo, hi) = the block's minimum and maximum
 * Errors: INVALID_ARG (bits not 8 or 16, null pointer with n > 0), OVERFLOW, HIP.
 */
gs_status gs_quantize_sh(int64_t n, const float* sh, int32_t sh_degree, int32_t bits, void* codes,
                         float* bounds, void* stream);

/*
 * gs_project_qsh -- gs_project with the SH coefficients given as gs_quantize_sh's codes and
 * bounds (sh_bits 8 or 16).  Each coefficient decodes, in float32 with every operation
 * rounded, as lo + code * ((hi - lo) * (1 / qmax)); the rest is gs_project unchanged, and the
 * outputs feed gs_bin_tiles and the compositing calls as they are.  (The backward reads
 * float32 SH: gs_render_bwd.)  Reads 96 (q16) or 48 (q8) instead of 192 bytes of SH per
 * degree-3 Gaussian.
 * Errors: as gs_project, and INVALID_ARG for sh_bits not 8 or 16.
 */
gs_status gs_project_qsh(int64_t n, const float* means, const float* scales, const float* quats,
                         const float* opacities, const void* sh_codes, const float* sh_bounds,
                         int32_t sh_bits, int32_t sh_degree, const gs_camera* cam, gs_projected out,
                         void* stream);

/*
 * gs_workspace_bytes -- bytes of device workspace that gs_bin_tiles and gs_sort_keys need
 * for n Gaussians, up to pair_capacity pairs and num_tiles tiles (the largest stage; the
 * two calls reuse the same workspace).  Returns 0 for invalid arguments.
 */
size_t gs_workspace_bytes(int64_t n, int64_t pair_capacity, int32_t num_tiles);

/*
 * gs_bin_tiles -- duplicate every visible Gaussian once per covered tile ("Better Gaussian
 * Splatting in Julia" s3.2 assign_to_tiles):
 *   keys[p] = tile_id << 32 | bits(depth),  tile_id = ty * tiles_x + tx
 *   vals[p] = Gaussian id
 * Pairs come out ordered by (tile_id & 255, bits(depth), Gaussian id): the visible
 * Gaussians are radix-sorted by depth, and their expansion into tiles performs the first
 * 8-bit digit pass over the tile id.  So the keys are already stably ordered by their low
 * 40 bits, and gs_sort_keys(sorted_low_bits = 40) completes the (tile, depth, id) order
 * with passes over the tile bits above the low byte only (none when num_tiles <= 256).
 * Writes the pair count P to *n_pairs [host], the call's one device->host read.  When
 * n_pairs points to page-locked host memory (hipHostMalloc, a pinned torch tensor) the
 * count is copied straight into it and the call waits for that copy only: the depth
 * ordering of the Gaussians, which needs no host value, is already queued behind it and
 * keeps the GPU busy meanwhile.  Into pageable memory HIP performs the copy synchronously,
 * so the depth ordering is queued after it.  Results are the same either way.  The wait
 * uses one HIP event per host thread and GPU, created on the thread's first call on that
 * GPU and kept by the library: a call creates nothing.  With keys == NULL only P
 * is computed.  If P > capacity,
 * returns GS_ERR_CAPACITY with *n_pairs = P and writes no pairs.  The workspace must hold
 * gs_workspace_bytes(n, P, num_tiles) bytes (checked before and after P is known).
 * tile_digit_counts [device, optional, GS_TILE_DIGIT_COUNTS uint64]: when the call writes
 * pairs, receives [p][d] = the number of pairs whose tile id has bits [8 + 8p, 16 + 8p)
 * equal to d, for the digit passes gs_sort_keys will make (rows it will not use are 0),
 * counted by the expansion's counting pass.  Passed to gs_sort_keys(sorted_low_bits
 * = 40) with the same pairs, it replaces that call's counting read of every key.
 * Errors: INVALID_ARG, WORKSPACE, CAPACITY, OVERFLOW, HIP.
 */
gs_status gs_bin_tiles(int64_t n, gs_projected proj, const gs_camera* cam, uint64_t* keys,
                       uint32_t* vals, int64_t capacity, int64_t* n_pairs,
                       uint64_t* tile_digit_counts, void* workspace, size_t workspace_bytes,
                       void* stream);

/*
 * gs_sort_keys -- stable LSD radix sort of (keys, vals) over key bits [sorted_low_bits,
 * 32 + ceil(log2(num_tiles))), 8 bits per pass ("Better Gaussian Splatting in Julia" s3.2
 * sort_by_depth!; "Implementing Better Gaussian Splatting in Julia" s3.3 depth order).
 * The input must already be stably ordered by its low sorted_low_bits bits (0 = no
 * assumption: a full sort; 40 = the output of gs_bin_tiles).  Equal keys keep their input
 * order, so depth ties stay broken by Gaussian id.  The passes ping-pong between
 * keys/vals and keys_tmp/vals_tmp (same sizes), so an odd pass count ends in the _tmp
 * pair.  result_in_tmp [host]: NULL = the result is moved back to keys/vals; non-NULL =
 * the result stays where the last pass wrote it and *result_in_tmp is set to 1 when that
 * is keys_tmp/vals_tmp, else 0 (the other pair then holds scratch).  The pass count, and
 * so *result_in_tmp, depends only on n_pairs > 1, num_tiles and sorted_low_bits.  Then
 * writes tile_ranges[num_tiles][2] = [first, last + 1) of each tile in the sorted order
 * ([0, 0) for an empty tile) and, when tile_order is non-NULL, tile_order[num_tiles] =
 * every tile id once, longest lists first (a schedule for the compositing calls; it does
 * not change their results).  Keys must have tile_id < num_tiles.
 * digit_counts [device, optional]: [p][256] counts of each pass's digit (key bits
 * [sorted_low_bits + 8p, + 8)) over the keys, one row per pass; NULL = the call counts
 * them with one read of the keys.  gs_bin_tiles' tile_digit_counts are exactly this for
 * its pairs and sorted_low_bits = 40.  Counts that do not match the keys give an
 * unspecified order, but every write stays inside the n_pairs slots.
 * Errors: INVALID_ARG, WORKSPACE, OVERFLOW, HIP.
 */
gs_status gs_sort_keys(int64_t n_pairs, int32_t num_tiles, int32_t sorted_low_bits, uint64_t* keys,
                       uint32_t* vals, uint64_t* keys_tmp, uint32_t* vals_tmp,
                       int64_t* tile_ranges, int32_t* tile_order, const uint64_t* digit_counts,
                       int32_t* result_in_tmp, void* workspace, size_t workspace_bytes, void* stream);

/*
 * gs_sort_ids -- gs_sort_keys for the compositing calls, which read only the sorted ids
 * and the tile ranges ("Better Gaussian Splatting in Julia" s3.2: blend takes each tile's
 * depth-ordered Gaussians).  Same arguments and results, except that the last digit pass
 * does not write the sorted keys (8 of the pass's 24 bytes per pair): after the call the
 * keys of the buffer pair holding the result are unspecified when a digit pass ran, while
 * the ids, tile_ranges, tile_order and *result_in_tmp are those of gs_sort_keys.
 * result_in_tmp [host] is required.
 * Errors: INVALID_ARG (also for result_in_tmp NULL), WORKSPACE, OVERFLOW, HIP.
 */
gs_status gs_sort_ids(int64_t n_pairs, int32_t num_tiles, int32_t sorted_low_bits, uint64_t* keys,
                      uint32_t* vals, uint64_t* keys_tmp, uint32_t* vals_tmp, int64_t* tile_ranges,
                      int32_t* tile_order, const uint64_t* digit_counts, int32_t* result_in_tmp,
                      void* workspace, size_t workspace_bytes, void* stream);

/*
 * gs_sort_keys_noalloc -- gs_sort_keys for callers that cannot allocate device memory or
 * hand over a workspace: code under HIP graph capture, tight serving loops, harnesses that
 * forbid allocation.  Same arguments, results and errors as gs_sort_keys, without the
 * workspace.  Its scratch is a fixed device array of GS_SORT_NOALLOC_SCRATCH_BYTES inside
 * the library, one copy per GPU, which that GPU holds until the process ends; its address
 * is looked up on the first call on the GPU the stream belongs to.  The call allocates
 * nothing.  A sort needs 279,040 bytes plus 2 KiB per digit pass per started 4096 pairs
 * (gs_workspace_bytes' sort part): one pass (gs_bin_tiles' pairs for up to 65,536 tiles,
 * sorted_low_bits = 40) fits up to 66,551,808 pairs, a full six-pass sort up to about 11M;
 * a larger sort returns GS_ERR_WORKSPACE before any HIP call.  Every call on one GPU uses
 * that GPU's array and clears what it reads before writing it, so calls run one after
 * another on one GPU give the results of gs_sort_keys; calls that overlap on one GPU
 * (other streams, other threads) race on the array and must be serialised by the caller.
 * Errors: INVALID_ARG, WORKSPACE (the sort needs more than the fixed scratch), OVERFLOW, HIP.
 */
#define GS_SORT_NOALLOC_SCRATCH_BYTES (32u << 20)
gs_status gs_sort_keys_noalloc(int64_t n_pairs, int32_t num_tiles, int32_t sorted_low_bits, uint64_t* keys,
                               uint32_t* vals, uint64_t* keys_tmp, uint32_t* vals_tmp, int64_t* tile_ranges,
                               int32_t* tile_order, const uint64_t* digit_counts, int32_t* result_in_tmp,
                               void* stream);

/*
 * gs_render_fwd -- composite every pixel front to back over its tile's sorted list
 * ("Implementing Better Gaussian Splatting in Julia" s3.3 and s5.4, the tile method):
 *   alpha = min(0.99, opacity * exp(-q/2)), q = A dx^2 + 2 B dx dy + C dy^2,
 *   (dx, dy) = pixel centre - (u, v); contributions with alpha < 1/255 are skipped;
 *   C += rgb * alpha * T; T *= 1 - alpha; the pixel stops once T < 1e-4;
 *   image = C + T * bg.
 *  image[3][H][W] (planar), final_T[H][W], n_contrib[H][W] = 1 + the tile-list position
 *  of the last contributor (0 if none), which gs_render_bwd needs.  tile_order (nullable)
 *  is the schedule written by gs_sort_keys; NULL processes tiles in id order.  Ids in the
 *  lists are clamped to n - 1 (as in gs_render_bwd): lists holding ids >= n give
 *  unspecified pixels but no read outside the records.
 * Errors: INVALID_ARG, HIP.
 */
gs_status gs_render_fwd(int64_t n, gs_projected proj, const uint32_t* sorted_vals,
                        const int64_t* tile_ranges, const int32_t* tile_order,
                        const gs_camera* cam, const float bg[3], float* image, float* final_T,
                        uint32_t* n_contrib, void* stream);

/*
 * gs_render_bwd -- reverse pass of gs_render_fwd and of gs_project, plus densification
 * statistics ("Enabling the absolute-gradient strategy in 3D Gaussian Splatting" s1-s3):
 * given dL/dimage[3][H][W], writes every gradient in `out` (overwritten) and, when
 * densify_accum / densify_denom are non-NULL, ACCUMULATES for every visible Gaussian
 * (n_tiles > 0):
 *   densify_accum[i][0] += || (dL/du, dL/dv) ||_2          (view-space gradient norm)
 *   densify_accum[i][1] += sum_p || dL_p/d(u, v) ||_2       (absolute gradient)
 *   densify_denom[i]    += 1
 * Inputs are those of the matching gs_project / gs_sort_keys / gs_render_fwd calls.
 * Float atomics make the screen gradients' summation order, and so their last bits,
 * vary between runs.
 * Errors: INVALID_ARG, HIP.
 */
gs_status gs_render_bwd(int64_t n, const float* means, const float* scales, const float* quats,
                        const float* opacities, const float* sh, int32_t sh_degree,
                        const gs_camera* cam, gs_projected proj, const uint32_t* sorted_vals,
                        const int64_t* tile_ranges, const int32_t* tile_order, const float bg[3],
                        const float* final_T, const uint32_t* n_contrib, const float* dL_dimage,
                        gs_grads out, float* densify_accum, int32_t* densify_denom, void* stream);

/* Parameters of gs_densify (values, host). */
typedef struct gs_densify_params {
  float grad_threshold;  /* average view-space gradient (pixel units) above which a Gaussian densifies */
  int32_t use_abs;       /* 1: average the absolute-gradient column densify_accum[:, 1]; 0: column 0 */
  float scale_threshold; /* largest axis scale <= this: clone; above: split (world units) */
  int32_t split_n;       /* children per split, 2..4 */
  float split_shrink;    /* children's scales = parent's / split_shrink (> 0) */
  float min_opacity;     /* outputs with opacity below this are pruned */
  float max_scale;       /* outputs whose largest scale exceeds this are pruned; <= 0: no such test */
} gs_densify_params;

/*
 * gs_densify -- densify and prune N Gaussians from the statistics gs_render_bwd accumulated
 * ("Enabling the absolute-gradient strategy in 3D Gaussian Splatting" s1, s3.3; "Better
 * Gaussian Splatting in Julia" s3.4; "Implementing Better Gaussian Splatting in Julia"
 * s4.2).  Per Gaussian, average = accum[col] / denom in float64 (col = use_abs; denom = 0
 * never densifies).  average > grad_threshold and largest scale <= scale_threshold: the
 * Gaussian is kept and cloned (an exact copy right after it); average > grad_threshold and
 * a larger scale: it is replaced by split_n children, child j centred at
 * mean + R(q / |q|) (scale * normals[i][j]) (float64, rounded once), scales = scale /
 * split_shrink, quaternion, opacity and SH copied; otherwise it is kept as is.  Every
 * output whose opacity < min_opacity, or (max_scale > 0) whose largest scale > max_scale,
 * is pruned.
 *  accum[n][2], denom[n]  the statistics (read only; the caller resets them)
 *  normals[n][split_n][3] standard normal samples for the children (read for split inputs)
 *  out_*                  the new set, same layouts as the inputs; out_src[m] = the input
 *                         index output m comes from.  Outputs keep input order, each input's
 *                         outputs contiguous.  Output buffers must not alias the inputs.
 *  capacity, n_out [host] as gs_bin_tiles: *n_out = the output count (one device->host
 *                         read and stream synchronisation); with out_means == NULL only the
 *                         count is computed; n_out > capacity: GS_ERR_CAPACITY, nothing written.
 *  workspace              gs_densify_workspace_bytes(n) bytes.
 * Errors: INVALID_ARG (null pointer, sh_degree or split_n out of range, split_shrink <= 0),
 * OVERFLOW, CAPACITY, WORKSPACE, HIP.
 */
size_t gs_densify_workspace_bytes(int64_t n);
gs_status gs_densify(int64_t n, const float* means, const float* scales, const float* quats,
                     const float* opacities, const float* sh, int32_t sh_degree,
                     const float* densify_accum, const int32_t* densify_denom, const float* normals,
                     const gs_densify_params* params, float* out_means, float* out_scales,
                     float* out_quats, float* out_opacities, float* out_sh, uint32_t* out_src,
                     int64_t capacity, int64_t* n_out, void* workspace, size_t workspace_bytes,
                     void* stream);

/* Hyper-parameters of gs_adam_q16 (values, host). */
typedef struct gs_adam_params {
  float lr, beta1, beta2, eps; /* learning rate, moment decays in [0, 1), epsilon */
  int64_t step;                /* 1-based step number (bias correction 1 - beta^step) */
} gs_adam_params;

/*
 * gs_adam_q16 -- one fused Adam step over n float32 parameters whose two moments are kept as
 * 16-bit codes ("Training 10M Gaussians in 8 GB: Spirula Studio's VRAM efficiency",
 * quantised training section: 16-bit moments packed side by side in a transposed layout,
 * bounds per 256 units, float32 gradients).
 *  params[n]   float32, updated in place
 *  grads[n]    float32 gradients
 *  state[n]    uint32 per unit: m code | v code << 16 (unit-major, so 64 lanes read 256
 *              contiguous bytes), updated in place
 *  bounds[ceil(n/256)][4]  float32 (m_lo, m_hi, v_lo, v_hi) of each 256-unit block, updated
 *              in place.  A zero state with zero bounds is the start (both moments 0).
 * Adam (Kingma and Ba) with bias correction: m = b1 m + (1 - b1) g, v = b2 v + (1 - b2) g^2,
 * param -= lr (m / (1 - b1^step)) / (sqrt(v / (1 - b2^step)) + eps).  A moment decodes as
 * lo + code (hi - lo) / 65535; the moments are updated in float64, the parameter's step in
 * float32 (about 5e-7 relative) and the parameter rounded once.  Each block's new bounds are
 * its moments' minimum and maximum rounded to float32, and a code is
 * rint((x - lo) / (hi - lo) * 65535) clamped to [0, 65535] (0 when hi == lo).  Constants
 * enter as reciprocals computed once, so a code decided within a few float64 roundings of
 * a half-integer can differ by one from the definition's.
 * Errors: INVALID_ARG (null pointer with n > 0, step < 1, beta outside [0, 1)), HIP.
 */
gs_status gs_adam_q16(int64_t n, float* params, const float* grads, uint32_t* state, float* bounds,
                      const gs_adam_params* hyper, void* stream);

/*
 * gs_fpbo_pack / gs_adam_fpbo -- the fused Adam step with the parameters kept as 16-bit codes
 * too, beside both moments ("Training 10M Gaussians in 8 GB: Spirula Studio's VRAM
 * efficiency", quantised training section: parameters and moments packed together into
 * 16-bit words in a transposed layout, bounds per 256 units, float32 gradients).
 *  state[ceil(n/256)][3][256]  uint16 (device; 8-byte aligned): per block of 256 units three
 *              planes of codes, the parameters', the first moments', the second moments'; codes
 *              past unit n - 1 are 0.  Updated in place.
 *  bounds[ceil(n/256)][6]  float32 (device; 8-byte aligned): (p_lo, p_hi, m_lo, m_hi, v_lo,
 *              v_hi) of each block.  Updated in place.
 * gs_fpbo_pack writes the start state from float32 params[n] (device, 16-byte aligned): the
 * parameters' codes with their blocks' exact minimum and maximum, both moments 0 (codes 0,
 * bounds 0).
 * gs_adam_fpbo takes grads[n] (float32, device, 16-byte aligned) and hyper as gs_adam_q16.  Per
 * unit it decodes the parameter and both moments (lo + code (hi - lo) / 65535), updates the
 * moments in float64, takes the parameter's step in float32 (about 5e-7 relative) and
 * subtracts it in float64; each block's new bounds are the float32 roundings of the minimum
 * and maximum of each quantity, and a code is rint((x - lo) / (hi - lo) * 65535) clamped to
 * [0, 65535] (0 when hi == lo).  A parameter's update smaller than half its block's code
 * step leaves its code unchanged.  params_out[n] (float32, device, 16-byte aligned; may be
 * NULL) receives the new parameters as stored, each new code decoded and rounded once.
 * Constants enter as reciprocals computed once, so a code decided within a few float64
 * roundings of a half-integer can differ by one from the definition's.
 * Errors: INVALID_ARG (null pointer with n > 0, misaligned pointer, step < 1, beta outside
 * [0, 1)), OVERFLOW (n >= 2^40), HIP.
 */
gs_status gs_fpbo_pack(int64_t n, const float* params, uint16_t* state, float* bounds, void* stream);
gs_status gs_adam_fpbo(int64_t n, uint16_t* state, float* bounds, const float* grads, float* params_out,
                       const gs_adam_params* hyper, void* stream);

/* Human-readable name of a status code (static string). */
const char* gs_status_string(gs_status status);

#ifdef __cplusplus
}
#endif

#endif /* GS_RASTER_H */
