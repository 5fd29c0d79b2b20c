// gs_densify.hip -- densify-and-prune of a Gaussian set from its accumulated gradient
// statistics, for gfx950.
//
// "Enabling the absolute-gradient strategy in 3D Gaussian Splatting" (jsqmd.com) s1 and
// s3.3: a Gaussian's average view-space gradient (accumulated norm / views, from the first
// accumulator column or, with the absolute-gradient strategy, the second) above a threshold
// makes it densify: cloned when its scale is small, split when it is large; Gaussians with
// too low an opacity or an abnormal scale are pruned.  "Better Gaussian Splatting in Julia"
// (lshu.cn) s3.4 and "Implementing Better Gaussian Splatting in Julia" (pwwt.cn) s4.2
// describe the same adaptive density control.  A clone is an exact copy; a split draws
// split_n children from the Gaussian itself with caller-supplied normal samples.
//
// A stream compaction in two passes over workgroups of 256 Gaussians (one per lane):
//   k_densify_count  each lane's output count (0, 1, 2 or split_n), summed per workgroup
//   (scan of the workgroup sums: the workgroup's first output)
//   k_densify_emit   the same decisions; a workgroup scan places each lane's outputs, the
//                    lanes stage their rows' centres, scales and source lanes in LDS, and
//                    the workgroup writes every output array as one contiguous range
//                    (coalesced stores; the SH rows are copied float4 by float4 from the
//                    source rows).
// The decisions use float64 averages and the float32 scales and opacities as given, so
// they are bit-exact against a float64 reference.
#include "gs_device.h"

namespace gs {

hipError_t launch_scan_sums(int64_t nb, uint64_t* sums, uint64_t* total, hipStream_t s);

constexpr int kDensBlock = 256;
constexpr int kMaxSplit = 4;
constexpr int kMaxRows = kDensBlock * kMaxSplit;  // outputs of one workgroup at most

struct DensParams {
  float grad_threshold, scale_threshold, split_shrink, min_opacity, max_scale;
  int use_abs, split_n;
};

// Largest of three, NaN if any is NaN.
__device__ __forceinline__ float max3_nan(float a, float b, float c) {
  const float m = a > b || a != a ? a : b;
  return m > c || m != m ? m : c;
}

// 0 keep, 1 clone, 2 split (kind), and the Gaussian's output count after pruning.
struct Decision {
  int kind, count;
};

__device__ __forceinline__ Decision decide(int64_t i, const float* __restrict__ scales,
                                          const float* __restrict__ opac, const float* __restrict__ accum,
                                          const int32_t* __restrict__ denom, const DensParams& p) {
  const int32_t d = denom[i];
  const double avg = d > 0 ? (double)accum[2 * i + (p.use_abs ? 1 : 0)] / (double)d : 0.0;
  const bool dens = avg > (double)p.grad_threshold;
  const float smax = max3_nan(scales[3 * i], scales[3 * i + 1], scales[3 * i + 2]);
  Decision r;
  r.kind = dens ? (smax <= p.scale_threshold ? 1 : 2) : 0;
  // children's largest scale is the parent's divided (division is monotonic)
  const float out_smax = r.kind == 2 ? smax / p.split_shrink : smax;
  const bool keep = opac[i] >= p.min_opacity && (p.max_scale <= 0.0f || out_smax <= p.max_scale);
  r.count = keep ? (r.kind == 2 ? p.split_n : r.kind == 1 ? 2 : 1) : 0;
  return r;
}

__global__ __launch_bounds__(kDensBlock) void k_densify_count(int64_t n, const float* __restrict__ scales,
                                                              const float* __restrict__ opac,
                                                              const float* __restrict__ accum,
                                                              const int32_t* __restrict__ denom, DensParams p,
                                                              uint64_t* __restrict__ sums) {
  __shared__ uint32_t s_w[kDensBlock / kWave];
  const int64_t i = (int64_t)blockIdx.x * kDensBlock + threadIdx.x;
  const uint32_t c = i < n ? (uint32_t)decide(i, scales, opac, accum, denom, p).count : 0u;
  const uint32_t w = wave_sum(c);
  if (__lane_id() == 0) s_w[threadIdx.x / kWave] = w;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint64_t t = 0;
#pragma unroll
    for (int k = 0; k < kDensBlock / kWave; ++k) t += s_w[k];
    sums[blockIdx.x] = t;
  }
}

// Rotation of the unit quaternion q / |q| (w, x, y, z), float64.
__device__ __forceinline__ void rot_of(const float4 qf, double R[9]) {
  const double qw = qf.x, qx = qf.y, qy = qf.z, qz = qf.w;
  const double il = 1.0 / sqrt(qw * qw + qx * qx + qy * qy + qz * qz);
  const double w = qw * il, x = qx * il, y = qy * il, z = qz * il;
  R[0] = 1.0 - 2.0 * (y * y + z * z); R[1] = 2.0 * (x * y - w * z); R[2] = 2.0 * (x * z + w * y);
  R[3] = 2.0 * (x * y + w * z); R[4] = 1.0 - 2.0 * (x * x + z * z); R[5] = 2.0 * (y * z - w * x);
  R[6] = 2.0 * (x * z - w * y); R[7] = 2.0 * (y * z + w * x); R[8] = 1.0 - 2.0 * (x * x + y * y);
}

// RU elements of `unit` floats per SH row (float4 when a row is a whole number of them).
template <int L>
struct ShRow {
  static constexpr int ROW = 3 * (L + 1) * (L + 1);
  static constexpr bool V4 = ROW % 4 == 0;
  static constexpr int RU = V4 ? ROW / 4 : ROW;
};

template <int L>
__global__ __launch_bounds__(kDensBlock) void k_densify_emit(
    int64_t n, const float* __restrict__ means, const float* __restrict__ scales, const float4* __restrict__ quats,
    const float* __restrict__ opac, const float* __restrict__ sh, const float* __restrict__ accum,
    const int32_t* __restrict__ denom, const float* __restrict__ normals, DensParams p,
    const uint64_t* __restrict__ block_off, float* __restrict__ out_means, float* __restrict__ out_scales,
    float4* __restrict__ out_quats, float* __restrict__ out_opac, float* __restrict__ out_sh,
    uint32_t* __restrict__ out_src) {
  __shared__ float s_mean[kMaxRows * 3];
  __shared__ float s_scale[kMaxRows * 3];
  __shared__ uint8_t s_lane[kMaxRows];
  __shared__ uint32_t s_w[kDensBlock / kWave];
  const int tid = threadIdx.x, lane = __lane_id(), wave = tid / kWave;
  const int64_t g0 = (int64_t)blockIdx.x * kDensBlock;
  const int64_t i = g0 + tid;
  Decision d = {0, 0};
  if (i < n) d = decide(i, scales, opac, accum, denom, p);
  // workgroup exclusive scan of the counts: this lane's first row
  const uint32_t inc = wave_inclusive_scan((uint32_t)d.count);
  if (lane == kWave - 1) s_w[wave] = inc;
  __syncthreads();
  uint32_t row = inc - (uint32_t)d.count, total = 0;
#pragma unroll
  for (int k = 0; k < kDensBlock / kWave; ++k) {
    if (k < wave) row += s_w[k];
    total += s_w[k];
  }
  if (d.count > 0) {
    const float m0 = means[3 * i], m1 = means[3 * i + 1], m2 = means[3 * i + 2];
    const float s0 = scales[3 * i], s1 = scales[3 * i + 1], s2 = scales[3 * i + 2];
    if (d.kind == 2) {  // children drawn from the Gaussian: mean + R (scale * z)
      double R[9];
      rot_of(quats[i], R);
      const float c0 = s0 / p.split_shrink, c1 = s1 / p.split_shrink, c2 = s2 / p.split_shrink;
      for (int j = 0; j < d.count; ++j) {
        const float* z = normals + ((size_t)i * p.split_n + j) * 3;
        const double v0 = (double)s0 * z[0], v1 = (double)s1 * z[1], v2 = (double)s2 * z[2];
        const int r = (int)row + j;
        s_mean[3 * r] = (float)((double)m0 + (R[0] * v0 + R[1] * v1 + R[2] * v2));
        s_mean[3 * r + 1] = (float)((double)m1 + (R[3] * v0 + R[4] * v1 + R[5] * v2));
        s_mean[3 * r + 2] = (float)((double)m2 + (R[6] * v0 + R[7] * v1 + R[8] * v2));
        s_scale[3 * r] = c0; s_scale[3 * r + 1] = c1; s_scale[3 * r + 2] = c2;
        s_lane[r] = (uint8_t)tid;
      }
    } else {  // kept, and cloned: exact copies
      for (int j = 0; j < d.count; ++j) {
        const int r = (int)row + j;
        s_mean[3 * r] = m0; s_mean[3 * r + 1] = m1; s_mean[3 * r + 2] = m2;
        s_scale[3 * r] = s0; s_scale[3 * r + 1] = s1; s_scale[3 * r + 2] = s2;
        s_lane[r] = (uint8_t)tid;
      }
    }
  }
  __syncthreads();
  // the workgroup's outputs are rows [base, base + total) of every output array
  const uint64_t base = block_off[blockIdx.x];
  for (uint32_t f = tid; f < 3 * total; f += kDensBlock) {
    out_means[3 * base + f] = s_mean[f];
    out_scales[3 * base + f] = s_scale[f];
  }
  for (uint32_t r = tid; r < total; r += kDensBlock) {
    const int64_t src = g0 + s_lane[r];
    out_src[base + r] = (uint32_t)src;
    out_quats[base + r] = quats[src];
    out_opac[base + r] = opac[src];
  }
  using Q = ShRow<L>;
  if constexpr (Q::V4) {
    const float4* s4 = reinterpret_cast<const float4*>(sh);
    float4* o4 = reinterpret_cast<float4*>(out_sh);
    for (uint32_t f = tid; f < Q::RU * total; f += kDensBlock) {
      const uint32_t r = f / Q::RU, c = f - r * Q::RU;
      o4[(base + r) * Q::RU + c] = s4[(g0 + s_lane[r]) * Q::RU + c];
    }
  } else {
    for (uint32_t f = tid; f < Q::RU * total; f += kDensBlock) {
      const uint32_t r = f / Q::RU, c = f - r * Q::RU;
      out_sh[(base + r) * Q::RU + c] = sh[(g0 + s_lane[r]) * Q::RU + c];
    }
  }
}

size_t densify_workspace_bytes(int64_t n) {
  const int64_t nb = (n + kDensBlock - 1) / kDensBlock;
  return sizeof(uint64_t) * (size_t)(nb + 1) + 256;
}

static DensParams dev_params(const gs_densify_params& q) {
  DensParams p;
  p.grad_threshold = q.grad_threshold;
  p.scale_threshold = q.scale_threshold;
  p.split_shrink = q.split_shrink;
  p.min_opacity = q.min_opacity;
  p.max_scale = q.max_scale;
  p.use_abs = q.use_abs ? 1 : 0;
  p.split_n = q.split_n;
  return p;
}

// Count pass: per-workgroup output counts, their scan, the total at ws + sums (device).
hipError_t launch_densify_count(int64_t n, const float* scales, const float* opac, const float* accum,
                                const int32_t* denom, const gs_densify_params& q, void* ws, uint64_t** total,
                                hipStream_t s) {
  const int64_t nb = (n + kDensBlock - 1) / kDensBlock;
  uint64_t* sums = static_cast<uint64_t*>(ws);
  *total = sums + nb;
  if (nb > 0)
    k_densify_count<<<(unsigned)nb, kDensBlock, 0, s>>>(n, scales, opac, accum, denom, dev_params(q), sums);
  return launch_scan_sums(nb, sums, *total, s);
}

template <int L>
static void emit_L(int64_t nb, int64_t n, const float* means, const float* scales, const float* quats,
                   const float* opac, const float* sh, const float* accum, const int32_t* denom,
                   const float* normals, const DensParams& p, const uint64_t* sums, float* om, float* os,
                   float* oq, float* oo, float* osh, uint32_t* osrc, hipStream_t s) {
  k_densify_emit<L><<<(unsigned)nb, kDensBlock, 0, s>>>(
      n, means, scales, reinterpret_cast<const float4*>(quats), opac, sh, accum, denom, normals, p, sums, om, os,
      reinterpret_cast<float4*>(oq), oo, osh, osrc);
}

// Emission pass (the host has checked the total against the capacity).
hipError_t launch_densify_emit(int64_t n, const float* means, const float* scales, const float* quats,
                               const float* opac, const float* sh, int L, const float* accum, const int32_t* denom,
                               const float* normals, const gs_densify_params& q, const void* ws, float* om,
                               float* os, float* oq, float* oo, float* osh, uint32_t* osrc, hipStream_t s) {
  const int64_t nb = (n + kDensBlock - 1) / kDensBlock;
  if (nb == 0) return hipSuccess;
  const DensParams p = dev_params(q);
  const uint64_t* sums = static_cast<const uint64_t*>(ws);
  switch (L) {
    case 0: emit_L<0>(nb, n, means, scales, quats, opac, sh, accum, denom, normals, p, sums, om, os, oq, oo, osh, osrc, s); break;
    case 1: emit_L<1>(nb, n, means, scales, quats, opac, sh, accum, denom, normals, p, sums, om, os, oq, oo, osh, osrc, s); break;
    case 2: emit_L<2>(nb, n, means, scales, quats, opac, sh, accum, denom, normals, p, sums, om, os, oq, oo, osh, osrc, s); break;
    default: emit_L<3>(nb, n, means, scales, quats, opac, sh, accum, denom, normals, p, sums, om, os, oq, oo, osh, osrc, s); break;
  }
  return hipGetLastError();
}

}  // namespace gs
