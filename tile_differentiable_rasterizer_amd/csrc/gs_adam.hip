// gs_adam.hip -- fused Adam step over float32 parameters with 16-bit packed moments, for
// gfx950.
//
// "Training 10M Gaussians in 8 GB: Spirula Studio's VRAM efficiency" (mhpq.cn), quantised
// training section: the Adam moments are stored as 16-bit codes packed side by side in a
// transposed (unit-major) layout, so a wavefront's 64 units are 256 contiguous bytes of
// state, with one (min, max) bounds pair per 256 units; gradients stay float32.  The update
// is Adam (Kingma and Ba) with bias correction.
//
// One workgroup per 256-unit block, one unit per lane, one pass: decode both moments from
// the block's bounds, update them and the parameter in float64, reduce the block's new
// minimum and maximum of each moment across the workgroup, and re-encode.  The arithmetic
// is written in the order of its definition with contraction off, so the codes (integers
// decided by floating point) and the parameters are bit-exact against a float64 reference.
#include "gs_device.h"

namespace gs {

constexpr int kAdamBlock = 256;  // units per bounds block = lanes per workgroup
constexpr double kQMax = 65535.0;

struct AdamConsts {
  double lr, b1, b2, eps, bc1, bc2;  // bc = 1 - beta^step
};

__device__ __forceinline__ double decode_q16(uint32_t code, float lo, float hi) {
#pragma clang fp contract(off)
  const double l = lo, h = hi;
  return l + (double)code * ((h - l) / kQMax);
}

__device__ __forceinline__ uint32_t encode_q16(double x, float lo, float hi) {
#pragma clang fp contract(off)
  const double l = lo, h = hi;
  if (h == l) return 0u;
  const double c = rint((x - l) / (h - l) * kQMax);
  return c <= 0.0 ? 0u : c >= kQMax ? 65535u : (uint32_t)c;
}

// Minimum and maximum over the workgroup (valid lanes only), returned to every lane.
__device__ __forceinline__ void block_minmax(double& mn, double& mx, double* s_mn, double* s_mx) {
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) {
    mn = fmin(mn, __shfl_xor(mn, d, kWave));
    mx = fmax(mx, __shfl_xor(mx, d, kWave));
  }
  const int wave = threadIdx.x / kWave;
  if (__lane_id() == 0) {
    s_mn[wave] = mn;
    s_mx[wave] = mx;
  }
  __syncthreads();
  mn = s_mn[0];
  mx = s_mx[0];
#pragma unroll
  for (int w = 1; w < kAdamBlock / kWave; ++w) {
    mn = fmin(mn, s_mn[w]);
    mx = fmax(mx, s_mx[w]);
  }
}

__global__ __launch_bounds__(kAdamBlock) void k_adam_q16(int64_t U, float* __restrict__ params,
                                                         const float* __restrict__ grads,
                                                         uint32_t* __restrict__ state, float4* __restrict__ bounds,
                                                         AdamConsts k) {
#pragma clang fp contract(off)
  __shared__ double s_m[2][kAdamBlock / kWave], s_v[2][kAdamBlock / kWave];
  const int64_t u = (int64_t)blockIdx.x * kAdamBlock + threadIdx.x;
  const bool valid = u < U;
  const float4 bd = bounds[blockIdx.x];  // m_lo, m_hi, v_lo, v_hi
  double m = 0.0, v = 0.0;
  if (valid) {
    const uint32_t w = state[u];
    const double g = grads[u];
    m = decode_q16(w & 0xFFFFu, bd.x, bd.y);
    v = decode_q16(w >> 16, bd.z, bd.w);
    m = k.b1 * m + (1.0 - k.b1) * g;
    v = k.b2 * v + (1.0 - k.b2) * (g * g);
    const double upd = k.lr * (m / k.bc1) / (sqrt(v / k.bc2) + k.eps);
    params[u] = (float)((double)params[u] - upd);
  }
  double mn = valid ? m : INFINITY, mx = valid ? m : -INFINITY;
  block_minmax(mn, mx, s_m[0], s_m[1]);
  double vn = valid ? v : INFINITY, vx = valid ? v : -INFINITY;
  block_minmax(vn, vx, s_v[0], s_v[1]);
  const float mlo = (float)mn, mhi = (float)mx, vlo = (float)vn, vhi = (float)vx;
  if (valid) state[u] = encode_q16(m, mlo, mhi) | (encode_q16(v, vlo, vhi) << 16);
  if (threadIdx.x == 0) bounds[blockIdx.x] = make_float4(mlo, mhi, vlo, vhi);
}

hipError_t launch_adam_q16(int64_t U, float* params, const float* grads, uint32_t* state, float* bounds,
                           const gs_adam_params& p, hipStream_t s) {
  if (U == 0) return hipSuccess;
  AdamConsts k;
  k.lr = (double)p.lr;
  k.b1 = (double)p.beta1;
  k.b2 = (double)p.beta2;
  k.eps = (double)p.eps;
  k.bc1 = 1.0 - pow(k.b1, (double)p.step);
  k.bc2 = 1.0 - pow(k.b2, (double)p.step);
  const int64_t nb = (U + kAdamBlock - 1) / kAdamBlock;
  k_adam_q16<<<(unsigned)nb, kAdamBlock, 0, s>>>(U, params, grads, state, reinterpret_cast<float4*>(bounds), k);
  return hipGetLastError();
}

}  // namespace gs
