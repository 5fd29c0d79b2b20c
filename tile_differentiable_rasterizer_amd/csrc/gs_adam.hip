// gs_adam.hip -- fused Adam step over float32 parameters with 16-bit packed moments, for
// gfx950.
//
// "Training 10M Gaussians in 8 GB: Spirula Studio's VRAM efficiency" (mhpq.cn), quantised
// training section: the Adam moments are stored as 16-bit codes packed side by side in a
// transposed (unit-major) layout, so a wavefront's 64 units are 256 contiguous bytes of
// state, with one (min, max) bounds pair per 256 units; gradients stay float32.  The update
// is Adam (Kingma and Ba) with bias correction.
//
// One wavefront per block of 256 units, four contiguous units per lane, one pass: decode
// both moments from
// the block's bounds, update them and the parameter in float64, reduce the block's new
// minimum and maximum of each moment (in the lane, then across the wavefront), and
// re-encode.  Constants enter
// as reciprocals computed once (1/65535, 1/(1 - beta^t), and 65535/(hi - lo) per block by one
// lane), which leaves one float64 division and one square root per unit.  The arithmetic is
// written in the order of its definition with contraction off, so the codes (integers
// decided by floating point) and the parameters are bit-exact against a float64 reference.
#include "gs_device.h"
#include "gs_wave.h"

namespace gs {

constexpr int kAdamBlock = 256;  // units per bounds block = lanes per workgroup
constexpr double kQMax = 65535.0;
constexpr double kInvQMax = 1.0 / 65535.0;

struct AdamConsts {
  double lr, b1, b2, eps, ib1, ib2;  // ib = 1 / (1 - beta^step)
};

__device__ __forceinline__ double decode_q16(uint32_t code, float lo, float hi) {
#pragma clang fp contract(off)
  const double l = lo, h = hi;
  return l + (double)code * ((h - l) * kInvQMax);
}

// scale = 65535 / (hi - lo) of the block; unused when hi == lo
__device__ __forceinline__ uint32_t encode_q16(double x, float lo, float hi, double scale) {
#pragma clang fp contract(off)
  const double l = lo, h = hi;
  if (h == l) return 0u;
  const double c = rint((x - l) * scale);
  return c <= 0.0 ? 0u : c >= kQMax ? 65535u : (uint32_t)c;
}

constexpr int kUnitsPerLane = kAdamBlock / kWave;  // 4: one wavefront owns one block

// Wavefront w of workgroup g owns block 4 g + w; lane l owns its units 4 l .. 4 l + 3 (16-byte
// accesses).  The block's extremes are the float32 roundings of its float64 moments (rounding
// is monotonic, so this rounds the float64 extremes; the values are finite), reduced inside
// the lane and then across the wavefront: no LDS, no barrier.
__global__ __launch_bounds__(kAdamBlock) void k_adam_q16(int64_t U, float* __restrict__ params,
                                                         const float* __restrict__ grads,
                                                         uint32_t* __restrict__ state, float4* __restrict__ bounds,
                                                         AdamConsts k) {
#pragma clang fp contract(off)
  constexpr int R = kUnitsPerLane;
  const int64_t nb = (U + kAdamBlock - 1) / kAdamBlock;
  const int64_t blk = (int64_t)blockIdx.x * (kAdamBlock / kWave) + threadIdx.x / kWave;
  if (blk >= nb) return;  // uniform per wavefront
  const int64_t u0 = blk * kAdamBlock + (int64_t)__lane_id() * R;
  const float4 bd = bounds[blk];  // m_lo, m_hi, v_lo, v_hi
  float pv[R], gv[R];
  uint32_t wv[R];
  const bool full = u0 + R <= U;
  if (full) {
    const float4 p4 = *reinterpret_cast<const float4*>(params + u0);
    const float4 g4 = *reinterpret_cast<const float4*>(grads + u0);
    const uint4 w4 = *reinterpret_cast<const uint4*>(state + u0);
    pv[0] = p4.x; pv[1] = p4.y; pv[2] = p4.z; pv[3] = p4.w;
    gv[0] = g4.x; gv[1] = g4.y; gv[2] = g4.z; gv[3] = g4.w;
    wv[0] = w4.x; wv[1] = w4.y; wv[2] = w4.z; wv[3] = w4.w;
  } else {
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const bool ok = u0 + r < U;
      pv[r] = ok ? params[u0 + r] : 0.0f;
      gv[r] = ok ? grads[u0 + r] : 0.0f;
      wv[r] = ok ? state[u0 + r] : 0u;
    }
  }
  double m[R], v[R];
  int mn = INT32_MAX, mx = INT32_MIN, vn = INT32_MAX, vx = INT32_MIN;
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const double g = gv[r];
    m[r] = decode_q16(wv[r] & 0xFFFFu, bd.x, bd.y);
    v[r] = decode_q16(wv[r] >> 16, bd.z, bd.w);
    m[r] = k.b1 * m[r] + (1.0 - k.b1) * g;
    v[r] = k.b2 * v[r] + (1.0 - k.b2) * (g * g);
    const double upd = k.lr * (m[r] * k.ib1) / (sqrt(v[r] * k.ib2) + k.eps);
    pv[r] = (float)((double)pv[r] - upd);
    if (u0 + r < U) {
      const int km = order_key((float)m[r]), kv = order_key((float)v[r]);
      mn = min(mn, km); mx = max(mx, km);
      vn = min(vn, kv); vx = max(vx, kv);
    }
  }
  const float mlo = key_float(wave_minmax<false>(mn)), mhi = key_float(wave_minmax<true>(mx));
  const float vlo = key_float(wave_minmax<false>(vn)), vhi = key_float(wave_minmax<true>(vx));
  const double sm = mhi == mlo ? 0.0 : kQMax / ((double)mhi - (double)mlo);
  const double sv = vhi == vlo ? 0.0 : kQMax / ((double)vhi - (double)vlo);
#pragma unroll
  for (int r = 0; r < R; ++r) wv[r] = encode_q16(m[r], mlo, mhi, sm) | (encode_q16(v[r], vlo, vhi, sv) << 16);
  if (full) {
    *reinterpret_cast<float4*>(params + u0) = make_float4(pv[0], pv[1], pv[2], pv[3]);
    *reinterpret_cast<uint4*>(state + u0) = make_uint4(wv[0], wv[1], wv[2], wv[3]);
  } else {
#pragma unroll
    for (int r = 0; r < R; ++r)
      if (u0 + r < U) {
        params[u0 + r] = pv[r];
        state[u0 + r] = wv[r];
      }
  }
  if (__lane_id() == 0) bounds[blk] = make_float4(mlo, mhi, vlo, vhi);
}

hipError_t launch_adam_q16(int64_t U, float* params, const float* grads, uint32_t* state, float* bounds,
                           const gs_adam_params& p, hipStream_t s) {
  if (U == 0) return hipSuccess;
  AdamConsts k;
  k.lr = (double)p.lr;
  k.b1 = (double)p.beta1;
  k.b2 = (double)p.beta2;
  k.eps = (double)p.eps;
  k.ib1 = 1.0 / (1.0 - pow(k.b1, (double)p.step));
  k.ib2 = 1.0 / (1.0 - pow(k.b2, (double)p.step));
  const int64_t nb = (U + kAdamBlock - 1) / kAdamBlock;
  const int64_t groups = (nb + kAdamBlock / kWave - 1) / (kAdamBlock / kWave);
  k_adam_q16<<<(unsigned)groups, kAdamBlock, 0, s>>>(U, params, grads, state, reinterpret_cast<float4*>(bounds), k);
  return hipGetLastError();
}

}  // namespace gs
