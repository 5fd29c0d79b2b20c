// gs_qsh.hip -- q8 / q16 codes of SH coefficients with (min, max) bounds per 256 units, for
// gfx950.
//
// "Training 10M Gaussians in 8 GB: Spirula Studio's VRAM efficiency" (mhpq.cn), quantised
// training section: SH coefficients kept as 8- or 16-bit fixed-point codes with a (min, max)
// table, one pair per 256 units.  The units are the coefficients in their [n][K][3] order.
// A code is rint((x - lo) * (qmax / (hi - lo))) in float64, clamped (0 when hi == lo); the
// projection decodes lo + code * ((hi - lo) * (1 / qmax)) in float32 (gs_project.hip).
//
// One wavefront per 256-unit block, four contiguous units per lane: the block's extremes
// reduce inside the lane and across the wavefront (order-preserving integer keys with DPP),
// with no LDS and no barrier.
#include "gs_device.h"
#include "gs_wave.h"

namespace gs {

constexpr int kQBlock = 256;                 // units per bounds pair
constexpr int kQPerLane = kQBlock / kWave;   // 4

template <int QB>
__global__ __launch_bounds__(256) void k_quantize_sh(int64_t U, const float* __restrict__ x, void* __restrict__ codes,
                                                     float2* __restrict__ bounds) {
#pragma clang fp contract(off)
  using Code = typename std::conditional<QB == 16, uint16_t, uint8_t>::type;
  constexpr double kQ = QB == 16 ? 65535.0 : 255.0;
  const int64_t nb = (U + kQBlock - 1) / kQBlock;
  const int64_t blk = (int64_t)blockIdx.x * (256 / kWave) + threadIdx.x / kWave;
  if (blk >= nb) return;  // uniform per wavefront
  const int64_t u0 = blk * kQBlock + (int64_t)__lane_id() * kQPerLane;
  float v[kQPerLane];
  const bool full = u0 + kQPerLane <= U;
  if (full) {
    const float4 a = *reinterpret_cast<const float4*>(x + u0);
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
  } else {
#pragma unroll
    for (int r = 0; r < kQPerLane; ++r) v[r] = u0 + r < U ? x[u0 + r] : 0.0f;
  }
  int kn = INT32_MAX, kx = INT32_MIN;
#pragma unroll
  for (int r = 0; r < kQPerLane; ++r)
    if (u0 + r < U) {
      const int k = order_key(v[r]);
      kn = min(kn, k);
      kx = max(kx, k);
    }
  const float lo = key_float(wave_minmax<false>(kn)), hi = key_float(wave_minmax<true>(kx));
  const double scale = hi == lo ? 0.0 : kQ / ((double)hi - (double)lo);
  Code c[kQPerLane];
#pragma unroll
  for (int r = 0; r < kQPerLane; ++r) {
    const double q = hi == lo ? 0.0 : rint(((double)v[r] - (double)lo) * scale);
    c[r] = (Code)(q <= 0.0 ? 0.0 : q >= kQ ? kQ : q);
  }
  Code* out = static_cast<Code*>(codes);
  if (full) {
    if constexpr (QB == 16)
      *reinterpret_cast<uint2*>(out + u0) = make_uint2((uint32_t)c[0] | ((uint32_t)c[1] << 16),
                                                       (uint32_t)c[2] | ((uint32_t)c[3] << 16));
    else
      *reinterpret_cast<uint32_t*>(out + u0) =
          (uint32_t)c[0] | ((uint32_t)c[1] << 8) | ((uint32_t)c[2] << 16) | ((uint32_t)c[3] << 24);
  } else {
#pragma unroll
    for (int r = 0; r < kQPerLane; ++r)
      if (u0 + r < U) out[u0 + r] = c[r];
  }
  if (__lane_id() == 0) bounds[blk] = make_float2(lo, hi);
}

hipError_t launch_quantize_sh(int64_t U, const float* sh, int bits, void* codes, float* bounds, hipStream_t s) {
  if (U == 0) return hipSuccess;
  const int64_t nb = (U + kQBlock - 1) / kQBlock;
  const unsigned groups = (unsigned)((nb + 3) / 4);
  if (bits == 16)
    k_quantize_sh<16><<<groups, 256, 0, s>>>(U, sh, codes, reinterpret_cast<float2*>(bounds));
  else
    k_quantize_sh<8><<<groups, 256, 0, s>>>(U, sh, codes, reinterpret_cast<float2*>(bounds));
  return hipGetLastError();
}

}  // namespace gs
