// gs_device.h -- device-side constants and helpers shared by the gfx950 kernels.
// Internal to libgsraster; not part of the C ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/gs_raster.h"

namespace gs {

constexpr int kTile = GS_TILE;
constexpr int kRec = GS_REC_FLOATS;
constexpr int kWave = 64;

// Thresholds of the compositing rule, as fp32 constants.
constexpr float kAlphaMax = 0.99f;
constexpr float kAlphaMin = 1.0f / 255.0f;
constexpr float kTMin = 1e-4f;
constexpr float kLog2e = 1.4426950408889634f;

// Camera as the kernels see it: float64 copy of the fp32 camera plus derived values.
struct DevCamera {
  double R[9];
  double t[3];
  double fx, fy, cx, cy, near_z;
  double campos[3];  // -R^T t
  int32_t width, height, tiles_x, tiles_y;
};

__device__ __forceinline__ uint64_t lanemask_lt() {
  const uint32_t lane = __lane_id();
  return lane == 0 ? 0ull : (~0ull >> (64 - lane));
}

// Inclusive prefix sum across a 64-wide wavefront.
template <typename T>
__device__ __forceinline__ T wave_inclusive_scan(T x) {
  const int lane = __lane_id();
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    T y = __shfl_up(x, d, 64);
    if (lane >= d) x += y;
  }
  return x;
}

// Lanes of the calling wavefront (among `active`) whose `bits`-bit digit equals this lane's:
// the intersection of one ballot per digit bit.
__device__ __forceinline__ uint64_t match_digit(uint32_t d, int bits, uint64_t active) {
  uint64_t m = active;
  for (int b = 0; b < bits; ++b) {
    const bool bit = (d >> b) & 1u;
    const uint64_t bb = __ballot(bit);
    m &= bit ? bb : ~bb;
  }
  return m;
}

template <typename T>
__device__ __forceinline__ T wave_sum(T x) {
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) x += __shfl_xor(x, d, 64);
  return x;
}

template <typename T>
__device__ __forceinline__ T wave_max(T x) {
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) {
    T y = __shfl_xor(x, d, 64);
    x = y > x ? y : x;
  }
  return x;
}

}  // namespace gs
