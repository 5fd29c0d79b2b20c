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

// Decoupled look-back (the chained scan of Merrill & Garland) over per-partition status
// words, one column per counter: a word holds a 62-bit value and a flag, 0 while
// unpublished, kFlagAgg for the partition's own count, kFlagPre for the inclusive prefix
// through it.  Status words are read and written at device scope, with no fences: a word
// carries its own flag.
constexpr uint64_t kFlagAgg = 1ull << 62;
constexpr uint64_t kFlagPre = 2ull << 62;
constexpr uint64_t kValMask = (1ull << 62) - 1;
constexpr int kLookBack = 4;  // status words read per look-back round trip

__device__ __forceinline__ uint64_t status_load(const uint64_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void status_store(uint64_t* p, uint64_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Exclusive prefix of partition `part` (> 0) in one column: sums the published values of
// the partitions before it, kLookBack words per round trip, back to the first inclusive
// prefix; a word not yet published ends the round and the next round starts at it.
// `col` points at the column's word of partition 0, `stride` words apart per partition;
// `early` is the predecessor's word if already read (else 0).  Every partition before
// `part` must already be running (partitions go out in order, by ticket).
__device__ __forceinline__ uint64_t lookback_exclusive(const uint64_t* col, int64_t stride, int64_t part,
                                                       uint64_t early) {
  uint64_t excl = 0;
  int64_t p = part - 1;
  while (true) {
    uint64_t sv[kLookBack];
    sv[0] = (early & ~kValMask) ? early : status_load(col + p * stride);
    early = 0;
#pragma unroll
    for (int i = 1; i < kLookBack; ++i) sv[i] = p - i >= 0 ? status_load(col + (p - i) * stride) : 0;
    int used = 0;
    bool done = false;
#pragma unroll
    for (int i = 0; i < kLookBack; ++i) {
      if (done || used < i) continue;  // stopped at an inclusive prefix or an unpublished word
      const uint64_t flag = sv[i] & ~kValMask;
      if (flag == 0) continue;
      excl += sv[i] & kValMask;
      used = i + 1;
      done = flag == kFlagPre;
    }
    if (done) return excl;
    p -= used;
    if (used < kLookBack) __builtin_amdgcn_s_sleep(1);
  }
}

// One DPP move of a 32-bit word: lanes whose source lies outside their row (or whose row the
// row mask leaves out) receive 0.
template <int kCtrl, int kRowMask>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t x) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, kCtrl, kRowMask, 0xF, false);
}
template <int kCtrl, int kRowMask>
__device__ __forceinline__ uint64_t dpp_u64(uint64_t x) {
  const uint32_t lo = dpp_u32<kCtrl, kRowMask>((uint32_t)x), hi = dpp_u32<kCtrl, kRowMask>((uint32_t)(x >> 32));
  return ((uint64_t)hi << 32) | lo;
}
template <int kCtrl, int kRowMask, typename T>
__device__ __forceinline__ T dpp_move(T x) {
  static_assert(sizeof(T) == 4 || sizeof(T) == 8, "32- or 64-bit words");
  if constexpr (sizeof(T) == 8)
    return (T)dpp_u64<kCtrl, kRowMask>((uint64_t)x);
  else
    return (T)dpp_u32<kCtrl, kRowMask>((uint32_t)x);
}

// Inclusive prefix sum across a 64-wide wavefront (every lane active), with DPP moves and no
// LDS round trips: shifts right by 1, 2, 4 and 8 within each row of 16 lanes scan the rows;
// the last lane of row 0 (2) is then added into row 1 (3), and the last lane of row 1 into
// rows 2 and 3.
template <typename T>
__device__ __forceinline__ T wave_inclusive_scan(T x) {
  x += dpp_move<0x111, 0xF>(x);  // row_shr:1
  x += dpp_move<0x112, 0xF>(x);  // row_shr:2
  x += dpp_move<0x114, 0xF>(x);  // row_shr:4
  x += dpp_move<0x118, 0xF>(x);  // row_shr:8
  x += dpp_move<0x142, 0xA>(x);  // row_bcast:15 into rows 1 and 3
  x += dpp_move<0x143, 0xC>(x);  // row_bcast:31 into rows 2 and 3
  return x;
}

// Lanes of the calling wavefront (among `active`) whose `bits`-bit digit equals this lane's:
// one ballot per digit bit gives the lanes with that bit set; flipped where this lane's bit
// is set, it is the lanes that differ from this one in that bit, and the lanes that differ
// in no bit match.  A bit costs four instructions: the bit as a 0 / all-ones word (one
// bitfield extract, kept opaque so that the ballot compares that word), the ballot's
// compare, and per half of the 64-lane mask one three-input logic op that ors in the
// exclusive-or (truth table 0xde over (s, differ, ones)).
__device__ __forceinline__ uint64_t match_digit(uint32_t d, int bits, uint64_t active) {
  uint32_t differ_lo = 0, differ_hi = 0;
  for (int b = 0; b < bits; ++b) {
    uint32_t s;  // 0 or 0xFFFFFFFF
    asm("v_bfe_i32 %0, %1, %2, 1" : "=v"(s) : "v"(d), "s"(b));
    const uint64_t ones = __ballot(s != 0u);
    differ_lo = __builtin_amdgcn_bitop3_b32(s, differ_lo, (uint32_t)ones, 0xde);
    differ_hi = __builtin_amdgcn_bitop3_b32(s, differ_hi, (uint32_t)(ones >> 32), 0xde);
  }
  return active & ~(((uint64_t)differ_hi << 32) | differ_lo);
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
