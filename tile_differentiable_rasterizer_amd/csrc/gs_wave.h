// gs_wave.h -- wavefront-wide reductions for the 64-lane gfx950 wavefront.
// Internal to libgsraster.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gs {

template <int kCtrl, int kRowMask>
__device__ __forceinline__ float dpp_get(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), kCtrl, kRowMask, 0xF, false));
}

// Sum over the 64 lanes; the total lands in lane 63.  DPP row operations reduce each row
// of 16, then row broadcasts fold the four rows.
__device__ __forceinline__ float wave_reduce_to_last(float v) {
  v += dpp_get<0xB1, 0xF>(v);   // quad_perm [1,0,3,2]
  v += dpp_get<0x4E, 0xF>(v);   // quad_perm [2,3,0,1]
  v += dpp_get<0x141, 0xF>(v);  // row_half_mirror
  v += dpp_get<0x140, 0xF>(v);  // row_mirror
  v += dpp_get<0x142, 0xA>(v);  // row_bcast:15 into rows 1 and 3
  v += dpp_get<0x143, 0xC>(v);  // row_bcast:31 into rows 2 and 3
  return v;
}

// Transposed reduction of 30 per-lane values: on return lanes 2i and 2i + 1 (i < 30) hold
// the sum over all 64 lanes of v[i]; lanes 60..63 hold values of no use.  Each butterfly
// step halves the values a lane keeps: bit 5 and bit 4 of the lane id with the gfx950
// half/row swaps, bits 3 and 2 with two DPP adds per pair whose bank masks write the two
// halves of each row or half row (a row rotate by 8, then a half-row mirror, reads the
// partner lane), bit 1 with DPP (quad permute)
// and a select of the half to keep; the last step (bit 0) adds the one remaining value of
// the neighbouring lane.  About 62 instructions for 30 sums, against 6 per value for
// independent reductions.
//
// The two-add steps are inline assembly (the compiler forms DPP adds with partial bank
// masks only for an identity "old" value).  A DPP operand must be written at least two
// wait states before it is read: each block starts with s_nop 1, and inside a block no
// instruction reads through DPP a register that an earlier one in the block wrote.  The
// wavefront's lanes are all active wherever this is called.
__device__ __forceinline__ void dpp_pair_step8(float& y, float a, float b) {
  // lanes 0-7 of each row: a + a(lane ^ 8); lanes 8-15: b + b(lane ^ 8)
  asm volatile(
      "s_nop 1\n\t"
      "v_add_f32_dpp %0, %1, %1 row_ror:8 row_mask:0xf bank_mask:0x3\n\t"
      "v_add_f32_dpp %0, %2, %2 row_ror:8 row_mask:0xf bank_mask:0xc"
      : "=&v"(y)
      : "v"(a), "v"(b));
}
__device__ __forceinline__ void dpp_pair_step4(float& y, float a, float b) {
  // the partner is the mirror lane inside the half row (bit 2 differs): lanes with bit 2
  // clear (banks 0, 2) take a + a(partner), lanes with it set (banks 1, 3) b + b(partner)
  asm volatile(
      "s_nop 1\n\t"
      "v_add_f32_dpp %0, %1, %1 row_half_mirror row_mask:0xf bank_mask:0x5\n\t"
      "v_add_f32_dpp %0, %2, %2 row_half_mirror row_mask:0xf bank_mask:0xa"
      : "=&v"(y)
      : "v"(a), "v"(b));
}

__device__ __forceinline__ float wave_transpose_reduce30(const float (&v)[30]) {
  const int lane = __lane_id();
  float w[16];
  uint32_t spare = 0;  // a register whose value no longer matters, partner of values 14, 15
#pragma unroll
  for (int i = 0; i < 16; ++i) {  // lanes < 32 keep v[i], lanes >= 32 keep v[i + 16]
    const uint32_t hi = i + 16 < 30 ? __float_as_uint(v[i + 16]) : spare;
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v[i]), hi, false, false);
    w[i] = __uint_as_float(r[0]) + __uint_as_float(r[1]);
    spare = r[1];
  }
  float x[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {  // rows 0, 2 keep w[i]; rows 1, 3 keep w[i + 8]
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(w[i]), __float_as_uint(w[i + 8]), false, false);
    x[i] = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  }
  float y[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) dpp_pair_step8(y[i], x[i], x[i + 4]);  // lanes 0-7 of a row keep x[i]
  float z[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) dpp_pair_step4(z[i], y[i], y[i + 2]);  // bit 2 clear keeps y[i]
  const bool b1 = (lane >> 1) & 1;
  const float keep = b1 ? z[1] : z[0], send = b1 ? z[0] : z[1];
  float t = keep + dpp_get<0x4E, 0xF>(send);  // partner: lane ^ 2
  return t + dpp_get<0xB1, 0xF>(t);            // partner: lane ^ 1
}

// float32 <-> int32 keys whose signed order is the floats' order (negative floats have
// their magnitude bits flipped), so extremes reduce with integer min / max.
__device__ __forceinline__ int order_key(float f) {
  const int b = __float_as_int(f);
  return b < 0 ? b ^ 0x7FFFFFFF : b;
}
__device__ __forceinline__ float key_float(int k) { return __int_as_float(k < 0 ? k ^ 0x7FFFFFFF : k); }

// Minimum (kMax = false) or maximum key over the wavefront, in every lane: DPP steps within
// rows, row broadcasts across them (the result gathers in lane 63), then a read of lane 63.
// Lanes a row mask leaves out take the identity, so only lane 63's value matters.
template <bool kMax>
__device__ __forceinline__ int wave_minmax(int v) {
  constexpr int id = kMax ? INT32_MIN : INT32_MAX;
  auto step = [](int x, int y) { return kMax ? max(x, y) : min(x, y); };
  v = step(v, __builtin_amdgcn_update_dpp(id, v, 0xB1, 0xF, 0xF, false));   // quad_perm [1,0,3,2]
  v = step(v, __builtin_amdgcn_update_dpp(id, v, 0x4E, 0xF, 0xF, false));   // quad_perm [2,3,0,1]
  v = step(v, __builtin_amdgcn_update_dpp(id, v, 0x141, 0xF, 0xF, false));  // row_half_mirror
  v = step(v, __builtin_amdgcn_update_dpp(id, v, 0x140, 0xF, 0xF, false));  // row_mirror
  v = step(v, __builtin_amdgcn_update_dpp(id, v, 0x142, 0xA, 0xF, false));  // row_bcast:15 into rows 1, 3
  v = step(v, __builtin_amdgcn_update_dpp(id, v, 0x143, 0xC, 0xF, false));  // row_bcast:31 into rows 2, 3
  return __builtin_amdgcn_readlane(v, 63);
}

}  // namespace gs
