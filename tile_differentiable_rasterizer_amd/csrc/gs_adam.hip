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
// both moments from the block's bounds and update them in float64 (the codes are decided on
// these values, so they stay within a few float64 roundings of the definition's), update
// the parameter in float32 (it is stored in float32: the bias-corrected moments rounded to
// float32, the hardware square root and reciprocal, about 5e-7 relative), reduce the
// block's new minimum and maximum of each moment (in the lane, then across the wavefront)
// and re-encode.  Constants enter as reciprocals computed once (1/65535, 1/(1 - beta^t), and
// 65535/(hi - lo) per block), so no unit pays a division or a float64 square root: the
// pass is bound by its 20 bytes per unit.
//
// The second form (k_fpbo_pack, k_adam_fpbo) keeps the parameters as 16-bit codes too, as the
// page's fused layout does, so a step moves 16 bytes per unit (20 with the decoded float32
// parameters written for a renderer).
#include "gs_device.h"
#include "gs_wave.h"

namespace gs {

constexpr int kAdamBlock = 256;  // units per bounds block = lanes per workgroup
constexpr double kQMax = 65535.0;
constexpr double kInvQMax = 1.0 / 65535.0;

struct AdamConsts {
  double b1, b2, c1, c2, ib1, ib2;  // c = 1 - beta, ib = 1 / (1 - beta^step)
  float lr, eps;
};

// step = (hi - lo) / 65535 of the block, as (hi - lo) * (1 / 65535)
__device__ __forceinline__ double decode_q16(uint32_t code, float lo, double step) {
#pragma clang fp contract(off)
  return (double)lo + (double)code * step;
}

// scale = 65535 / (hi - lo) of the block, 0 when hi == lo (every code is then 0); the clamp
// to [0, 65535] is a float64 max and min
__device__ __forceinline__ uint32_t encode_q16(double x, float lo, double scale) {
#pragma clang fp contract(off)
  const double c = rint((x - (double)lo) * scale);
  return (uint32_t)fmin(fmax(c, 0.0), kQMax);
}

constexpr int kUnitsPerLane = kAdamBlock / kWave;  // 4: one wavefront owns one block

// Wavefront w of workgroup g owns block 4 g + w; lane l owns its units 4 l .. 4 l + 3 (16-byte
// accesses).  The block's extremes are the float32 roundings of its float64 moments (rounding
// is monotonic, so this rounds the float64 extremes; the values are finite), reduced inside
// the lane and then across the wavefront: no LDS, no barrier.  kFull: every unit of the block
// is below U (all blocks but a ragged last one), so no unit needs a bounds test.
template <bool kFull>
__device__ __forceinline__ void adam_q16_block(int64_t U, int64_t blk, float* __restrict__ params,
                                               const float* __restrict__ grads, uint32_t* __restrict__ state,
                                               float4* __restrict__ bounds, const AdamConsts& k) {
#pragma clang fp contract(off)
  constexpr int R = kUnitsPerLane;
  const int64_t u0 = blk * kAdamBlock + (int64_t)__lane_id() * R;
  const float4 bd = bounds[blk];  // m_lo, m_hi, v_lo, v_hi
  float pv[R], gv[R];
  uint32_t wv[R];
  const bool full = kFull || u0 + R <= U;
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
  const double mstep = ((double)bd.y - (double)bd.x) * kInvQMax;
  const double vstep = ((double)bd.w - (double)bd.z) * kInvQMax;
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const double g = gv[r];
    m[r] = decode_q16(wv[r] & 0xFFFFu, bd.x, mstep);
    v[r] = decode_q16(wv[r] >> 16, bd.z, vstep);
    m[r] = k.b1 * m[r] + k.c1 * g;
    v[r] = k.b2 * v[r] + k.c2 * (g * g);
    // the parameter's step in float32: lr m_hat / (sqrt(v_hat) + eps)
    const float mh = (float)(m[r] * k.ib1), vh = (float)(v[r] * k.ib2);
    const float den = __builtin_amdgcn_sqrtf(vh) + k.eps;
    const float upd = k.lr * mh * __builtin_amdgcn_rcpf(den);
    pv[r] = (float)((double)pv[r] - (double)upd);
    if (kFull || u0 + r < U) {
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
  for (int r = 0; r < R; ++r) wv[r] = encode_q16(m[r], mlo, sm) | (encode_q16(v[r], vlo, sv) << 16);
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

__global__ __launch_bounds__(kAdamBlock) void k_adam_q16(int64_t U, float* __restrict__ params,
                                                         const float* __restrict__ grads,
                                                         uint32_t* __restrict__ state, float4* __restrict__ bounds,
                                                         AdamConsts k) {
  const int64_t nb = (U + kAdamBlock - 1) / kAdamBlock;
  const int64_t blk = (int64_t)blockIdx.x * (kAdamBlock / kWave) + threadIdx.x / kWave;
  if (blk >= nb) return;  // uniform per wavefront
  if ((blk + 1) * kAdamBlock <= U)
    adam_q16_block<true>(U, blk, params, grads, state, bounds, k);
  else
    adam_q16_block<false>(U, blk, params, grads, state, bounds, k);
}

// Parameters packed too.  The same page keeps the parameters as 16-bit codes beside both
// moments; here a block of 256 units is three transposed planes of 256 uint16 codes (the
// parameters', the first moments', the second moments'), 1536 bytes, with three (lo, hi)
// pairs of float32 bounds.  Lane l owns units 4 l .. 4 l + 3 of its wavefront's block, one
// 8-byte word of each plane, so a plane is 512 contiguous bytes per wavefront.  The
// parameter is decoded and updated in float64 like the moments, its step taken in float32
// as above, and re-encoded with its block's new bounds; codes past the last unit are 0.
constexpr int kPlaneWords = kAdamBlock / kUnitsPerLane;  // uint2 words per plane of a block

__device__ __forceinline__ void unpack4(uint2 w, uint32_t c[4]) {
  c[0] = w.x & 0xFFFFu; c[1] = w.x >> 16; c[2] = w.y & 0xFFFFu; c[3] = w.y >> 16;
}
__device__ __forceinline__ uint2 pack4(const uint32_t c[4]) { return make_uint2(c[0] | (c[1] << 16), c[2] | (c[3] << 16)); }

// The block's float32 gradients (or parameters) of this lane, 0 past the last unit.  kFull:
// every unit of the block is below U (no bounds tests).
template <bool kFull>
__device__ __forceinline__ void load4(const float* __restrict__ x, int64_t u0, int64_t U, float v[4]) {
  if (kFull || u0 + kUnitsPerLane <= U) {
    const float4 q = *reinterpret_cast<const float4*>(x + u0);
    v[0] = q.x; v[1] = q.y; v[2] = q.z; v[3] = q.w;
  } else {
#pragma unroll
    for (int r = 0; r < kUnitsPerLane; ++r) v[r] = u0 + r < U ? x[u0 + r] : 0.0f;
  }
}

template <bool kFull>
__device__ __forceinline__ void store4(float* __restrict__ x, int64_t u0, int64_t U, const float v[4]) {
  if (kFull || u0 + kUnitsPerLane <= U) {
    *reinterpret_cast<float4*>(x + u0) = make_float4(v[0], v[1], v[2], v[3]);
  } else {
#pragma unroll
    for (int r = 0; r < kUnitsPerLane; ++r)
      if (u0 + r < U) x[u0 + r] = v[r];
  }
}

// Block bounds (lo, hi) of the float32 roundings of x over this lane's units below U, reduced
// across the wavefront.
template <bool kFull>
__device__ __forceinline__ float2 block_bounds(const double x[4], int64_t u0, int64_t U) {
  int lo = INT32_MAX, hi = INT32_MIN;
#pragma unroll
  for (int r = 0; r < kUnitsPerLane; ++r)
    if (kFull || u0 + r < U) {
      const int kx = order_key((float)x[r]);
      lo = min(lo, kx);
      hi = max(hi, kx);
    }
  return make_float2(key_float(wave_minmax<false>(lo)), key_float(wave_minmax<true>(hi)));
}

// Codes of x with the block's bounds b, 0 past the last unit.
template <bool kFull>
__device__ __forceinline__ uint2 encode4(const double x[4], float2 b, int64_t u0, int64_t U) {
  const double sc = b.y == b.x ? 0.0 : kQMax / ((double)b.y - (double)b.x);
  uint32_t c[kUnitsPerLane];
#pragma unroll
  for (int r = 0; r < kUnitsPerLane; ++r) c[r] = kFull || u0 + r < U ? encode_q16(x[r], b.x, sc) : 0u;
  return pack4(c);
}

// Initial packed state: the parameters' codes, both moments zero.
template <bool kFull>
__device__ __forceinline__ void fpbo_pack_block(int64_t U, int64_t blk, const float* __restrict__ params,
                                                uint2* __restrict__ state, float2* __restrict__ bounds) {
  const int lane = (int)__lane_id();
  const int64_t u0 = blk * kAdamBlock + (int64_t)lane * kUnitsPerLane;
  float pv[kUnitsPerLane];
  load4<kFull>(params, u0, U, pv);
  double x[kUnitsPerLane];
#pragma unroll
  for (int r = 0; r < kUnitsPerLane; ++r) x[r] = pv[r];
  const float2 b = block_bounds<kFull>(x, u0, U);
  uint2* st = state + blk * 3 * kPlaneWords;
  st[lane] = encode4<kFull>(x, b, u0, U);
  st[kPlaneWords + lane] = make_uint2(0u, 0u);
  st[2 * kPlaneWords + lane] = make_uint2(0u, 0u);
  if (lane == 0) {
    bounds[3 * blk] = b;
    bounds[3 * blk + 1] = make_float2(0.0f, 0.0f);
    bounds[3 * blk + 2] = make_float2(0.0f, 0.0f);
  }
}

__global__ __launch_bounds__(kAdamBlock) void k_fpbo_pack(int64_t U, const float* __restrict__ params,
                                                          uint2* __restrict__ state, float2* __restrict__ bounds) {
  const int64_t nb = (U + kAdamBlock - 1) / kAdamBlock;
  const int64_t blk = (int64_t)blockIdx.x * (kAdamBlock / kWave) + threadIdx.x / kWave;
  if (blk >= nb) return;  // uniform per wavefront
  if ((blk + 1) * kAdamBlock <= U)
    fpbo_pack_block<true>(U, blk, params, state, bounds);
  else
    fpbo_pack_block<false>(U, blk, params, state, bounds);
}

template <bool kFull>
__device__ __forceinline__ void adam_fpbo_block(int64_t U, int64_t blk, uint2* __restrict__ state,
                                                float2* __restrict__ bounds, const float* __restrict__ grads,
                                                float* __restrict__ params_out, const AdamConsts& k) {
#pragma clang fp contract(off)
  constexpr int R = kUnitsPerLane;
  const int lane = (int)__lane_id();
  const int64_t u0 = blk * kAdamBlock + (int64_t)lane * R;
  uint2* st = state + blk * 3 * kPlaneWords;
  const float2 bp = bounds[3 * blk], bm = bounds[3 * blk + 1], bv = bounds[3 * blk + 2];
  uint32_t cp[R], cm[R], cv[R];
  unpack4(st[lane], cp);
  unpack4(st[kPlaneWords + lane], cm);
  unpack4(st[2 * kPlaneWords + lane], cv);
  float gv[R];
  load4<kFull>(grads, u0, U, gv);
  const double pstep = ((double)bp.y - (double)bp.x) * kInvQMax;
  const double mstep = ((double)bm.y - (double)bm.x) * kInvQMax;
  const double vstep = ((double)bv.y - (double)bv.x) * kInvQMax;
  double th[R], m[R], v[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const double g = gv[r];
    th[r] = decode_q16(cp[r], bp.x, pstep);
    m[r] = decode_q16(cm[r], bm.x, mstep);
    v[r] = decode_q16(cv[r], bv.x, vstep);
    m[r] = k.b1 * m[r] + k.c1 * g;
    v[r] = k.b2 * v[r] + k.c2 * (g * g);
    const float mh = (float)(m[r] * k.ib1), vh = (float)(v[r] * k.ib2);
    const float den = __builtin_amdgcn_sqrtf(vh) + k.eps;
    const float upd = k.lr * mh * __builtin_amdgcn_rcpf(den);
    th[r] = th[r] - (double)upd;
  }
  const float2 np = block_bounds<kFull>(th, u0, U), nm = block_bounds<kFull>(m, u0, U),
               nv = block_bounds<kFull>(v, u0, U);
  const uint2 wp = encode4<kFull>(th, np, u0, U);
  st[lane] = wp;
  st[kPlaneWords + lane] = encode4<kFull>(m, nm, u0, U);
  st[2 * kPlaneWords + lane] = encode4<kFull>(v, nv, u0, U);
  if (lane == 0) {
    bounds[3 * blk] = np;
    bounds[3 * blk + 1] = nm;
    bounds[3 * blk + 2] = nv;
  }
  if (params_out) {  // the parameters as stored: their new codes decoded, rounded once
    uint32_t c[R];
    unpack4(wp, c);
    const double step = ((double)np.y - (double)np.x) * kInvQMax;
    float pv[R];
#pragma unroll
    for (int r = 0; r < R; ++r) pv[r] = (float)decode_q16(c[r], np.x, step);
    store4<kFull>(params_out, u0, U, pv);
  }
}

hipError_t launch_adam_q16(int64_t U, float* params, const float* grads, uint32_t* state, float* bounds,
                           const gs_adam_params& p, hipStream_t s) {
  if (U == 0) return hipSuccess;
  AdamConsts k;
  k.lr = p.lr;
  k.eps = p.eps;
  k.b1 = (double)p.beta1;
  k.b2 = (double)p.beta2;
  k.c1 = 1.0 - k.b1;
  k.c2 = 1.0 - k.b2;
  k.ib1 = 1.0 / (1.0 - pow(k.b1, (double)p.step));
  k.ib2 = 1.0 / (1.0 - pow(k.b2, (double)p.step));
  const int64_t nb = (U + kAdamBlock - 1) / kAdamBlock;
  const int64_t groups = (nb + kAdamBlock / kWave - 1) / (kAdamBlock / kWave);
  k_adam_q16<<<(unsigned)groups, kAdamBlock, 0, s>>>(U, params, grads, state, reinterpret_cast<float4*>(bounds), k);
  return hipGetLastError();
}

__global__ __launch_bounds__(kAdamBlock) void k_adam_fpbo(int64_t U, uint2* __restrict__ state,
                                                          float2* __restrict__ bounds,
                                                          const float* __restrict__ grads,
                                                          float* __restrict__ params_out, AdamConsts k) {
  const int64_t nb = (U + kAdamBlock - 1) / kAdamBlock;
  const int64_t blk = (int64_t)blockIdx.x * (kAdamBlock / kWave) + threadIdx.x / kWave;
  if (blk >= nb) return;  // uniform per wavefront
  if ((blk + 1) * kAdamBlock <= U)
    adam_fpbo_block<true>(U, blk, state, bounds, grads, params_out, k);
  else
    adam_fpbo_block<false>(U, blk, state, bounds, grads, params_out, k);
}

namespace {
AdamConsts adam_consts(const gs_adam_params& p) {
  AdamConsts k;
  k.lr = p.lr;
  k.eps = p.eps;
  k.b1 = (double)p.beta1;
  k.b2 = (double)p.beta2;
  k.c1 = 1.0 - k.b1;
  k.c2 = 1.0 - k.b2;
  k.ib1 = 1.0 / (1.0 - pow(k.b1, (double)p.step));
  k.ib2 = 1.0 / (1.0 - pow(k.b2, (double)p.step));
  return k;
}
unsigned adam_groups(int64_t U) {
  const int64_t nb = (U + kAdamBlock - 1) / kAdamBlock;
  return (unsigned)((nb + kAdamBlock / kWave - 1) / (kAdamBlock / kWave));
}
}  // namespace

hipError_t launch_fpbo_pack(int64_t U, const float* params, uint16_t* state, float* bounds, hipStream_t s) {
  if (U == 0) return hipSuccess;
  k_fpbo_pack<<<adam_groups(U), kAdamBlock, 0, s>>>(U, params, reinterpret_cast<uint2*>(state),
                                                    reinterpret_cast<float2*>(bounds));
  return hipGetLastError();
}

hipError_t launch_adam_fpbo(int64_t U, uint16_t* state, float* bounds, const float* grads, float* params_out,
                            const gs_adam_params& p, hipStream_t s) {
  if (U == 0) return hipSuccess;
  k_adam_fpbo<<<adam_groups(U), kAdamBlock, 0, s>>>(U, reinterpret_cast<uint2*>(state),
                                                    reinterpret_cast<float2*>(bounds), grads, params_out,
                                                    adam_consts(p));
  return hipGetLastError();
}

}  // namespace gs
