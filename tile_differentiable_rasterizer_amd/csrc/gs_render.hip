// gs_render.hip -- per-tile front-to-back compositing (forward) and its reverse walk
// (backward), for gfx950.
//
// "Implementing Better Gaussian Splatting in Julia" (pwwt.cn) s3.3: each pixel blends the
// Gaussians of its list front to back, adding colour * alpha * T and multiplying T by
// (1 - alpha); s5.4: one thread group per pixel block, serial over the list inside the
// group and parallel across groups, so no two threads write one pixel; s4.3: 16x16 tiles
// bound each pixel's list.  The thresholds (alpha clamp 0.99, skip below 1/255, stop
// below T = 1e-4) are those of the workloads.  "Enabling the absolute-gradient strategy
// in 3D Gaussian Splatting" (jsqmd.com) s2: the backward also sums, per Gaussian, the
// L2 norms of every pixel's 2D-mean gradient (the absolute gradient).
//
// Mapping: one 256-lane workgroup per 16x16 tile, one pixel per lane; wavefront w owns the
// 8x8 quadrant (w & 1, w >> 1) and walks the tile's list on its own, 64 records at a time:
// each lane gathers one record (the next chunk is prefetched into registers), tests it
// against the quadrant (support box, then the exact ellipse bound) and stages it in the
// wavefront's slice of LDS.  The wavefront ballots the test and visits only the set bits,
// reading records back as uniform broadcasts, one record ahead of the arithmetic.  No
// workgroup barrier couples the four quadrants, so a quadrant with a short list does not
// wait for the others.  A pixel stops once T < 1e-4, a wavefront once its 64 pixels have.
// Tiles run in the order given by tile_order (longest lists first) so that the long tiles
// start early.  Ids read from the lists are clamped to n - 1, so lists that do not hold
// valid ids give wrong pixels but never a read outside the records.
//
// The backward walks each wavefront's records [0, last contributor) in reverse three at a
// time and sums the three records' ten per-pixel gradient terms over the wavefront in one
// transposed reduction; each wavefront adds its sums to the Gaussians' gradients with
// fp32 atomics.
#include "gs_device.h"
#include "gs_wave.h"

namespace gs {

constexpr int kRenderBlock = 256;
constexpr int kRenderWaves = kRenderBlock / kWave;

// Staged record: (u, v, a2, b2) (c2, lo, r, g) (b, box x, box y, id) [A, B, C, 1 / opacity].
// a2, b2, c2 are the conic scaled to the base-2 exponent: -log2(e)/2 * (A, 2B, C); lo is
// log2(opacity), so that alpha = 2^(exponent + lo) needs no product with the opacity.
__device__ __forceinline__ void stage_transform(const float4 r0, const float4 r1, float4& s0, float4& s1) {
  s0 = make_float4(r0.x, r0.y, -0.5f * kLog2e * r0.z, -kLog2e * r0.w);
  s1 = make_float4(-0.5f * kLog2e * r1.x, __builtin_amdgcn_logf(r1.y), r1.z, r1.w);
}

// Base-2 exponent of opacity * (Gaussian factor) at offset (dx, dy) from the 2D mean, lo =
// log2(opacity).  Every operation is spelled out so that the forward and the backward
// round identically.
__device__ __forceinline__ float gauss_exponent(float a2, float b2, float c2, float lo, float dx, float dy) {
#pragma clang fp contract(off)
  const float inner = fmaf(a2, dx, b2 * dy);  // a2 dx + b2 dy
  const float cy = c2 * dy;
  return fmaf(dx, inner, fmaf(cy, dy, lo));
}

__device__ __forceinline__ float gauss_factor(float e) { return __builtin_amdgcn_exp2f(e); }

// Largest value over the box [X0, X1] x [Y0, Y1] (offsets from the 2D mean) of the
// negative-definite exponent f = a2 x^2 + b2 x y + c2 y^2: 0 if the box holds the mean,
// else the best of the four edges (on an edge f is a 1D concave quadratic, maximised at
// its vertex clamped to the edge).
__device__ __forceinline__ float box_max_exponent(float a2, float b2, float c2, float X0, float X1, float Y0,
                                                  float Y1) {
  if (X0 <= 0.0f && X1 >= 0.0f && Y0 <= 0.0f && Y1 >= 0.0f) return 0.0f;
  const float ia = __builtin_amdgcn_rcpf(a2), ic = __builtin_amdgcn_rcpf(c2);
  float best = -INFINITY;
#pragma unroll
  for (int e = 0; e < 2; ++e) {
    const float X = e ? X1 : X0, Y = e ? Y1 : Y0;
    const float ys = fminf(fmaxf(-0.5f * b2 * X * ic, Y0), Y1);
    best = fmaxf(best, a2 * X * X + b2 * X * ys + c2 * ys * ys);
    const float xs = fminf(fmaxf(-0.5f * b2 * Y * ia, X0), X1);
    best = fmaxf(best, a2 * xs * xs + b2 * xs * Y + c2 * Y * Y);
  }
  return best;
}

// Can the record reach a pixel centre of the 8x8 quadrant with top-left pixel (qx0, qy0)
// with alpha >= 1/255?  The record's pixel box (packed u16 pairs bx, by) must meet the
// quadrant, and the exact maximum of its exponent over the quadrant must clear the
// threshold with a margin of 0.01 in the base-2 exponent (so float32 rounding in the
// per-pixel evaluation can never make a skipped pixel reach it).  s0, s1 are the staged
// record words.
__device__ __forceinline__ bool quadrant_reach(const float4 s0, const float4 s1, uint32_t bx, uint32_t by, int qx0,
                                               int qy0) {
  const int x0 = (int)(bx & 0xFFFFu), x1 = (int)(bx >> 16);
  const int y0 = (int)(by & 0xFFFFu), y1 = (int)(by >> 16);
  if (!(x0 <= qx0 + 7 && x1 >= qx0 && y0 <= qy0 + 7 && y1 >= qy0)) return false;
  const float thr = __builtin_amdgcn_logf(kAlphaMin) - s1.y - 0.01f;
  const float X0 = (float)qx0 + 0.5f - s0.x, Y0 = (float)qy0 + 0.5f - s0.y;
  return box_max_exponent(s0.z, s0.w, s1.x, X0, X0 + 7.0f, Y0, Y0 + 7.0f) >= thr;
}

__device__ __forceinline__ int tile_of(const int32_t* __restrict__ order, int b) { return order ? order[b] : b; }

__global__ __launch_bounds__(kRenderBlock) void k_render_fwd(
    const float4* __restrict__ rec, const uint32_t* __restrict__ vals, uint32_t id_max,
    const int64_t* __restrict__ ranges,
    const int32_t* __restrict__ order, int W, int H, int tiles_x, float bg0, float bg1, float bg2,
    float* __restrict__ image, float* __restrict__ final_T, uint32_t* __restrict__ n_contrib) {
  // each wavefront's staged chunk: the records that reach its quadrant, compacted, then one
  // inert record, then room for the walk's read-ahead
  constexpr int kSlots = kWave + 3;
  __shared__ float4 s_rec[kRenderWaves][kSlots * 3];
  const int tile = tile_of(order, blockIdx.x);
  const int tx = tile % tiles_x, ty = tile / tiles_x;
  const int lane = __lane_id(), wave = threadIdx.x / kWave;
  const int qx0 = tx * kTile + (wave & 1) * 8, qy0 = ty * kTile + (wave >> 1) * 8;
  const int px = qx0 + (lane & 7), py = qy0 + (lane >> 3);
  const float fx = (float)px + 0.5f, fy = (float)py + 0.5f;
  const bool inside = px < W && py < H;
  float T = 1.0f, cr = 0.0f, cg = 0.0f, cb = 0.0f;
  uint32_t nc = 0;
  const int64_t start = ranges[2 * tile], end = ranges[2 * tile + 1];
  float4* my = s_rec[wave];

  // Each wavefront walks the whole list on its own, 64 records at a time: lane l gathers
  // record c + l (the next chunk is prefetched into registers while this one is
  // composited) and tests it against the wavefront's quadrant; the records that reach it
  // are staged in list order in consecutive slots of the wavefront's LDS slice, each with
  // its list position.  No workgroup barrier: a wavefront never waits for the others.
  float4 p0 = make_float4(0.f, 0.f, 0.f, 0.f), p1 = p0, p2 = p0;
  if (start + lane < end) {
    const uint32_t id = min(vals[start + lane], id_max);
    p0 = rec[3 * (size_t)id]; p1 = rec[3 * (size_t)id + 1]; p2 = rec[3 * (size_t)id + 2];
  }
  // ids run one chunk ahead of the records, so a chunk's record gathers wait on one
  // memory round trip instead of two
  uint32_t nid = start + kWave + lane < end ? vals[start + kWave + lane] : 0u;  // clamped where used
  for (int64_t b = start; b < end; b += kWave) {
    if (!__ballot(inside && T >= kTMin)) break;  // this wavefront's pixels are all done
    float4 s0, s1;
    stage_transform(p0, p1, s0, s1);
    const bool reach =
        b + lane < end && quadrant_reach(s0, s1, __float_as_uint(p2.y), __float_as_uint(p2.z), qx0, qy0);
    const uint64_t m = __ballot(reach);
    const uint32_t cnt = (uint32_t)__popcll(m);
    const uint32_t slot = (uint32_t)__popcll(m & lanemask_lt());
    // the previous chunk's reads are done before these writes, which are done before the
    // reads below (LDS operations of one wavefront stay in order once issued)
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    if (reach) {
      my[3 * slot] = s0;
      my[3 * slot + 1] = s1;
      // colour b, and the list position + 1 of the record (what n_contrib counts)
      my[3 * slot + 2] = make_float4(p2.x, __uint_as_float((uint32_t)(b - start) + 1u + (uint32_t)lane), 0.f, 0.f);
    }
    if (lane == 0) {  // an inert record after the last (opacity 0, lo = -inf: alpha 0, never taken)
      const float4 z = make_float4(0.f, 0.f, 0.f, 0.f);
      my[3 * cnt] = z; my[3 * cnt + 1] = make_float4(0.f, -INFINITY, 0.f, 0.f); my[3 * cnt + 2] = z;
    }
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
    __builtin_amdgcn_wave_barrier();
    if (b + kWave + lane < end) {  // prefetch the next chunk
      const uint32_t id = min(nid, id_max);
      p0 = rec[3 * (size_t)id]; p1 = rec[3 * (size_t)id + 1]; p2 = rec[3 * (size_t)id + 2];
    }
    nid = b + 2 * kWave + lane < end ? vals[b + 2 * kWave + lane] : 0u;
    if (!cnt) continue;
    // one record's contribution: the pixel takes it when it is inside the image, not done
    // (T >= 1e-4) and alpha >= 1/255; a record it does not take gets alpha 0, which leaves
    // T and the colour exactly as they were
    auto blend = [&](const float4 a, const float4 e1, const float2 e2) {
      const float dx = fx - a.x, dy = fy - a.y;
      const float alpha = fminf(kAlphaMax, gauss_factor(gauss_exponent(a.z, a.w, e1.x, e1.y, dx, dy)));
      const bool take = alpha >= kAlphaMin && T >= kTMin && inside;
      const float at = take ? alpha : 0.0f;
      const float w = at * T;
      cr = fmaf(e1.z, w, cr);
      cg = fmaf(e1.w, w, cg);
      cb = fmaf(e2.x, w, cb);
      T = fmaf(-at, T, T);  // T (1 - alpha), rounded once
      nc = take ? __float_as_uint(e2.y) : nc;
    };
    // two records per step (an odd count ends on the inert record); the next step's
    // records are read while this step's are evaluated (the read-ahead past the inert
    // record stays inside the slice and is never used)
    auto third = [](const float4* r) { return *reinterpret_cast<const float2*>(r); };  // (b, position)
    float4 a0 = my[0], b0 = my[1], a1 = my[3], b1 = my[4];
    float2 c0 = third(my + 2), c1 = third(my + 5);
    for (uint32_t i = 0; i < cnt; i += 2) {
      const float4* nx = my + 3 * (i + 2);
      const float4 na0 = nx[0], nb0 = nx[1], na1 = nx[3], nb1 = nx[4];
      const float2 nc0 = third(nx + 2), nc1 = third(nx + 5);
      blend(a0, b0, c0);
      blend(a1, b1, c1);
      a0 = na0; b0 = nb0; c0 = nc0; a1 = na1; b1 = nb1; c1 = nc1;
    }
  }
  if (inside) {
    const size_t plane = (size_t)W * H;
    const size_t o = (size_t)py * W + px;
    image[o] = fmaf(T, bg0, cr);
    image[plane + o] = fmaf(T, bg1, cg);
    image[2 * plane + o] = fmaf(T, bg2, cb);
    final_T[o] = T;
    n_contrib[o] = nc;
  }
}

// Per-lane state of the reverse walk for one pixel.
struct BwdPixel {
  float fx, fy;        // pixel centre
  float T;             // transmittance behind the next record to visit
  float H;             // sum over channels of dL/dpixel * (colour behind it, background included)
  float dr, dg, db;    // dL/dpixel
  uint32_t nc;         // records at positions >= nc did not contribute
  int32_t ncr;         // nc relative to the first position of the chunk being walked
};

// Exact scale of each reduced term to its gradient: terms 2..4 are summed as
// dq' dx^2, dq' dx dy, dq' dy^2 with dq' = dL/dalpha * o G, while dL/dq = -dq' / 2 and
// q = A dx^2 + 2 B dx dy + C dy^2.
__device__ __forceinline__ float term_scale(int e) { return e == 2 || e == 4 ? -0.5f : e == 3 ? -1.0f : 1.0f; }

// Even lanes that receive record r's ten sums (lanes 20 r .. 20 r + 19).
constexpr uint64_t kRedLanes0 = 0x5555555555555555ull & ((1ull << 20) - 1);
constexpr uint64_t kRedLanes1 = kRedLanes0 << 20;
constexpr uint64_t kRedLanes2 = kRedLanes0 << 40;

// One record's ten gradient terms at this lane's pixel, written to g[0..9] (terms 2..4
// before term_scale); zeros where the record did not contribute (a later position than
// the pixel's last contributor, or alpha < 1/255).  kr is the record's position relative
// to the chunk's first (p.ncr is the pixel's count on the same scale).  Branch-free: a non-contributing lane
// computes with a zero weight and keeps its walk state.  Returns the wavefront's lanes that
// contributed (taken from the compare's lane mask where it is formed).
//   dL/dalpha = T_k (dL . rgb) - H / (1 - alpha), with T_k = T / (1 - alpha) in front of
//   the record and H the dL-weighted colour behind it; then H += (dL . rgb) alpha T_k.
__device__ __forceinline__ uint64_t bwd_record(const float4* __restrict__ s_rec, int j, int32_t kr, BwdPixel& p,
                                               float* __restrict__ g, uint32_t& id) {
  const float4 s0 = s_rec[4 * j], s1 = s_rec[4 * j + 1], s2 = s_rec[4 * j + 2], s3 = s_rec[4 * j + 3];
  id = __float_as_uint(s2.w);  // the Gaussian the record belongs to
  const float dx = p.fx - s0.x, dy = p.fy - s0.y;
  const float oG = gauss_factor(gauss_exponent(s0.z, s0.w, s1.x, s1.y, dx, dy));  // opacity * G
  const float alpha = fminf(kAlphaMax, oG);
  const bool contrib = kr < p.ncr && alpha >= kAlphaMin;
  // the same two compares as lane masks (ICmp SLT = 40, FCmp OGE = 3), so the wavefront's
  // contributing lanes come straight from them
  const uint64_t hits = __builtin_amdgcn_sicmp(kr, p.ncr, 40) & __builtin_amdgcn_fcmpf(alpha, kAlphaMin, 3);
  // hardware reciprocal (about 1 ulp): T is recovered from the stored final T by repeated
  // division, whose float32 error stays far below the gradient tolerance
  const float iom = __builtin_amdgcn_rcpf(1.0f - alpha);
  const float Tk = p.T * iom;  // transmittance in front of this Gaussian
  const float w = contrib ? alpha * Tk : 0.0f;
  g[6] = p.dr * w;
  g[7] = p.dg * w;
  g[8] = p.db * w;
  const float D = fmaf(p.db, s2.x, fmaf(p.dg, s1.w, p.dr * s1.z));
  float dalpha = fmaf(Tk, D, -(iom * p.H));
  p.H = fmaf(D, w, p.H);
  p.T = contrib ? Tk : p.T;
  dalpha = contrib && oG <= kAlphaMax ? dalpha : 0.0f;  // the clamp at 0.99 stops the gradient
  const float dq = dalpha * oG;
  g[5] = dq * s3.w;  // dL/dalpha * G, with G = oG / opacity
  const float dqx = dq * dx, dqy = dq * dy;
  g[2] = dqx * dx;
  g[3] = dqx * dy;
  g[4] = dqy * dy;
  g[0] = fmaf(s3.x, dqx, s3.y * dqy);
  g[1] = fmaf(s3.y, dqx, s3.z * dqy);
  g[9] = __builtin_amdgcn_sqrtf(fmaf(g[0], g[0], g[1] * g[1]));
  return hits;
}

__global__ __launch_bounds__(kRenderBlock) void k_render_bwd(
    const float4* __restrict__ rec, const uint32_t* __restrict__ vals, uint32_t id_max,
    const int64_t* __restrict__ ranges,
    const int32_t* __restrict__ order, int W, int H, int tiles_x, float bg0, float bg1, float bg2,
    const float* __restrict__ final_T, const uint32_t* __restrict__ n_contrib, const float* __restrict__ dL,
    float* __restrict__ gscreen) {
  __shared__ float4 s_rec[kRenderWaves][kWave * 4];  // each wavefront's staged chunk
  const int tile = tile_of(order, blockIdx.x);
  const int tx = tile % tiles_x, ty = tile / tiles_x;
  const int lane = __lane_id(), wave = threadIdx.x / kWave;
  const int qx0 = tx * kTile + (wave & 1) * 8, qy0 = ty * kTile + (wave >> 1) * 8;
  const int px = qx0 + (lane & 7), py = qy0 + (lane >> 3);
  const size_t plane = (size_t)W * H;
  BwdPixel p;
  p.fx = (float)px + 0.5f;
  p.fy = (float)py + 0.5f;
  p.T = 1.0f; p.H = 0.0f; p.dr = p.dg = p.db = 0.0f; p.nc = 0;
  if (px < W && py < H) {
    const size_t o = (size_t)py * W + px;
    p.T = final_T[o];
    p.nc = n_contrib[o];
    p.dr = dL[o]; p.dg = dL[plane + o]; p.db = dL[2 * plane + o];
  }
  p.H = fmaf(p.db, bg2, fmaf(p.dg, bg1, p.dr * bg0)) * p.T;
  const int64_t start = ranges[2 * tile], end = ranges[2 * tile + 1];
  // this wavefront walks [0, wlast): up to its last contributor, and never past the tile's
  // list (contributor counts that do not belong to these lists stay inside them)
  const uint32_t wlast = (uint32_t)min((int64_t)wave_max(p.nc), end - start);
  // the (record, term) whose wavefront sum this lane receives from the transposed reduction
  const int red_r = (lane >> 1) / GS_GRAD_SCREEN, red_e = (lane >> 1) - red_r * GS_GRAD_SCREEN;
  const float red_scale = term_scale(red_e);
  float4* my = s_rec[wave];
  // Each wavefront walks its own records [0, wlast) down from the top, 64 at a time:
  // lane l gathers record lo + l (the next, earlier chunk is prefetched into registers
  // while this one is processed), tests it against the wavefront's quadrant and stages it
  // in the wavefront's LDS slice.  No workgroup barrier: a wavefront never waits for the
  // others.
  uint32_t pid = 0;
  float4 q0 = make_float4(0.f, 0.f, 0.f, 0.f), q1 = q0, q2 = q0;
  {
    const int64_t hi = start + wlast, lo = hi - kWave > start ? hi - kWave : start;
    if (lo + lane < hi) {
      pid = min(vals[lo + lane], id_max);
      q0 = rec[3 * (size_t)pid]; q1 = rec[3 * (size_t)pid + 1]; q2 = rec[3 * (size_t)pid + 2];
    }
  }
  for (int64_t hi = start + wlast; hi > start; hi -= kWave) {
    const int64_t lo = hi - kWave > start ? hi - kWave : start;
    bool reach;
    {
      float4 s0, s1;
      stage_transform(q0, q1, s0, s1);
      reach = lo + lane < hi && quadrant_reach(s0, s1, __float_as_uint(q2.y), __float_as_uint(q2.z), qx0, qy0);
      // the previous chunk's reads are done before these writes, which are done before
      // the reads below (LDS operations of one wavefront stay in order once issued)
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      my[4 * lane] = s0;
      my[4 * lane + 1] = s1;
      my[4 * lane + 2] = make_float4(q2.x, q2.y, q2.z, __uint_as_float(pid));
      my[4 * lane + 3] = make_float4(q0.z, q0.w, q1.x, __builtin_amdgcn_rcpf(q1.y));
      __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
      __builtin_amdgcn_wave_barrier();
    }
    uint64_t m = __ballot(reach);
    p.ncr = (int32_t)p.nc - (int32_t)(lo - start);
    {  // prefetch the next (earlier) chunk
      const int64_t nhi = lo, nlo = nhi - kWave > start ? nhi - kWave : start;
      if (nlo + lane < nhi) {
        pid = min(vals[nlo + lane], id_max);
        q0 = rec[3 * (size_t)pid]; q1 = rec[3 * (size_t)pid + 1]; q2 = rec[3 * (size_t)pid + 2];
      }
    }
    while (m) {
      // the next three records of the reverse walk (highest position first); the bit
      // positions stay scalar so the walk is a uniform loop.  A step short of three
      // records repeats the first one at relative position 2^31 - 1, past every pixel's
      // last contributor, so it adds zeros and leaves the walk unchanged.
      int js[3];
      int32_t ks[3];
#pragma unroll
      for (int r = 0; r < 3; ++r) {
        const bool has = m != 0;
        const int bit = has ? __builtin_amdgcn_readfirstlane(63 - __builtin_clzll(m)) : 0;
        js[r] = has ? bit : js[0];
        ks[r] = has ? bit : INT32_MAX;
        if (has) m &= ~(1ull << bit);
      }
      float v[30];
      uint64_t hm[3];
      uint32_t ids[3];
#pragma unroll
      for (int r = 0; r < 3; ++r) hm[r] = bwd_record(my, js[r], ks[r], p, v + GS_GRAD_SCREEN * r, ids[r]);
      const uint64_t h0 = hm[0], h1 = hm[1], h2 = hm[2];
      if (h0 | h1 | h2) {
        // lanes 2i and 2i + 1 now hold the wavefront's sum of v[i]; the even lane of each
        // (record, term) pair of a record some pixel took adds it to the Gaussian's gradient
        const float sum = wave_transpose_reduce30(v);
        const uint64_t act = (h0 ? kRedLanes0 : 0ull) | (h1 ? kRedLanes1 : 0ull) | (h2 ? kRedLanes2 : 0ull);
        const uint32_t id = red_r == 0 ? ids[0] : red_r == 1 ? ids[1] : ids[2];
        if ((act >> lane) & 1ull) atomicAdd(gscreen + (size_t)GS_GRAD_SCREEN * id + red_e, sum * red_scale);
      }
    }
  }
}

hipError_t launch_render_fwd(const gs_projected& proj, const uint32_t* vals, uint32_t id_max, const int64_t* ranges,
                             const int32_t* order, const DevCamera& cam, const float bg[3], float* image,
                             float* final_T, uint32_t* n_contrib, hipStream_t s) {
  const unsigned tiles = (unsigned)(cam.tiles_x * cam.tiles_y);
  k_render_fwd<<<tiles, kRenderBlock, 0, s>>>(reinterpret_cast<const float4*>(proj.rec), vals, id_max, ranges, order,
                                             cam.width, cam.height, cam.tiles_x, bg[0], bg[1], bg[2], image, final_T,
                                             n_contrib);
  return hipGetLastError();
}

hipError_t launch_render_bwd(const gs_projected& proj, const uint32_t* vals, uint32_t id_max, const int64_t* ranges,
                             const int32_t* order, const DevCamera& cam, const float bg[3], const float* final_T,
                             const uint32_t* n_contrib, const float* dL, float* gscreen, hipStream_t s) {
  const unsigned tiles = (unsigned)(cam.tiles_x * cam.tiles_y);
  k_render_bwd<<<tiles, kRenderBlock, 0, s>>>(reinterpret_cast<const float4*>(proj.rec), vals, id_max, ranges, order,
                                             cam.width, cam.height, cam.tiles_x, bg[0], bg[1], bg[2], final_T,
                                             n_contrib, dL, gscreen);
  return hipGetLastError();
}

}  // namespace gs
