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
// 8x8 quadrant (w & 1, w >> 1).  The tile's list is gathered a batch at a time (one record
// per lane, the next batch prefetched into registers) and staged in LDS with a 4-bit mask
// of the quadrants each record's support box touches.  Each wavefront ballots that mask
// and visits only its set bits, reading records back as uniform broadcasts, one record
// ahead of the arithmetic.  A pixel stops once T < 1e-4, a wavefront once its 64 pixels
// have, the tile once all four have.  Tiles run in the order given by tile_order (longest
// lists first) so that the long tiles start early.
//
// The backward walks each wavefront's records in reverse three at a time and sums the
// three records' ten per-pixel gradient terms over the wavefront in one transposed
// reduction; each wavefront adds its sums to the Gaussians' gradients with fp32 atomics.
#include "gs_device.h"
#include "gs_wave.h"

namespace gs {

constexpr int kRenderBlock = 256;
constexpr int kRenderWaves = kRenderBlock / kWave;
constexpr int kBwdBatch = 128;  // records staged per backward batch (bounds LDS use)

// Staged record: (u, v, a2, b2) (c2, opacity, r, g) (b, box x, box y, id) [A, B, C, 0].
// a2, b2, c2 are the conic scaled to the base-2 exponent: -log2(e)/2 * (A, 2B, C).
__device__ __forceinline__ void stage_transform(const float4 r0, const float4 r1, float4& s0, float4& s1) {
  s0 = make_float4(r0.x, r0.y, -0.5f * kLog2e * r0.z, -kLog2e * r0.w);
  s1 = make_float4(-0.5f * kLog2e * r1.x, r1.y, r1.z, r1.w);
}

// Base-2 exponent of the Gaussian factor at offset (dx, dy) from the 2D mean.  Every
// operation is spelled out so that the forward and the backward round identically.
__device__ __forceinline__ float gauss_exponent(float a2, float b2, float c2, float dx, float dy) {
#pragma clang fp contract(off)
  const float inner = fmaf(a2, dx, b2 * dy);  // a2 dx + b2 dy
  const float cy = c2 * dy;
  return fmaf(dx, inner, cy * dy);
}

__device__ __forceinline__ float gauss_factor(float e) { return __builtin_amdgcn_exp2f(e); }

// Which 8x8 quadrants of the tile at pixel (tx0, ty0) does the record's pixel box
// [x0, x1] x [y0, y1] (packed u16 pairs) touch?  Bit q = quadrant (q & 1, q >> 1).
__device__ __forceinline__ uint32_t quadrant_mask(uint32_t bx, uint32_t by, int tx0, int ty0) {
  const int x0 = (int)(bx & 0xFFFFu), x1 = (int)(bx >> 16);
  const int y0 = (int)(by & 0xFFFFu), y1 = (int)(by >> 16);
  const uint32_t cx = (x0 <= tx0 + 7 && x1 >= tx0 ? 1u : 0u) | (x0 <= tx0 + 15 && x1 >= tx0 + 8 ? 2u : 0u);
  const uint32_t cy = (y0 <= ty0 + 7 && y1 >= ty0 ? 1u : 0u) | (y0 <= ty0 + 15 && y1 >= ty0 + 8 ? 2u : 0u);
  return (cy & 1u ? cx : 0u) | (cy & 2u ? cx << 2 : 0u);
}

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

// The quadrants of a tile whose pixel centres the record can reach with alpha >= 1/255:
// the support box test, refined by the exact ellipse-versus-quadrant test with a margin of
// 0.01 in the base-2 exponent (so float32 rounding in the per-pixel evaluation can never
// make a skipped pixel reach the threshold).  s0, s1 are the staged record words.
__device__ __forceinline__ uint32_t reach_mask(const float4 s0, const float4 s1, uint32_t bx, uint32_t by, int tx0,
                                               int ty0) {
  uint32_t m = quadrant_mask(bx, by, tx0, ty0);
  if (!m) return 0u;
  const float thr = __builtin_amdgcn_logf(kAlphaMin) - __builtin_amdgcn_logf(s1.y) - 0.01f;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    if (!((m >> q) & 1u)) continue;
    const float X0 = (float)(tx0 + (q & 1) * 8) + 0.5f - s0.x, Y0 = (float)(ty0 + (q >> 1) * 8) + 0.5f - s0.y;
    if (box_max_exponent(s0.z, s0.w, s1.x, X0, X0 + 7.0f, Y0, Y0 + 7.0f) < thr) m &= ~(1u << q);
  }
  return m;
}

__device__ __forceinline__ int tile_of(const int32_t* __restrict__ order, int b) { return order ? order[b] : b; }

__global__ __launch_bounds__(kRenderBlock) void k_render_fwd(
    const float4* __restrict__ rec, const uint32_t* __restrict__ vals, const int64_t* __restrict__ ranges,
    const int32_t* __restrict__ order, int W, int H, int tiles_x, float bg0, float bg1, float bg2,
    float* __restrict__ image, float* __restrict__ final_T, uint32_t* __restrict__ n_contrib) {
  __shared__ float4 s_rec[kRenderBlock * 3];
  __shared__ uint8_t s_qm[kRenderBlock];  // quadrants each staged record touches
  const int tile = tile_of(order, blockIdx.x);
  const int tx = tile % tiles_x, ty = tile / tiles_x;
  const int t = threadIdx.x, lane = __lane_id(), wave = t / kWave;
  const int qx0 = tx * kTile + (wave & 1) * 8, qy0 = ty * kTile + (wave >> 1) * 8;
  const int px = qx0 + (lane & 7), py = qy0 + (lane >> 3);
  const float fx = (float)px + 0.5f, fy = (float)py + 0.5f;
  const bool inside = px < W && py < H;
  bool live = inside;
  float T = 1.0f, cr = 0.0f, cg = 0.0f, cb = 0.0f;
  uint32_t nc = 0;
  const int64_t start = ranges[2 * tile], end = ranges[2 * tile + 1];

  float4 p0 = make_float4(0.f, 0.f, 0.f, 0.f), p1 = p0, p2 = p0;
  if (start + t < end) {
    const uint32_t id = vals[start + t];
    p0 = rec[3 * (size_t)id]; p1 = rec[3 * (size_t)id + 1]; p2 = rec[3 * (size_t)id + 2];
  }
  for (int64_t b = start; b < end; b += kRenderBlock) {
    if (__syncthreads_count(live) == 0) break;  // also fences the previous batch's reads
    const int cnt = (int)min((int64_t)kRenderBlock, end - b);
    {
      float4 s0, s1;
      stage_transform(p0, p1, s0, s1);
      s_rec[3 * t] = s0; s_rec[3 * t + 1] = s1; s_rec[3 * t + 2] = p2;
      s_qm[t] = t < cnt ? (uint8_t)reach_mask(s0, s1, __float_as_uint(p2.y), __float_as_uint(p2.z), tx * kTile,
                                              ty * kTile)
                        : (uint8_t)0;
    }
    __syncthreads();
    if (b + kRenderBlock + t < end) {  // prefetch the next batch
      const uint32_t id = vals[b + kRenderBlock + t];
      p0 = rec[3 * (size_t)id]; p1 = rec[3 * (size_t)id + 1]; p2 = rec[3 * (size_t)id + 2];
    }
    const uint32_t kb = (uint32_t)(b - start) + 1u;  // list position + 1 of staged record 0
    for (int c = 0; c < cnt; c += kWave) {
      if (!__ballot(live)) break;  // this wavefront's pixels are all done
      // the records of this chunk that touch this wavefront's quadrant, as a scalar mask
      uint64_t m = __ballot((s_qm[c + lane] >> wave) & 1u);
      if (!m) continue;
      int j = c + __builtin_ctzll(m);
      m &= m - 1;
      float4 a = s_rec[3 * j], e1 = s_rec[3 * j + 1];
      float bb = s_rec[3 * j + 2].x;
      while (true) {
        // read the next record while this one is evaluated
        const bool more = m != 0;
        const int jn = more ? c + __builtin_ctzll(m) : j;
        m &= m - 1;
        const float4 an = s_rec[3 * jn], e1n = s_rec[3 * jn + 1];
        const float bbn = s_rec[3 * jn + 2].x;

        const float dx = fx - a.x, dy = fy - a.y;
        const float alpha = fminf(kAlphaMax, e1.y * gauss_factor(gauss_exponent(a.z, a.w, e1.x, dx, dy)));
        const bool take = live && alpha >= kAlphaMin;
        const float w = take ? alpha * T : 0.0f;
        cr = fmaf(e1.z, w, cr);
        cg = fmaf(e1.w, w, cg);
        cb = fmaf(bb, w, cb);
        T = take ? T * (1.0f - alpha) : T;
        nc = take ? kb + (uint32_t)j : nc;
        live = live && !(T < kTMin);
        if (!more) break;
        a = an; e1 = e1n; bb = bbn; j = jn;
      }
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
// the pixel's last contributor, or alpha < 1/255).  Branch-free: a non-contributing lane
// computes with a zero weight and keeps its walk state.  Returns whether it contributed.
//   dL/dalpha = T_k (dL . rgb) - H / (1 - alpha), with T_k = T / (1 - alpha) in front of
//   the record and H the dL-weighted colour behind it; then H += (dL . rgb) alpha T_k.
__device__ __forceinline__ bool bwd_record(const float4* __restrict__ s_rec, int j, uint32_t k, BwdPixel& p,
                                           float* __restrict__ g) {
  const float4 s0 = s_rec[4 * j], s1 = s_rec[4 * j + 1], s2 = s_rec[4 * j + 2], s3 = s_rec[4 * j + 3];
  const float dx = p.fx - s0.x, dy = p.fy - s0.y;
  const float G = gauss_factor(gauss_exponent(s0.z, s0.w, s1.x, dx, dy));
  const float oG = s1.y * G;
  const float alpha = fminf(kAlphaMax, oG);
  const bool contrib = k < p.nc && alpha >= kAlphaMin;
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
  g[5] = dalpha * G;
  const float dq = dalpha * oG;
  g[2] = dq * dx * dx;
  g[3] = dq * dx * dy;
  g[4] = dq * dy * dy;
  g[0] = dq * fmaf(s3.x, dx, s3.y * dy);
  g[1] = dq * fmaf(s3.y, dx, s3.z * dy);
  g[9] = __builtin_amdgcn_sqrtf(fmaf(g[0], g[0], g[1] * g[1]));
  return contrib;
}

__global__ __launch_bounds__(kRenderBlock) void k_render_bwd(
    const float4* __restrict__ rec, const uint32_t* __restrict__ vals, const int64_t* __restrict__ ranges,
    const int32_t* __restrict__ order, int W, int H, int tiles_x, float bg0, float bg1, float bg2,
    const float* __restrict__ final_T, const uint32_t* __restrict__ n_contrib, const float* __restrict__ dL,
    float* __restrict__ gscreen) {
  __shared__ float4 s_rec[kBwdBatch * 4];
  __shared__ uint8_t s_qm[kBwdBatch];
  __shared__ uint32_t s_last[kRenderWaves];
  const int tile = tile_of(order, blockIdx.x);
  const int tx = tile % tiles_x, ty = tile / tiles_x;
  const int t = threadIdx.x, lane = __lane_id(), wave = t / kWave;
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
  const uint32_t wlast = wave_max(p.nc);  // this wavefront walks [0, wlast)
  // the (record, term) whose wavefront sum this lane receives from the transposed reduction
  const int red_r = (lane >> 1) / GS_GRAD_SCREEN, red_e = (lane >> 1) - red_r * GS_GRAD_SCREEN;
  const float red_scale = term_scale(red_e);
  if (lane == 0) s_last[wave] = wlast;
  __syncthreads();
  uint32_t last = 0;
#pragma unroll
  for (int w = 0; w < kRenderWaves; ++w) last = s_last[w] > last ? s_last[w] : last;
  const int64_t start = ranges[2 * tile];
  // batches walk down from the last contributor; each one's records are gathered into
  // registers while the previous batch is processed
  uint32_t pid = 0;
  float4 q0 = make_float4(0.f, 0.f, 0.f, 0.f), q1 = q0, q2 = q0;
  {
    const int64_t hi = start + last, lo = hi - kBwdBatch > start ? hi - kBwdBatch : start;
    if (t < hi - lo) {
      pid = vals[lo + t];
      q0 = rec[3 * (size_t)pid]; q1 = rec[3 * (size_t)pid + 1]; q2 = rec[3 * (size_t)pid + 2];
    }
  }
  for (int64_t hi = start + last; hi > start; hi -= kBwdBatch) {
    const int64_t lo = hi - kBwdBatch > start ? hi - kBwdBatch : start;
    const int cnt = (int)(hi - lo);
    __syncthreads();  // every wavefront is done with the previous batch
    if (t < cnt) {
      const uint32_t id = pid;
      const float4 r0 = q0, r1 = q1, r2 = q2;
      float4 s0, s1;
      stage_transform(r0, r1, s0, s1);
      s_rec[4 * t] = s0;
      s_rec[4 * t + 1] = s1;
      s_rec[4 * t + 2] = make_float4(r2.x, r2.y, r2.z, __uint_as_float(id));
      s_rec[4 * t + 3] = make_float4(r0.z, r0.w, r1.x, 0.0f);
      s_qm[t] = (uint8_t)reach_mask(s0, s1, __float_as_uint(r2.y), __float_as_uint(r2.z), tx * kTile, ty * kTile);
    } else if (t < kBwdBatch) {
      s_qm[t] = 0;
    }
    __syncthreads();
    {  // prefetch the next (earlier) batch
      const int64_t nhi = lo, nlo = nhi - kBwdBatch > start ? nhi - kBwdBatch : start;
      if (t < nhi - nlo) {
        pid = vals[nlo + t];
        q0 = rec[3 * (size_t)pid]; q1 = rec[3 * (size_t)pid + 1]; q2 = rec[3 * (size_t)pid + 2];
      }
    }
    const int jtop = (int)min((int64_t)cnt, (int64_t)wlast - (lo - start));  // records this wave may use
    for (int c = ((jtop - 1) / kWave) * kWave; c >= 0 && jtop > 0; c -= kWave) {
      uint64_t m = __ballot(c + lane < jtop && ((s_qm[c + lane] >> wave) & 1u));
      while (m) {
        // the next three records of the reverse walk (highest position first); the bit
        // positions stay scalar so the walk is a uniform loop
        // a step short of three records repeats the first one at position 2^32 - 1, past
        // every pixel's last contributor, so it adds zeros and leaves the walk unchanged
        int js[3];
        uint32_t ks[3];
#pragma unroll
        for (int r = 0; r < 3; ++r) {
          const bool has = m != 0;
          const int bit = has ? __builtin_amdgcn_readfirstlane(63 - __builtin_clzll(m)) : 0;
          js[r] = has ? c + bit : js[0];
          ks[r] = has ? (uint32_t)(lo - start + c + bit) : 0xFFFFFFFFu;
          if (has) m &= ~(1ull << bit);
        }
        float v[32];
        bool hit[3];
#pragma unroll
        for (int r = 0; r < 3; ++r) hit[r] = bwd_record(s_rec, js[r], ks[r], p, v + GS_GRAD_SCREEN * r);
        v[30] = 0.0f;
        v[31] = 0.0f;
        const uint64_t h0 = __ballot(hit[0]), h1 = __ballot(hit[1]), h2 = __ballot(hit[2]);
        if (h0 | h1 | h2) {
          // lanes 2i and 2i + 1 now hold the wavefront's sum of v[i]; the even lane of each
          // (record, term) pair of a record some pixel took adds it to the Gaussian's gradient
          const float sum = wave_transpose_reduce32(v);
          const uint64_t act = (h0 ? kRedLanes0 : 0ull) | (h1 ? kRedLanes1 : 0ull) | (h2 ? kRedLanes2 : 0ull);
          const int jr = red_r == 0 ? js[0] : red_r == 1 ? js[1] : js[2];
          if ((act >> lane) & 1ull) {
            const uint32_t id = __float_as_uint(s_rec[4 * jr + 2].w);
            atomicAdd(gscreen + (size_t)GS_GRAD_SCREEN * id + red_e, sum * red_scale);
          }
        }
      }
    }
  }
}

hipError_t launch_render_fwd(const gs_projected& proj, const uint32_t* vals, const int64_t* ranges,
                             const int32_t* order, const DevCamera& cam, const float bg[3], float* image,
                             float* final_T, uint32_t* n_contrib, hipStream_t s) {
  const unsigned tiles = (unsigned)(cam.tiles_x * cam.tiles_y);
  k_render_fwd<<<tiles, kRenderBlock, 0, s>>>(reinterpret_cast<const float4*>(proj.rec), vals, ranges, order,
                                             cam.width, cam.height, cam.tiles_x, bg[0], bg[1], bg[2], image, final_T,
                                             n_contrib);
  return hipGetLastError();
}

hipError_t launch_render_bwd(const gs_projected& proj, const uint32_t* vals, const int64_t* ranges,
                             const int32_t* order, const DevCamera& cam, const float bg[3], const float* final_T,
                             const uint32_t* n_contrib, const float* dL, float* gscreen, hipStream_t s) {
  const unsigned tiles = (unsigned)(cam.tiles_x * cam.tiles_y);
  k_render_bwd<<<tiles, kRenderBlock, 0, s>>>(reinterpret_cast<const float4*>(proj.rec), vals, ranges, order,
                                             cam.width, cam.height, cam.tiles_x, bg[0], bg[1], bg[2], final_T,
                                             n_contrib, dL, gscreen);
  return hipGetLastError();
}

}  // namespace gs
