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
// 8x8 quadrant (w & 1, w >> 1).  The tile's list is gathered 256 records at a time (one
// per lane, the next batch prefetched into registers) and staged in LDS; every wavefront
// then reads the records back as uniform broadcasts and skips, with a scalar branch, any
// record whose support box misses its quadrant.  A pixel stops once T < 1e-4, a
// wavefront once its 64 pixels have, the tile once all four have.  Tiles run in the order
// given by tile_order (longest lists first) so that the long tiles start early.
#include "gs_device.h"

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
  const float tx = a2 * dx;
  const float ty = c2 * dy;
  const float bxy = b2 * dx;
  return fmaf(tx, dx, fmaf(bxy, dy, ty * dy));
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

// Sum over the 64 lanes of a wavefront; the total lands in lane 63.  DPP row operations
// reduce each row of 16, then row broadcasts fold the four rows.
template <int kCtrl, int kRowMask>
__device__ __forceinline__ float dpp_add(float x) {
  const int t = __builtin_amdgcn_update_dpp(0, __float_as_int(x), kCtrl, kRowMask, 0xF, false);
  return x + __int_as_float(t);
}

__device__ __forceinline__ float wave_reduce_to_last(float v) {
  v = dpp_add<0xB1, 0xF>(v);   // quad_perm [1,0,3,2]
  v = dpp_add<0x4E, 0xF>(v);   // quad_perm [2,3,0,1]
  v = dpp_add<0x141, 0xF>(v);  // row_half_mirror
  v = dpp_add<0x140, 0xF>(v);  // row_mirror
  v = dpp_add<0x142, 0xA>(v);  // row_bcast:15 into rows 1 and 3
  v = dpp_add<0x143, 0xC>(v);  // row_bcast:31 into rows 2 and 3
  return v;
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
      s_qm[t] = t < cnt ? (uint8_t)quadrant_mask(__float_as_uint(p2.y), __float_as_uint(p2.z), tx * kTile,
                                                  ty * kTile)
                        : (uint8_t)0;
    }
    __syncthreads();
    if (b + kRenderBlock + t < end) {  // prefetch the next batch
      const uint32_t id = vals[b + kRenderBlock + t];
      p0 = rec[3 * (size_t)id]; p1 = rec[3 * (size_t)id + 1]; p2 = rec[3 * (size_t)id + 2];
    }
    if (!__ballot(live)) continue;  // this wavefront's pixels are all done
    bool wave_done = false;
    for (int c = 0; c < cnt && !wave_done; c += kWave) {
      // the records of this chunk that touch this wavefront's quadrant, as a scalar mask
      uint64_t m = __ballot((s_qm[c + lane] >> wave) & 1u);
      while (m) {
        const int j = c + __builtin_ctzll(m);
        m &= m - 1;
        const float4 s0 = s_rec[3 * j], s1 = s_rec[3 * j + 1], s2 = s_rec[3 * j + 2];
        bool finished = false;
        if (live) {
          const float dx = fx - s0.x, dy = fy - s0.y;
          const float e = gauss_exponent(s0.z, s0.w, s1.x, dx, dy);
          const float alpha = fminf(kAlphaMax, s1.y * gauss_factor(e));
          if (alpha >= kAlphaMin) {
            const float w = alpha * T;
            cr = fmaf(s1.z, w, cr);
            cg = fmaf(s1.w, w, cg);
            cb = fmaf(s2.x, w, cb);
            T = T * (1.0f - alpha);
            nc = (uint32_t)(b - start + j + 1);
            if (T < kTMin) { live = false; finished = true; }
          }
        }
        if (__ballot(finished) && !__ballot(live)) { wave_done = true; break; }
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

__global__ __launch_bounds__(kRenderBlock) void k_render_bwd(
    const float4* __restrict__ rec, const uint32_t* __restrict__ vals, const int64_t* __restrict__ ranges,
    const int32_t* __restrict__ order, int W, int H, int tiles_x, float bg0, float bg1, float bg2,
    const float* __restrict__ final_T, const uint32_t* __restrict__ n_contrib, const float* __restrict__ dL,
    float* __restrict__ gscreen) {
  __shared__ float4 s_rec[kBwdBatch * 4];
  __shared__ float s_part[kRenderWaves][kBwdBatch][GS_GRAD_SCREEN];
  __shared__ uint8_t s_hit[kRenderWaves][kBwdBatch];
  __shared__ uint8_t s_qm[kBwdBatch];
  __shared__ uint32_t s_last[kRenderWaves];
  const int tile = tile_of(order, blockIdx.x);
  const int tx = tile % tiles_x, ty = tile / tiles_x;
  const int t = threadIdx.x, lane = __lane_id(), wave = t / kWave;
  const int qx0 = tx * kTile + (wave & 1) * 8, qy0 = ty * kTile + (wave >> 1) * 8;
  const int px = qx0 + (lane & 7), py = qy0 + (lane >> 3);
  const float fx = (float)px + 0.5f, fy = (float)py + 0.5f;
  const size_t plane = (size_t)W * H;
  float T = 1.0f, dr = 0.0f, dg = 0.0f, db = 0.0f;
  uint32_t nc = 0;
  if (px < W && py < H) {
    const size_t o = (size_t)py * W + px;
    T = final_T[o];
    nc = n_contrib[o];
    dr = dL[o]; dg = dL[plane + o]; db = dL[2 * plane + o];
  }
  // colour behind the current contributor, starting with the background's share
  float hr = bg0 * T, hg = bg1 * T, hb = bg2 * T;
  const uint32_t wlast = wave_max(nc);  // this wavefront walks [0, wlast)
  if (lane == 0) s_last[wave] = wlast;
  __syncthreads();
  uint32_t last = 0;
#pragma unroll
  for (int w = 0; w < kRenderWaves; ++w) last = s_last[w] > last ? s_last[w] : last;
  const int64_t start = ranges[2 * tile];
  for (int64_t hi = start + last; hi > start; hi -= kBwdBatch) {
    const int64_t lo = hi - kBwdBatch > start ? hi - kBwdBatch : start;
    const int cnt = (int)(hi - lo);
    __syncthreads();  // the previous batch's partial sums have been flushed
    if (t < cnt) {
      const uint32_t id = vals[lo + t];
      const float4 r0 = rec[3 * (size_t)id], r1 = rec[3 * (size_t)id + 1], r2 = rec[3 * (size_t)id + 2];
      float4 s0, s1;
      stage_transform(r0, r1, s0, s1);
      s_rec[4 * t] = s0;
      s_rec[4 * t + 1] = s1;
      s_rec[4 * t + 2] = make_float4(r2.x, r2.y, r2.z, __uint_as_float(id));
      s_rec[4 * t + 3] = make_float4(r0.z, r0.w, r1.x, 0.0f);
      s_qm[t] = (uint8_t)quadrant_mask(__float_as_uint(r2.y), __float_as_uint(r2.z), tx * kTile, ty * kTile);
    } else if (t < kBwdBatch) {
      s_qm[t] = 0;
    }
    if (t < kBwdBatch) {
#pragma unroll
      for (int w = 0; w < kRenderWaves; ++w) s_hit[w][t] = 0;
    }
    __syncthreads();
    const int jtop = (int)min((int64_t)cnt, (int64_t)wlast - (lo - start));  // records this wave may use
    for (int c = ((jtop - 1) / kWave) * kWave; c >= 0 && jtop > 0; c -= kWave) {
     uint64_t m = __ballot(c + lane < jtop && ((s_qm[c + lane] >> wave) & 1u));
     while (m) {  // highest position first: the reverse walk
      const int bit = 63 - __builtin_clzll(m);
      m &= ~(1ull << bit);
      const int j = c + bit;
      const uint32_t k = (uint32_t)(lo - start + j);  // position in the tile's list
      const float4 s0 = s_rec[4 * j], s1 = s_rec[4 * j + 1], s2 = s_rec[4 * j + 2];
      float g0 = 0.f, g1 = 0.f, g2 = 0.f, g3 = 0.f, g4 = 0.f, g5 = 0.f, g6 = 0.f, g7 = 0.f, g8 = 0.f, g9 = 0.f;
      bool hit = false;
      if (k < nc) {
        const float dx = fx - s0.x, dy = fy - s0.y;
        const float e = gauss_exponent(s0.z, s0.w, s1.x, dx, dy);
        const float G = gauss_factor(e);
        const float oG = s1.y * G;
        const float alpha = fminf(kAlphaMax, oG);
        if (alpha >= kAlphaMin) {
          hit = true;
          const float iom = 1.0f / (1.0f - alpha);
          const float Tk = T * iom;  // transmittance in front of this Gaussian
          const float w = alpha * Tk;
          g6 = dr * w;
          g7 = dg * w;
          g8 = db * w;
          const float dalpha = dr * (s1.z * Tk - hr * iom) + dg * (s1.w * Tk - hg * iom) + db * (s2.x * Tk - hb * iom);
          hr = fmaf(s1.z, w, hr);
          hg = fmaf(s1.w, w, hg);
          hb = fmaf(s2.x, w, hb);
          T = Tk;
          if (oG <= kAlphaMax) {  // the clamp at 0.99 stops the gradient
            const float4 s3 = s_rec[4 * j + 3];
            g5 = dalpha * G;
            const float dq = -0.5f * dalpha * oG;  // dL/dq, q = A dx^2 + 2 B dx dy + C dy^2
            g2 = dq * dx * dx;
            g3 = dq * 2.0f * dx * dy;
            g4 = dq * dy * dy;
            g0 = -2.0f * dq * fmaf(s3.x, dx, s3.y * dy);
            g1 = -2.0f * dq * fmaf(s3.y, dx, s3.z * dy);
            g9 = sqrtf(fmaf(g0, g0, g1 * g1));
          }
        }
      }
      if (__ballot(hit)) {
        g0 = wave_reduce_to_last(g0); g1 = wave_reduce_to_last(g1); g2 = wave_reduce_to_last(g2);
        g3 = wave_reduce_to_last(g3); g4 = wave_reduce_to_last(g4); g5 = wave_reduce_to_last(g5);
        g6 = wave_reduce_to_last(g6); g7 = wave_reduce_to_last(g7); g8 = wave_reduce_to_last(g8);
        g9 = wave_reduce_to_last(g9);
        if (lane == kWave - 1) {
          float* p = s_part[wave][j];
          p[0] = g0; p[1] = g1; p[2] = g2; p[3] = g3; p[4] = g4;
          p[5] = g5; p[6] = g6; p[7] = g7; p[8] = g8; p[9] = g9;
          s_hit[wave][j] = 1;
        }
      }
     }
    }
    __syncthreads();
    // one thread per record: combine the four quadrants, then one atomic per value
    if (t < cnt) {
      float acc[GS_GRAD_SCREEN];
#pragma unroll
      for (int e = 0; e < GS_GRAD_SCREEN; ++e) acc[e] = 0.0f;
      bool any = false;
#pragma unroll
      for (int w = 0; w < kRenderWaves; ++w) {
        if (s_hit[w][t]) {
          any = true;
#pragma unroll
          for (int e = 0; e < GS_GRAD_SCREEN; ++e) acc[e] += s_part[w][t][e];
        }
      }
      if (any) {
        const uint32_t id = __float_as_uint(s_rec[4 * t + 2].w);
        float* out = gscreen + (size_t)GS_GRAD_SCREEN * id;
#pragma unroll
        for (int e = 0; e < GS_GRAD_SCREEN; ++e) atomicAdd(out + e, acc[e]);
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
