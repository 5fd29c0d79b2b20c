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
// Mapping: one 64-lane wavefront per 16x16 tile; lane (lx, ly) owns the four pixels
// (lx + 8 qx, ly + 8 qy) of the tile's 8x8 quadrants.  Records are gathered 64 at a time
// (one per lane, the next batch prefetched into registers) and staged in LDS, then read
// back as wavefront-uniform broadcasts.  A record whose support box misses a quadrant is
// skipped for that quadrant with a scalar branch; a pixel leaves once T < 1e-4 and the
// tile leaves once all its pixels have.
#include "gs_device.h"

namespace gs {

constexpr int kRenderLanes = kWave;

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

__device__ __forceinline__ bool box_misses(uint32_t bx, uint32_t by, int qx0, int qy0) {
  const int x0 = (int)(bx & 0xFFFFu), x1 = (int)(bx >> 16);
  const int y0 = (int)(by & 0xFFFFu), y1 = (int)(by >> 16);
  return x0 > qx0 + 7 || x1 < qx0 || y0 > qy0 + 7 || y1 < qy0;
}

__global__ __launch_bounds__(kRenderLanes) void k_render_fwd(
    const float4* __restrict__ rec, const uint32_t* __restrict__ vals, const int64_t* __restrict__ ranges,
    int W, int H, int tiles_x, float bg0, float bg1, float bg2, float* __restrict__ image,
    float* __restrict__ final_T, uint32_t* __restrict__ n_contrib) {
  __shared__ float4 s_rec[kRenderLanes * 3];
  const int tile = blockIdx.x;
  const int tx = tile % tiles_x, ty = tile / tiles_x;
  const int lane = threadIdx.x, lx = lane & 7, ly = lane >> 3;
  const int x0 = tx * kTile, y0 = ty * kTile;
  const float fxq[2] = {(float)(x0 + lx) + 0.5f, (float)(x0 + 8 + lx) + 0.5f};
  const float fyq[2] = {(float)(y0 + ly) + 0.5f, (float)(y0 + 8 + ly) + 0.5f};
  float T[4], cr[4], cg[4], cb[4];
  uint32_t nc[4];
  uint32_t live = 0;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    T[q] = 1.0f; cr[q] = cg[q] = cb[q] = 0.0f; nc[q] = 0;
    const int px = x0 + (q & 1) * 8 + lx, py = y0 + (q >> 1) * 8 + ly;
    if (px < W && py < H) live |= 1u << q;
  }
  const int64_t start = ranges[2 * tile], end = ranges[2 * tile + 1];

  float4 p0 = make_float4(0.f, 0.f, 0.f, 0.f), p1 = p0, p2 = p0;
  if (start + lane < end) {
    const uint32_t id = vals[start + lane];
    p0 = rec[3 * (size_t)id]; p1 = rec[3 * (size_t)id + 1]; p2 = rec[3 * (size_t)id + 2];
  }
  uint32_t qact = 0;
#pragma unroll
  for (int q = 0; q < 4; ++q) if (__ballot((live >> q) & 1u)) qact |= 1u << q;

  for (int64_t b = start; b < end && qact; b += kRenderLanes) {
    const int cnt = (int)min((int64_t)kRenderLanes, end - b);
    __syncthreads();
    {
      float4 s0, s1;
      stage_transform(p0, p1, s0, s1);
      s_rec[3 * lane] = s0; s_rec[3 * lane + 1] = s1; s_rec[3 * lane + 2] = p2;
    }
    __syncthreads();
    if (b + kRenderLanes + lane < end) {  // prefetch the next batch
      const uint32_t id = vals[b + kRenderLanes + lane];
      p0 = rec[3 * (size_t)id]; p1 = rec[3 * (size_t)id + 1]; p2 = rec[3 * (size_t)id + 2];
    }
    for (int j = 0; j < cnt; ++j) {
      const float4 s0 = s_rec[3 * j], s1 = s_rec[3 * j + 1], s2 = s_rec[3 * j + 2];
      const uint32_t bx = __builtin_amdgcn_readfirstlane(__float_as_uint(s2.y));
      const uint32_t by = __builtin_amdgcn_readfirstlane(__float_as_uint(s2.z));
      bool finished = false;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        if (!((qact >> q) & 1u)) continue;
        if (box_misses(bx, by, x0 + (q & 1) * 8, y0 + (q >> 1) * 8)) continue;
        if ((live >> q) & 1u) {
          const float dx = fxq[q & 1] - s0.x, dy = fyq[q >> 1] - s0.y;
          const float e = gauss_exponent(s0.z, s0.w, s1.x, dx, dy);
          const float alpha = fminf(kAlphaMax, s1.y * gauss_factor(e));
          if (alpha >= kAlphaMin) {
            const float w = alpha * T[q];
            cr[q] = fmaf(s1.z, w, cr[q]);
            cg[q] = fmaf(s1.w, w, cg[q]);
            cb[q] = fmaf(s2.x, w, cb[q]);
            T[q] = T[q] * (1.0f - alpha);
            nc[q] = (uint32_t)(b - start + j + 1);
            if (T[q] < kTMin) { live &= ~(1u << q); finished = true; }
          }
        }
      }
      if (__ballot(finished)) {
        qact = 0;
#pragma unroll
        for (int q = 0; q < 4; ++q) if (__ballot((live >> q) & 1u)) qact |= 1u << q;
        if (!qact) break;
      }
    }
  }
  const size_t plane = (size_t)W * H;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int px = x0 + (q & 1) * 8 + lx, py = y0 + (q >> 1) * 8 + ly;
    if (px < W && py < H) {
      const size_t o = (size_t)py * W + px;
      image[o] = fmaf(T[q], bg0, cr[q]);
      image[plane + o] = fmaf(T[q], bg1, cg[q]);
      image[2 * plane + o] = fmaf(T[q], bg2, cb[q]);
      final_T[o] = T[q];
      n_contrib[o] = nc[q];
    }
  }
}

__global__ __launch_bounds__(kRenderLanes) void k_render_bwd(
    const float4* __restrict__ rec, const uint32_t* __restrict__ vals, const int64_t* __restrict__ ranges,
    int W, int H, int tiles_x, float bg0, float bg1, float bg2, const float* __restrict__ final_T,
    const uint32_t* __restrict__ n_contrib, const float* __restrict__ dL, float* __restrict__ gscreen) {
  __shared__ float4 s_rec[kRenderLanes * 4];
  const int tile = blockIdx.x;
  const int tx = tile % tiles_x, ty = tile / tiles_x;
  const int lane = threadIdx.x, lx = lane & 7, ly = lane >> 3;
  const int x0 = tx * kTile, y0 = ty * kTile;
  const float fxq[2] = {(float)(x0 + lx) + 0.5f, (float)(x0 + 8 + lx) + 0.5f};
  const float fyq[2] = {(float)(y0 + ly) + 0.5f, (float)(y0 + 8 + ly) + 0.5f};
  const size_t plane = (size_t)W * H;
  float T[4], dr[4], dg[4], db[4], hr[4], hg[4], hb[4];
  uint32_t nc[4];
  uint32_t last = 0;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int px = x0 + (q & 1) * 8 + lx, py = y0 + (q >> 1) * 8 + ly;
    T[q] = 1.0f; dr[q] = dg[q] = db[q] = 0.0f; nc[q] = 0;
    if (px < W && py < H) {
      const size_t o = (size_t)py * W + px;
      T[q] = final_T[o];
      nc[q] = n_contrib[o];
      dr[q] = dL[o]; dg[q] = dL[plane + o]; db[q] = dL[2 * plane + o];
    }
    // colour behind the current contributor, starting with the background's share
    hr[q] = bg0 * T[q]; hg[q] = bg1 * T[q]; hb[q] = bg2 * T[q];
    last = nc[q] > last ? nc[q] : last;
  }
  last = wave_max(last);
  const int64_t start = ranges[2 * tile];
  for (int64_t hi = start + last; hi > start; hi -= kRenderLanes) {
    const int64_t lo = hi - kRenderLanes > start ? hi - kRenderLanes : start;
    const int cnt = (int)(hi - lo);
    __syncthreads();
    if (lane < cnt) {
      const uint32_t id = vals[lo + lane];
      const float4 r0 = rec[3 * (size_t)id], r1 = rec[3 * (size_t)id + 1], r2 = rec[3 * (size_t)id + 2];
      float4 s0, s1;
      stage_transform(r0, r1, s0, s1);
      s_rec[4 * lane] = s0;
      s_rec[4 * lane + 1] = s1;
      s_rec[4 * lane + 2] = make_float4(r2.x, r2.y, r2.z, __uint_as_float(id));
      s_rec[4 * lane + 3] = make_float4(r0.z, r0.w, r1.x, 0.0f);
    }
    __syncthreads();
    for (int j = cnt - 1; j >= 0; --j) {
      const uint32_t k = (uint32_t)(lo - start + j);  // position in the tile's list
      const float4 s0 = s_rec[4 * j], s1 = s_rec[4 * j + 1], s2 = s_rec[4 * j + 2], s3 = s_rec[4 * j + 3];
      const uint32_t bx = __builtin_amdgcn_readfirstlane(__float_as_uint(s2.y));
      const uint32_t by = __builtin_amdgcn_readfirstlane(__float_as_uint(s2.z));
      float g[GS_GRAD_SCREEN];
#pragma unroll
      for (int e = 0; e < GS_GRAD_SCREEN; ++e) g[e] = 0.0f;
      bool hit = false;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        if (box_misses(bx, by, x0 + (q & 1) * 8, y0 + (q >> 1) * 8)) continue;
        if (k < nc[q]) {
          const float dx = fxq[q & 1] - s0.x, dy = fyq[q >> 1] - s0.y;
          const float e = gauss_exponent(s0.z, s0.w, s1.x, dx, dy);
          const float G = gauss_factor(e);
          const float oG = s1.y * G;
          const float alpha = fminf(kAlphaMax, oG);
          if (alpha >= kAlphaMin) {
            hit = true;
            const float om = 1.0f - alpha;
            const float iom = 1.0f / om;
            const float Tk = T[q] * iom;  // transmittance in front of this Gaussian
            const float w = alpha * Tk;
            g[6] = fmaf(dr[q], w, g[6]);
            g[7] = fmaf(dg[q], w, g[7]);
            g[8] = fmaf(db[q], w, g[8]);
            const float dalpha = dr[q] * (s1.z * Tk - hr[q] * iom) + dg[q] * (s1.w * Tk - hg[q] * iom) +
                                 db[q] * (s2.x * Tk - hb[q] * iom);
            hr[q] = fmaf(s1.z, w, hr[q]);
            hg[q] = fmaf(s1.w, w, hg[q]);
            hb[q] = fmaf(s2.x, w, hb[q]);
            T[q] = Tk;
            if (oG <= kAlphaMax) {  // the clamp at 0.99 stops the gradient
              g[5] = fmaf(dalpha, G, g[5]);
              const float dq = -0.5f * dalpha * oG;  // dL/dq, q = A dx^2 + 2 B dx dy + C dy^2
              g[2] = fmaf(dq, dx * dx, g[2]);
              g[3] = fmaf(dq, 2.0f * dx * dy, g[3]);
              g[4] = fmaf(dq, dy * dy, g[4]);
              const float gu = -2.0f * dq * fmaf(s3.x, dx, s3.y * dy);
              const float gv = -2.0f * dq * fmaf(s3.y, dx, s3.z * dy);
              g[0] += gu;
              g[1] += gv;
              g[9] += sqrtf(fmaf(gu, gu, gv * gv));
            }
          }
        }
      }
      if (__ballot(hit)) {
        const uint32_t id = __float_as_uint(s2.w);
        float* out = gscreen + (size_t)GS_GRAD_SCREEN * id;
#pragma unroll
        for (int e = 0; e < GS_GRAD_SCREEN; ++e) {
          const float sum = wave_sum(g[e]);
          if (lane == 0) atomicAdd(out + e, sum);
        }
      }
    }
  }
}

hipError_t launch_render_fwd(const gs_projected& proj, const uint32_t* vals, const int64_t* ranges,
                             const DevCamera& cam, const float bg[3], float* image, float* final_T,
                             uint32_t* n_contrib, hipStream_t s) {
  const unsigned tiles = (unsigned)(cam.tiles_x * cam.tiles_y);
  k_render_fwd<<<tiles, kRenderLanes, 0, s>>>(reinterpret_cast<const float4*>(proj.rec), vals, ranges, cam.width,
                                             cam.height, cam.tiles_x, bg[0], bg[1], bg[2], image, final_T,
                                             n_contrib);
  return hipGetLastError();
}

hipError_t launch_render_bwd(const gs_projected& proj, const uint32_t* vals, const int64_t* ranges,
                             const DevCamera& cam, const float bg[3], const float* final_T,
                             const uint32_t* n_contrib, const float* dL, float* gscreen, hipStream_t s) {
  const unsigned tiles = (unsigned)(cam.tiles_x * cam.tiles_y);
  k_render_bwd<<<tiles, kRenderLanes, 0, s>>>(reinterpret_cast<const float4*>(proj.rec), vals, ranges, cam.width,
                                             cam.height, cam.tiles_x, bg[0], bg[1], bg[2], final_T, n_contrib, dL,
                                             gscreen);
  return hipGetLastError();
}

}  // namespace gs
