// gs_project.hip -- projection of 3D Gaussians to screen (forward) and the per-Gaussian
// chain rule back to the 3D parameters (backward), for gfx950.
//
// "Implementing Better Gaussian Splatting in Julia" (pwwt.cn) s3.1: a Gaussian is a
// centre, a scale and a quaternion rotation (the covariance is built from them, so it
// stays positive semi-definite), an opacity and a colour; s3.2: the centre goes to camera
// then pixel coordinates and the 3D covariance is projected through the Jacobian of the
// perspective map.  "Better Gaussian Splatting in Julia" (lshu.cn) s3.1: colour from SH
// coefficients whose count depends on the degree.  The formulas (EWA 2D covariance, real
// SH) are the textbook ones; the pages omit them.
//
// Memory: every input is read once per call.  Degree-3 float32 SH rows (192 B each) reach
// LDS by direct 16-byte global-to-LDS copies, two of every three 128-byte lines, coalesced
// across the wavefront and overlapped with the float64 geometry; each lane loads the
// remaining line of its row pair itself (copy_rows_to_lds, row_from_lds).  Rows of the
// other degrees and quantised rows are read per lane with 16-byte loads, where the cache
// assembles the lines.  The backward writes its dL/dsh
// rows through LDS instead (odd float4 row stride, no bank conflicts) so the stores leave
// as whole lines: per-lane strided stores of them measured far slower.  The
// binning-critical geometry (camera-space mean, 2D covariance, support, pixel box) is
// evaluated in float64 and rounded once; colour is float32.
#include "gs_device.h"
#include "gs_sh.h"
#include "gs_tiles.h"

namespace gs {

constexpr int kProjBlock = 256;
// A wavefront's region of the row table (gs_projected.rows): kWaveRows entries for its
// large rectangles' rows, then one entry whose first word flags a rectangle that did not fit.
constexpr uint32_t kRegionRows = GS_ROWS_PER_BLOCK / (kProjBlock / kWave);
constexpr uint32_t kWaveRows = kRegionRows - 1;

template <int L>
struct ShLayout {
  static constexpr int K = (L + 1) * (L + 1);
  static constexpr int ROW = 3 * K;  // floats per Gaussian
  static constexpr bool V4 = (ROW % 4) == 0;
  // odd stride in the unit the rows are read with (float4 or float): conflict-free
  static constexpr int STRIDE = V4 ? (((ROW / 4) & 1) ? ROW : ROW + 4) : ((ROW & 1) ? ROW : ROW + 1);
};

// Coalesced copy of `cnt` LDS rows back to global memory.
template <int L>
__device__ __forceinline__ void store_sh_rows(float* __restrict__ dst, int cnt, const float* s_sh) {
  using S = ShLayout<L>;
  if constexpr (S::V4) {
    constexpr int R4 = S::ROW / 4;
    float4* d4 = reinterpret_cast<float4*>(dst);
    const int total = cnt * R4;
#pragma unroll
    for (int it = 0; it < R4; ++it) {
      const int f = it * kProjBlock + (int)threadIdx.x;
      if (f < total) {
        const int g = f / R4, c = f - g * R4;
        d4[f] = *reinterpret_cast<const float4*>(s_sh + g * S::STRIDE + 4 * c);
      }
    }
  } else {
    const int total = cnt * S::ROW;
    for (int it = 0; it < S::ROW; ++it) {
      const int f = it * kProjBlock + (int)threadIdx.x;
      if (f < total) {
        const int g = f / S::ROW, c = f - g * S::ROW;
        dst[f] = s_sh[g * S::STRIDE + c];
      }
    }
  }
}

// This lane's row into its LDS row (float4 stores when rows allow them: with the odd
// float4 stride they are conflict-free).
template <int L>
__device__ __forceinline__ void put_row(float* my_row, const float* v) {
  using S = ShLayout<L>;
  if constexpr (S::V4) {
#pragma unroll
    for (int c = 0; c < S::ROW / 4; ++c)
      reinterpret_cast<float4*>(my_row)[c] = make_float4(v[4 * c], v[4 * c + 1], v[4 * c + 2], v[4 * c + 3]);
  } else {
#pragma unroll
    for (int c = 0; c < S::ROW; ++c) my_row[c] = v[c];
  }
}

// This lane's SH row (ROW floats) from global memory into registers.
template <int L>
__device__ __forceinline__ void load_row(const float* __restrict__ row, float* coef) {
  using S = ShLayout<L>;
  if constexpr (S::V4) {
#pragma unroll
    for (int c = 0; c < S::ROW / 4; ++c) {
      const float4 q = reinterpret_cast<const float4*>(row)[c];
      coef[4 * c] = q.x; coef[4 * c + 1] = q.y; coef[4 * c + 2] = q.z; coef[4 * c + 3] = q.w;
    }
  } else {
#pragma unroll
    for (int c = 0; c < S::ROW; ++c) coef[c] = row[c];
  }
}

// Degree-3 float32 SH rows (192 bytes, twelve 16-byte pieces) reach a lane in two parts.  Two
// consecutive rows are three 128-byte lines: the even row's pieces 0-7, then its pieces 8-11
// with the odd row's pieces 0-3, then the odd row's pieces 4-11.  The first and third lines of
// every pair in a wavefront's 64 rows are copied into the wavefront's LDS slice (8 pieces a
// row) by direct global-to-LDS 16-byte loads: consecutive lanes of one copy take consecutive
// pieces, so the reads are coalesced, and the data bypasses the registers while the float64
// geometry runs.  The middle lines are loaded per lane (each lane its own half) when the
// colour is evaluated, so every line is fetched once, and the slice stays at 32 KB per 256
// lanes (four waves per SIMD, as the registers allow).
constexpr int kShPieces = 12;
constexpr int kShLds = 8;

// Issues the copies for the wavefront whose first Gaussian is wbase (n Gaussians in all) into
// dst (kWave * kShLds pieces).  Copy q = k 64 + lane is LDS piece q % kShLds of row r = q /
// kShLds: the row's piece q % kShLds, or q % kShLds + 4 for an odd row.  Every lane copies a
// piece, past the last row the array's last piece again into a slot that no lane reads, so
// the copies are unconditional: with copies that some lanes skip, the compiler's waits for
// later loads would also have to wait for every copy.  (Rows are paired by their index in the
// array; wbase is a multiple of 64.)
__device__ __forceinline__ void copy_rows_to_lds(const float* __restrict__ sh, int64_t n, int64_t wbase,
                                                 float4* dst) {
  const int lane = (int)__lane_id();
  const float4* src = reinterpret_cast<const float4*>(sh) + wbase * kShPieces;
  const int64_t last = (n - wbase) * kShPieces - 1;
#pragma unroll
  for (int k = 0; k < kShLds; ++k) {
    const int q = k * kWave + lane, r = q / kShLds;
    const int64_t p = min((int64_t)(r * kShPieces + (q - r * kShLds) + (r & 1) * (kShPieces - kShLds)), last);
    __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)(src + p),
                                     (__attribute__((address_space(3))) void*)(dst + k * kWave), 16, 0, 0);
  }
}

// Gaussian i's row (48 floats) from its LDS slot (the compiler waits for the copies) and its
// other four pieces from global memory: pieces 8-11 of an even row, 0-3 of an odd one.
__device__ __forceinline__ void row_from_lds(const float4* my_row, const float* __restrict__ sh, int64_t i,
                                             float* coef) {
  constexpr int kT = kShPieces - kShLds;
  const bool odd = (i & 1) != 0;
  float4 tail[kT], lds[kShLds];
#pragma unroll
  for (int t = 0; t < kT; ++t)
    tail[t] = reinterpret_cast<const float4*>(sh)[i * kShPieces + (odd ? 0 : kShLds) + t];
#pragma unroll
  for (int c = 0; c < kShLds; ++c) lds[c] = my_row[c];
#pragma unroll
  for (int c = 0; c < kShPieces; ++c) {
    const float4 e = c < kShLds ? lds[c] : tail[c - kShLds];  // even rows: LDS pieces, then the tail
    const float4 o = c < kT ? tail[c] : lds[c - kT];           // odd rows: the tail, then LDS pieces
    coef[4 * c] = odd ? o.x : e.x; coef[4 * c + 1] = odd ? o.y : e.y;
    coef[4 * c + 2] = odd ? o.z : e.z; coef[4 * c + 3] = odd ? o.w : e.w;
  }
}

// This lane's SH row from q8 / q16 codes (QB bits) with (lo, hi) bounds per 256 units ("Training
// 10M Gaussians in 8 GB: Spirula Studio's VRAM efficiency", quantised training section): unit
// u = i ROW + c lies in block u / 256, so a row spans one or two blocks.  Decoded in float32,
// each operation rounded: lo + code * ((hi - lo) * (1 / qmax)).  Degree 3 rows (48 codes) are
// read with 16-byte loads (96 or 48 bytes, 16-byte aligned).
template <int L, int QB>
__device__ __forceinline__ void load_row_q(const void* __restrict__ codes, const float2* __restrict__ bounds,
                                           int64_t i, float* coef) {
#pragma clang fp contract(off)
  using S = ShLayout<L>;
  using Code = typename std::conditional<QB == 16, uint16_t, uint8_t>::type;
  constexpr float kInvQ = QB == 16 ? 1.0f / 65535.0f : 1.0f / 255.0f;
  const int64_t u0 = i * S::ROW;
  const int64_t b0 = u0 >> 8;
  const int split = (int)(((b0 + 1) << 8) - u0);  // coefficients c < split are in block b0
  const float2 B0 = bounds[b0];
  const float2 B1 = split < S::ROW ? bounds[b0 + 1] : B0;
  const float st0 = (B0.y - B0.x) * kInvQ, st1 = (B1.y - B1.x) * kInvQ;
  uint32_t code[S::ROW];
  const Code* row = static_cast<const Code*>(codes) + u0;
  if constexpr (L == 3) {
    constexpr int kVec = S::ROW * sizeof(Code) / 16;  // 6 (q16) or 3 (q8) 16-byte loads
#pragma unroll
    for (int q = 0; q < kVec; ++q) {
      const uint4 w = reinterpret_cast<const uint4*>(row)[q];
      const uint32_t wv[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        if constexpr (QB == 16) {
          code[8 * q + 2 * k] = wv[k] & 0xFFFFu;
          code[8 * q + 2 * k + 1] = wv[k] >> 16;
        } else {
#pragma unroll
          for (int by = 0; by < 4; ++by) code[16 * q + 4 * k + by] = (wv[k] >> (8 * by)) & 0xFFu;
        }
      }
    }
  } else {
#pragma unroll
    for (int c = 0; c < S::ROW; ++c) code[c] = row[c];
  }
#pragma unroll
  for (int c = 0; c < S::ROW; ++c) {
    const bool first = c < split;
    coef[c] = (first ? B0.x : B1.x) + (float)code[c] * (first ? st0 : st1);
  }
}

// Geometry shared by the forward and the backward, float64.
struct Geom {
  double t[3];      // camera-space mean
  double qn[4];     // unit quaternion
  double qlen;      // |q| of the input
  double Rq[9];     // rotation of qn
  double M[9];      // Rq diag(s)
  double S[6];      // Sigma: xx, xy, xz, yy, yz, zz
};

__device__ __forceinline__ void geom(const DevCamera& cam, double mx, double my, double mz,
                                     const double s[3], const float4 qf, Geom& g) {
  const double* W = cam.R;
  g.t[0] = W[0] * mx + W[1] * my + W[2] * mz + cam.t[0];
  g.t[1] = W[3] * mx + W[4] * my + W[5] * mz + cam.t[1];
  g.t[2] = W[6] * mx + W[7] * my + W[8] * mz + cam.t[2];
  const double qw = qf.x, qx = qf.y, qy = qf.z, qz = qf.w;
  g.qlen = sqrt(qw * qw + qx * qx + qy * qy + qz * qz);
  const double il = 1.0 / g.qlen;
  const double w = qw * il, x = qx * il, y = qy * il, z = qz * il;
  g.qn[0] = w; g.qn[1] = x; g.qn[2] = y; g.qn[3] = z;
  double* R = g.Rq;
  R[0] = 1.0 - 2.0 * (y * y + z * z); R[1] = 2.0 * (x * y - w * z); R[2] = 2.0 * (x * z + w * y);
  R[3] = 2.0 * (x * y + w * z); R[4] = 1.0 - 2.0 * (x * x + z * z); R[5] = 2.0 * (y * z - w * x);
  R[6] = 2.0 * (x * z - w * y); R[7] = 2.0 * (y * z + w * x); R[8] = 1.0 - 2.0 * (x * x + y * y);
#pragma unroll
  for (int r = 0; r < 3; ++r)
#pragma unroll
    for (int c = 0; c < 3; ++c) g.M[3 * r + c] = R[3 * r + c] * s[c];
  const double* M = g.M;
  g.S[0] = M[0] * M[0] + M[1] * M[1] + M[2] * M[2];
  g.S[1] = M[0] * M[3] + M[1] * M[4] + M[2] * M[5];
  g.S[2] = M[0] * M[6] + M[1] * M[7] + M[2] * M[8];
  g.S[3] = M[3] * M[3] + M[4] * M[4] + M[5] * M[5];
  g.S[4] = M[3] * M[6] + M[4] * M[7] + M[5] * M[8];
  g.S[5] = M[6] * M[6] + M[7] * M[7] + M[8] * M[8];
}

__device__ __forceinline__ void sym_mul(const double S[6], const double v[3], double out[3]) {
  out[0] = S[0] * v[0] + S[1] * v[1] + S[2] * v[2];
  out[1] = S[1] * v[0] + S[3] * v[1] + S[4] * v[2];
  out[2] = S[2] * v[0] + S[4] * v[1] + S[5] * v[2];
}

// Rows of T = J W, J the perspective Jacobian at the camera-space mean.
__device__ __forceinline__ void proj_rows(const DevCamera& cam, const double t[3], double t0[3],
                                          double t1[3]) {
  const double iz = 1.0 / t[2];
  const double j00 = cam.fx * iz, j02 = -cam.fx * t[0] * iz * iz;
  const double j11 = cam.fy * iz, j12 = -cam.fy * t[1] * iz * iz;
  const double* W = cam.R;
#pragma unroll
  for (int c = 0; c < 3; ++c) {
    t0[c] = j00 * W[c] + j02 * W[6 + c];
    t1[c] = j11 * W[3 + c] + j12 * W[6 + c];
  }
}

// QB = 0: float32 SH rows in `sh`; QB = 8 / 16: codes in `shq` with bounds `shb`.
template <int L, int QB>
__global__ __launch_bounds__(kProjBlock) void k_project(
    int64_t n, const float* __restrict__ means, const float* __restrict__ scales,
    const float4* __restrict__ quats, const float* __restrict__ opac, const float* __restrict__ sh,
    const void* __restrict__ shq, const float2* __restrict__ shb,
    const DevCamera cam, float4* __restrict__ rec, float* __restrict__ depth_out,
    ushort4* __restrict__ rect_out, uint32_t* __restrict__ ntiles_out, uint8_t* __restrict__ clamp_out,
    uint4* __restrict__ runs_out, uint2* __restrict__ rows_out) {
  using S = ShLayout<L>;
  static_assert(kProjBlock == GS_ROW_BLOCK, "one row-table region per workgroup");
  // degree-3 float32 rows come through LDS (copy_rows_to_lds)
  constexpr bool kDma = L == 3 && QB == 0;
  static_assert(!kDma || S::ROW == 4 * kShPieces, "degree-3 rows");
  __shared__ float4 s_sh[kDma ? kProjBlock * kShLds : 1];
  const int64_t base = (int64_t)blockIdx.x * kProjBlock;
  const int cnt = (int)min((int64_t)kProjBlock, n - base);
  const int tid = threadIdx.x;
  const bool act = tid < cnt;
  const int64_t i = base + (act ? tid : 0);
  // the geometry's inputs are requested before the row copies, so that waiting for them
  // does not wait for the copies (vector memory counters drain in issue order)
  const float mxf = means[3 * i], myf = means[3 * i + 1], mzf = means[3 * i + 2];
  const float s0f = scales[3 * i], s1f = scales[3 * i + 1], s2f = scales[3 * i + 2];
  const float4 qt = quats[i];
  const float opf = opac[i];
  if constexpr (kDma) {
    // the inputs are in registers before the copies are issued: the compiler cannot count
    // direct-to-LDS loads apart from ordinary ones, so a later wait for the inputs would also
    // wait for every copy
    asm volatile("" ::"v"(mxf), "v"(myf), "v"(mzf), "v"(s0f), "v"(s1f), "v"(s2f), "v"(qt.x), "v"(qt.y), "v"(qt.z),
                 "v"(qt.w), "v"(opf));
    const int w = tid / kWave;
    copy_rows_to_lds(sh, n, base + (int64_t)w * kWave, s_sh + w * kWave * kShLds);
    __builtin_amdgcn_sched_barrier(0);
  }
  // lanes past the last Gaussian compute with Gaussian `base` and store nothing (no early
  // return: the input loads stay ahead of the row copies)
  const double mx = mxf, my = myf, mz = mzf;
  const double sc[3] = {s0f, s1f, s2f};
  Geom g;
  geom(cam, mx, my, mz, sc, qt, g);
  if (act) depth_out[i] = (float)g.t[2];

  // view-dependent colour: 0.5 + sum_k Y_k(d) sh_k, clamped at 0.  Evaluated before the
  // screen-space work, except where the row comes through LDS: there it is evaluated last,
  // once the copies have had the geometry's time to land
  float col[3];
  auto colour = [&]() {
    float coef[S::ROW];
    if constexpr (kDma) {
      __builtin_amdgcn_sched_barrier(0);  // the row is read after the geometry, not hoisted into it
      row_from_lds(s_sh + tid * kShLds, sh, i, coef);
    } else if constexpr (QB == 0)
      load_row<L>(sh + i * S::ROW, coef);
    else
      load_row_q<L, QB>(shq, shb, i, coef);
    const double vx = mx - cam.campos[0], vy = my - cam.campos[1], vz = mz - cam.campos[2];
    const double il = 1.0 / sqrt(vx * vx + vy * vy + vz * vz);
    float Y[S::K];
    sh_basis<L>((float)(vx * il), (float)(vy * il), (float)(vz * il), Y);
    uint32_t cl = 0;
#pragma unroll
    for (int ch = 0; ch < 3; ++ch) {
      float acc = 0.5f;
#pragma unroll
      for (int k = 0; k < S::K; ++k) acc = fmaf(Y[k], coef[3 * k + ch], acc);
      if (acc < 0.0f) { cl |= 1u << ch; acc = 0.0f; }
      col[ch] = acc;
    }
    if (act) clamp_out[i] = (uint8_t)cl;
  };
  if constexpr (!kDma) colour();


  float4 r0 = make_float4(0.f, 0.f, 0.f, 0.f), r1 = r0, r2 = r0;
  ushort4 rc = make_ushort4(0, 0, 0, 0);
  uint4 sp = make_uint4(0u, 0u, 0u, 0u);
  uint32_t nt = 0;
  bool overflow = false;  // a visible rectangle whose rows did not fit in the row table
  bool vis = false;
  if (act && g.t[2] > cam.near_z) {  // NaN fails
    double t0[3], t1[3], St0[3], St1[3];
    proj_rows(cam, g.t, t0, t1);
    sym_mul(g.S, t0, St0);
    sym_mul(g.S, t1, St1);
    const double a = t0[0] * St0[0] + t0[1] * St0[1] + t0[2] * St0[2];
    const double b = t0[0] * St1[0] + t0[1] * St1[1] + t0[2] * St1[2];
    const double c = t1[0] * St1[0] + t1[1] * St1[1] + t1[2] * St1[2];
    const double det = a * c - b * b;
    const double o = opf;
    // culled with det <= 1e-9 (a + c)^2 (screen-space axis ratio below ~3e-5, whatever the
    // rotation): a covariance that is a line to working precision, whose det, zero in exact
    // arithmetic for a rank-one covariance, would be rounding noise of either sign
    if (det > 1e-9 * ((a + c) * (a + c)) && o >= (double)kAlphaMin) {
      const double iz = 1.0 / g.t[2];
      const double u = cam.fx * g.t[0] * iz + cam.cx;
      const double v = cam.fy * g.t[1] * iz + cam.cy;
      // support: alpha >= 1/255  <=>  q <= tau; the ellipse's half extents
      const double tau = 2.0 * log(o / (double)kAlphaMin);
      const double ex = sqrt(tau * a), ey = sqrt(tau * c);
      double lx = ceil(u - ex - 0.5), hx = floor(u + ex - 0.5);
      double ly = ceil(v - ey - 0.5), hy = floor(v + ey - 0.5);
      if (lx < 0.0) lx = 0.0;
      if (ly < 0.0) ly = 0.0;
      if (hx > (double)(cam.width - 1)) hx = (double)(cam.width - 1);
      if (hy > (double)(cam.height - 1)) hy = (double)(cam.height - 1);
      if (lx <= hx && ly <= hy) {
        const uint32_t px0 = (uint32_t)lx, px1 = (uint32_t)hx, py0 = (uint32_t)ly, py1 = (uint32_t)hy;
        const double idet = 1.0 / det;
        r0 = make_float4((float)u, (float)v, (float)(c * idet), (float)(-b * idet));
        r1 = make_float4((float)(a * idet), (float)o, 0.0f, 0.0f);  // colour below
        r2 = make_float4(0.0f, __uint_as_float(px0 | (px1 << 16)), __uint_as_float(py0 | (py1 << 16)), 0.0f);
        vis = true;
        rc = make_ushort4((uint16_t)(px0 >> 4), (uint16_t)(px1 >> 4), (uint16_t)(py0 >> 4), (uint16_t)(py1 >> 4));
        // tiles of the rectangle that pass the ellipse test of the record as stored, and
        // their runs packed for the emission
        const TileEllipse te = tile_ellipse(r0.x, r0.y, r0.z, r0.w, r1.x, tau, __float_as_uint(r2.y),
                                            __float_as_uint(r2.z));
        const int tx0 = (int)(px0 >> 4), tx1 = (int)(px1 >> 4), ty0 = (int)(py0 >> 4), ty1 = (int)(py1 >> 4);
        if (spans_fit(tx0, tx1, ty0, ty1)) {
          uint32_t w[4] = {0u, 0u, 0u, 0u};
          for (int ty = ty0; ty <= ty1; ++ty) {
            int lo, hi;
            tile_row_span(te, ty, tx0, tx1, lo, hi);
            const uint32_t cnt = hi >= lo ? (uint32_t)(hi - lo + 1) : 0u;
            nt += cnt;
            const int k = ty - ty0;
            const uint32_t half = (cnt ? (uint32_t)(lo - tx0) : 0u) | (cnt << 8);
            w[k >> 1] |= half << (16 * (k & 1));
          }
          sp = make_uint4(w[0], w[1], w[2], w[3]);
        } else {  // the same test, rows kept in this wavefront's region of the row table when they fit
          // entries in lane order: the rows of the wavefront's lower large rectangles come first
          // (the loop is uniform over the lanes that take this branch)
          const uint32_t R = (uint32_t)(ty1 - ty0 + 1);
          const uint64_t large = __ballot(1);
          uint32_t off = 0;
          for (uint64_t m = large; m; m &= m - 1) {
            const int l = __builtin_ctzll(m);
            const uint32_t r = (uint32_t)__builtin_amdgcn_readlane((int)R, l);
            off += l < (int)__lane_id() ? r : 0u;
          }
          const bool fits = off + R <= kWaveRows;
          const uint32_t first = (uint32_t)blockIdx.x * GS_ROWS_PER_BLOCK + (uint32_t)(tid / kWave) * kRegionRows + off;
          for (int ty = ty0; ty <= ty1; ++ty) {
            int lo, hi;
            tile_row_span(te, ty, tx0, tx1, lo, hi);
            const uint32_t c = hi >= lo ? (uint32_t)(hi - lo + 1) : 0u;
            if (fits) rows_out[first + (uint32_t)(ty - ty0)] = make_uint2((c ? (uint32_t)lo : 0u) | (c << 16), nt);
            nt += c;
          }
          sp = fits ? make_uint4(kTableSpans, first, 0u, 0u) : make_uint4(kNoSpans, kNoSpans, kNoSpans, kNoSpans);
          overflow = !fits && nt > 0;
        }
      }
    }
  }
  if constexpr (kDma) colour();
  if (vis) {
    r1.z = col[0];
    r1.w = col[1];
    r2.x = col[2];
  }
  if (act) {
    rec[3 * i] = r0;
    rec[3 * i + 1] = r1;
    rec[3 * i + 2] = r2;
    rect_out[i] = rc;
    ntiles_out[i] = nt;
    runs_out[2 * i] = sp;
    runs_out[2 * i + 1] = make_uint4((uint32_t)rc.x | ((uint32_t)rc.y << 16),
                                     (uint32_t)rc.z | ((uint32_t)rc.w << 16), nt, 0u);
  }
  // the last entry of the wavefront's region says whether one of its rectangles overflowed,
  // so that the binning skips its float64 path when none did (written by lane 0 of every
  // wavefront that holds a Gaussian)
  const uint64_t ovf = __ballot(overflow);
  if (__lane_id() == 0 && act)
    rows_out[(size_t)(blockIdx.x * (kProjBlock / kWave) + tid / kWave) * kRegionRows + kWaveRows] =
        make_uint2(ovf ? 1u : 0u, 0u);
}

// Backward of the projection for one Gaussian (float64 geometry), plus the densification
// statistics of "Enabling the absolute-gradient strategy in 3D Gaussian Splatting"
// (jsqmd.com) s3.1: accumulate the view-space gradient norm and the absolute gradient,
// and count the views in which the Gaussian was visible.
template <int L>
__global__ __launch_bounds__(kProjBlock) void k_project_bwd(
    int64_t n, const float* __restrict__ means, const float* __restrict__ scales,
    const float4* __restrict__ quats, const float* __restrict__ sh, const DevCamera cam,
    const uint32_t* __restrict__ ntiles, const uint8_t* __restrict__ clampb,
    const float* __restrict__ gscreen, float* __restrict__ dmeans, float* __restrict__ dscales,
    float4* __restrict__ dquats, float* __restrict__ dsh, float2* __restrict__ accum,
    int32_t* __restrict__ denom) {
  using S = ShLayout<L>;
  __shared__ float s_sh[kProjBlock * S::STRIDE];
  const int64_t base = (int64_t)blockIdx.x * kProjBlock;
  const int cnt = (int)min((int64_t)kProjBlock, n - base);
  const int tid = threadIdx.x;
  float* my_row = s_sh + tid * S::STRIDE;
  if (tid < cnt) {
    const int64_t i = base + tid;
    const bool vis = ntiles[i] > 0;
    float gsv[GS_GRAD_SCREEN];
#pragma unroll
    for (int e = 0; e < GS_GRAD_SCREEN; ++e) gsv[e] = gscreen[GS_GRAD_SCREEN * i + e];
    float coef[S::ROW];
    load_row<L>(sh + i * S::ROW, coef);
    float drow[S::ROW];
    double dmu[3] = {0.0, 0.0, 0.0}, ds[3] = {0.0, 0.0, 0.0}, dq[4] = {0.0, 0.0, 0.0, 0.0};
    const double mx = means[3 * i], my = means[3 * i + 1], mz = means[3 * i + 2];
    if (vis) {
      // colour: rgb = max(raw, 0); the clamp stops the gradient
      const uint32_t cl = clampb[i];
      float draw[3];
#pragma unroll
      for (int ch = 0; ch < 3; ++ch) draw[ch] = (cl >> ch) & 1u ? 0.0f : gsv[6 + ch];
      const double vx = mx - cam.campos[0], vy = my - cam.campos[1], vz = mz - cam.campos[2];
      const double dist = sqrt(vx * vx + vy * vy + vz * vz);
      const double il = 1.0 / dist;
      const float dx = (float)(vx * il), dy = (float)(vy * il), dz = (float)(vz * il);
      float Y[S::K];
      float dY[S::K][3];
      sh_basis<L>(dx, dy, dz, Y);
      sh_basis_grad<L>(dx, dy, dz, dY);
      float dd[3] = {0.f, 0.f, 0.f};
#pragma unroll
      for (int k = 0; k < S::K; ++k) {
        float w = 0.f;
#pragma unroll
        for (int ch = 0; ch < 3; ++ch) {
          drow[3 * k + ch] = Y[k] * draw[ch];
          w = fmaf(coef[3 * k + ch], draw[ch], w);
        }
        dd[0] = fmaf(w, dY[k][0], dd[0]);
        dd[1] = fmaf(w, dY[k][1], dd[1]);
        dd[2] = fmaf(w, dY[k][2], dd[2]);
      }
      // d = v/|v|: dd/dmu = (I - d d^T)/|v|
      const double pr = (double)dd[0] * dx + (double)dd[1] * dy + (double)dd[2] * dz;
      dmu[0] = ((double)dd[0] - pr * dx) * il;
      dmu[1] = ((double)dd[1] - pr * dy) * il;
      dmu[2] = ((double)dd[2] - pr * dz) * il;
      put_row<L>(my_row, drow);  // now, so the row is not held in registers below

      const double sc[3] = {scales[3 * i], scales[3 * i + 1], scales[3 * i + 2]};
      Geom g;
      geom(cam, mx, my, mz, sc, quats[i], g);
      double t0[3], t1[3], St0[3], St1[3];
      proj_rows(cam, g.t, t0, t1);
      sym_mul(g.S, t0, St0);
      sym_mul(g.S, t1, St1);
      const double a = t0[0] * St0[0] + t0[1] * St0[1] + t0[2] * St0[2];
      const double b = t0[0] * St1[0] + t0[1] * St1[1] + t0[2] * St1[2];
      const double c = t1[0] * St1[0] + t1[1] * St1[1] + t1[2] * St1[2];
      const double det = a * c - b * b, id2 = 1.0 / (det * det);
      // conic (A, B, C) = (c, -b, a)/det
      const double gA = gsv[2], gB = gsv[3], gC = gsv[4];
      const double da = (-c * c * gA + b * c * gB - b * b * gC) * id2;
      const double db = (2.0 * b * c * gA - (a * c + b * b) * gB + 2.0 * a * b * gC) * id2;
      const double dc = (-b * b * gA + a * b * gB - a * a * gC) * id2;
      // a = t0.S t0, b = t0.S t1, c = t1.S t1
      double dT0[3], dT1[3];
#pragma unroll
      for (int e = 0; e < 3; ++e) {
        dT0[e] = 2.0 * da * St0[e] + db * St1[e];
        dT1[e] = db * St0[e] + 2.0 * dc * St1[e];
      }
      // T = J W  ->  dJ = dT W^T (only the non-zero entries of J matter)
      const double* W = cam.R;
      const double dJ00 = dT0[0] * W[0] + dT0[1] * W[1] + dT0[2] * W[2];
      const double dJ02 = dT0[0] * W[6] + dT0[1] * W[7] + dT0[2] * W[8];
      const double dJ11 = dT1[0] * W[3] + dT1[1] * W[4] + dT1[2] * W[5];
      const double dJ12 = dT1[0] * W[6] + dT1[1] * W[7] + dT1[2] * W[8];
      const double x = g.t[0], y = g.t[1], z = g.t[2], iz = 1.0 / z, iz2 = iz * iz, iz3 = iz2 * iz;
      const double fx = cam.fx, fy = cam.fy;
      const double du = gsv[0], dv = gsv[1];
      double dt[3];
      dt[0] = -fx * iz2 * dJ02 + du * fx * iz;
      dt[1] = -fy * iz2 * dJ12 + dv * fy * iz;
      dt[2] = -fx * iz2 * dJ00 + 2.0 * fx * x * iz3 * dJ02 - fy * iz2 * dJ11 + 2.0 * fy * y * iz3 * dJ12 -
              du * fx * x * iz2 - dv * fy * y * iz2;
#pragma unroll
      for (int e = 0; e < 3; ++e) dmu[e] += W[e] * dt[0] + W[3 + e] * dt[1] + W[6 + e] * dt[2];
      // dSigma (full matrix) = da t0 t0^T + db t0 t1^T + dc t1 t1^T; Sigma = M M^T
      double dSs[9];  // dSigma + dSigma^T
#pragma unroll
      for (int r = 0; r < 3; ++r)
#pragma unroll
        for (int cc = 0; cc < 3; ++cc)
          dSs[3 * r + cc] = 2.0 * da * t0[r] * t0[cc] + db * (t0[r] * t1[cc] + t1[r] * t0[cc]) +
                            2.0 * dc * t1[r] * t1[cc];
      double dR[9];
#pragma unroll
      for (int r = 0; r < 3; ++r)
#pragma unroll
        for (int cc = 0; cc < 3; ++cc) {
          const double dM = dSs[3 * r] * g.M[cc] + dSs[3 * r + 1] * g.M[3 + cc] + dSs[3 * r + 2] * g.M[6 + cc];
          ds[cc] += dM * g.Rq[3 * r + cc];
          dR[3 * r + cc] = dM * sc[cc];
        }
      const double w = g.qn[0], qx = g.qn[1], qy = g.qn[2], qz = g.qn[3];
      double dqn[4];
      dqn[0] = 2.0 * (-qz * dR[1] + qy * dR[2] + qz * dR[3] - qx * dR[5] - qy * dR[6] + qx * dR[7]);
      dqn[1] = 2.0 * (qy * dR[1] + qz * dR[2] + qy * dR[3] - 2.0 * qx * dR[4] - w * dR[5] + qz * dR[6] +
                      w * dR[7] - 2.0 * qx * dR[8]);
      dqn[2] = 2.0 * (-2.0 * qy * dR[0] + qx * dR[1] + w * dR[2] + qx * dR[3] + qz * dR[5] - w * dR[6] +
                      qz * dR[7] - 2.0 * qy * dR[8]);
      dqn[3] = 2.0 * (-2.0 * qz * dR[0] - w * dR[1] + qx * dR[2] + w * dR[3] - 2.0 * qz * dR[4] + qy * dR[5] +
                      qx * dR[6] + qy * dR[7]);
      // qn = q/|q|
      const double pq = dqn[0] * w + dqn[1] * qx + dqn[2] * qy + dqn[3] * qz;
      const double iq = 1.0 / g.qlen;
      dq[0] = (dqn[0] - pq * w) * iq;
      dq[1] = (dqn[1] - pq * qx) * iq;
      dq[2] = (dqn[2] - pq * qy) * iq;
      dq[3] = (dqn[3] - pq * qz) * iq;
      if (accum) {
        float2 acc = accum[i];
        acc.x += (float)sqrt(du * du + dv * dv);
        acc.y += gsv[9];
        accum[i] = acc;
      }
      if (denom) denom[i] += 1;
    } else {
#pragma unroll
      for (int k = 0; k < S::ROW; ++k) drow[k] = 0.0f;
      put_row<L>(my_row, drow);
    }
#pragma unroll
    for (int e = 0; e < 3; ++e) {
      dmeans[3 * i + e] = (float)dmu[e];
      dscales[3 * i + e] = (float)ds[e];
    }
    dquats[i] = make_float4((float)dq[0], (float)dq[1], (float)dq[2], (float)dq[3]);
  }
  __syncthreads();
  store_sh_rows<L>(dsh + base * S::ROW, cnt, s_sh);
}

template <int L, int QB>
static hipError_t launch_project_L(int64_t n, const float* means, const float* scales,
                                   const float* quats, const float* opac, const float* sh, const void* shq,
                                   const float* shb, const DevCamera& cam, const gs_projected& out, hipStream_t s) {
  const unsigned blocks = (unsigned)((n + kProjBlock - 1) / kProjBlock);
  k_project<L, QB><<<blocks, kProjBlock, 0, s>>>(
      n, means, scales, reinterpret_cast<const float4*>(quats), opac, sh, shq, reinterpret_cast<const float2*>(shb),
      cam, reinterpret_cast<float4*>(out.rec), out.depth, reinterpret_cast<ushort4*>(out.rect), out.n_tiles,
      out.clamp, reinterpret_cast<uint4*>(out.runs), reinterpret_cast<uint2*>(out.rows));
  return hipGetLastError();
}

template <int QB>
static hipError_t launch_project_Q(int64_t n, const float* means, const float* scales, const float* quats,
                                   const float* opac, const float* sh, const void* shq, const float* shb, int L,
                                   const DevCamera& cam, const gs_projected& out, hipStream_t s) {
  switch (L) {
    case 0: return launch_project_L<0, QB>(n, means, scales, quats, opac, sh, shq, shb, cam, out, s);
    case 1: return launch_project_L<1, QB>(n, means, scales, quats, opac, sh, shq, shb, cam, out, s);
    case 2: return launch_project_L<2, QB>(n, means, scales, quats, opac, sh, shq, shb, cam, out, s);
    default: return launch_project_L<3, QB>(n, means, scales, quats, opac, sh, shq, shb, cam, out, s);
  }
}

hipError_t launch_project(int64_t n, const float* means, const float* scales, const float* quats,
                          const float* opac, const float* sh, int L, const DevCamera& cam,
                          const gs_projected& out, hipStream_t s) {
  return launch_project_Q<0>(n, means, scales, quats, opac, sh, nullptr, nullptr, L, cam, out, s);
}

// The projection with q8 / q16 SH codes (bits 8 or 16) and their bounds per 256 units.
hipError_t launch_project_qsh(int64_t n, const float* means, const float* scales, const float* quats,
                              const float* opac, const void* shq, const float* shb, int bits, int L,
                              const DevCamera& cam, const gs_projected& out, hipStream_t s) {
  return bits == 16 ? launch_project_Q<16>(n, means, scales, quats, opac, nullptr, shq, shb, L, cam, out, s)
                    : launch_project_Q<8>(n, means, scales, quats, opac, nullptr, shq, shb, L, cam, out, s);
}

template <int L>
static hipError_t launch_project_bwd_L(int64_t n, const float* means, const float* scales,
                                       const float* quats, const float* sh, const DevCamera& cam,
                                       const gs_projected& proj, const gs_grads& gr, float* accum,
                                       int32_t* denom, hipStream_t s) {
  const unsigned blocks = (unsigned)((n + kProjBlock - 1) / kProjBlock);
  k_project_bwd<L><<<blocks, kProjBlock, 0, s>>>(
      n, means, scales, reinterpret_cast<const float4*>(quats), sh, cam, proj.n_tiles, proj.clamp,
      gr.grad_screen, gr.dmeans, gr.dscales, reinterpret_cast<float4*>(gr.dquats), gr.dsh,
      reinterpret_cast<float2*>(accum), denom);
  return hipGetLastError();
}

hipError_t launch_project_bwd(int64_t n, const float* means, const float* scales,
                              const float* quats, const float* sh, int L, const DevCamera& cam,
                              const gs_projected& proj, const gs_grads& gr, float* accum,
                              int32_t* denom, hipStream_t s) {
  switch (L) {
    case 0: return launch_project_bwd_L<0>(n, means, scales, quats, sh, cam, proj, gr, accum, denom, s);
    case 1: return launch_project_bwd_L<1>(n, means, scales, quats, sh, cam, proj, gr, accum, denom, s);
    case 2: return launch_project_bwd_L<2>(n, means, scales, quats, sh, cam, proj, gr, accum, denom, s);
    default: return launch_project_bwd_L<3>(n, means, scales, quats, sh, cam, proj, gr, accum, denom, s);
  }
}

}  // namespace gs

namespace gs {

// Measurement only (gs_measure_project_io): the projection's loads and stores, with the
// same widths, strides and grid, and none of its arithmetic.  Its time bounds what any
// projection with these input and output layouts can take.  The outputs hold no valid
// projection: each value is a sum or a copy of inputs, so that every load is used.
template <int L>
__global__ __launch_bounds__(kProjBlock) void k_project_io(
    int64_t n, const float* __restrict__ means, const float* __restrict__ scales, const float4* __restrict__ quats,
    const float* __restrict__ opac, const float* __restrict__ sh, float4* __restrict__ rec,
    float* __restrict__ depth_out, ushort4* __restrict__ rect_out, uint32_t* __restrict__ ntiles_out,
    uint8_t* __restrict__ clamp_out, uint4* __restrict__ runs_out, uint2* __restrict__ rows_out) {
  using S = ShLayout<L>;
  constexpr bool kDma = L == 3;  // degree-3 rows through LDS, as k_project reads them
  __shared__ float4 s_sh[kDma ? kProjBlock * kShLds : 1];
  const int64_t base = (int64_t)blockIdx.x * kProjBlock;
  const int cnt = (int)min((int64_t)kProjBlock, n - base);
  const int tid = threadIdx.x;
  const bool act = tid < cnt;
  const int64_t i = base + (act ? tid : 0);
  const float mx = means[3 * i], my = means[3 * i + 1], mz = means[3 * i + 2];
  const float sx = scales[3 * i], sy = scales[3 * i + 1], sz = scales[3 * i + 2];
  const float4 q = quats[i];
  const float o = opac[i];
  if constexpr (kDma) {
    asm volatile("" ::"v"(mx), "v"(my), "v"(mz), "v"(sx), "v"(sy), "v"(sz), "v"(q.x), "v"(q.y), "v"(q.z), "v"(q.w),
                 "v"(o));
    const int w = tid / kWave;
    copy_rows_to_lds(sh, n, base + (int64_t)w * kWave, s_sh + w * kWave * kShLds);
  }
  if (!act) return;
  float coef[S::ROW];
  if constexpr (kDma)
    row_from_lds(s_sh + tid * kShLds, sh, i, coef);
  else
    load_row<L>(sh + i * S::ROW, coef);
  float acc = 0.0f;
#pragma unroll
  for (int c = 0; c < S::ROW; ++c) acc += coef[c];
  depth_out[i] = mz;
  clamp_out[i] = (uint8_t)(acc > 0.0f);
  rec[3 * i] = make_float4(mx, my, sx + sy, sz);
  rec[3 * i + 1] = make_float4(q.x + q.y, o, acc, q.z);
  rec[3 * i + 2] = make_float4(q.w, mx + mz, my + mz, 0.0f);
  const uint32_t h = __float_as_uint(acc);
  rect_out[i] = make_ushort4((uint16_t)h, (uint16_t)(h >> 16), (uint16_t)__float_as_uint(o), (uint16_t)__float_as_uint(mz));
  ntiles_out[i] = h & 7u;
  runs_out[2 * i] = make_uint4(h, __float_as_uint(mx), __float_as_uint(my), __float_as_uint(sx));
  runs_out[2 * i + 1] = make_uint4(__float_as_uint(sy), __float_as_uint(sz), h & 7u, 0u);
  if (__lane_id() == 0)  // the wavefront region's overflow entry, as the projection writes it
    rows_out[(size_t)(blockIdx.x * (kProjBlock / kWave) + tid / kWave) * kRegionRows + kWaveRows] = make_uint2(0u, 0u);
}

hipError_t launch_project_io(int64_t n, const float* means, const float* scales, const float* quats,
                             const float* opac, const float* sh, int L, const gs_projected& out, hipStream_t s) {
  const unsigned blocks = (unsigned)((n + kProjBlock - 1) / kProjBlock);
  auto go = [&](auto kernel) {
    kernel<<<blocks, kProjBlock, 0, s>>>(n, means, scales, reinterpret_cast<const float4*>(quats), opac, sh,
                                         reinterpret_cast<float4*>(out.rec), out.depth,
                                         reinterpret_cast<ushort4*>(out.rect), out.n_tiles, out.clamp,
                                         reinterpret_cast<uint4*>(out.runs), reinterpret_cast<uint2*>(out.rows));
    return hipGetLastError();
  };
  switch (L) {
    case 0: return go(k_project_io<0>);
    case 1: return go(k_project_io<1>);
    case 2: return go(k_project_io<2>);
    default: return go(k_project_io<3>);
  }
}

}  // namespace gs
