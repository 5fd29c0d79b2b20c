// gs_tiles.h -- which tiles of a Gaussian's rectangle stay in its list.
// Internal to libgsraster.
//
// "Training 10M Gaussians in 8 GB: Spirula Studio's VRAM efficiency" (mhpq.cn), 16-bit
// AABB section: after the conservative screen box, an ellipse test culls a second time
// and the image is unchanged.  A tile stays when the box spanned by its pixel centres
// (inside the Gaussian's pixel box) meets the support ellipse q <= tau of the record as
// stored (float32 2D mean, conic and opacity), evaluated here in float64.
//
// Per tile row the kept tiles are one run of columns: the part of the ellipse inside the
// row's band of pixel-centre ys is convex, so its x-extent is an interval [xl, xr], and a
// tile stays iff its x-range meets it.  The rightmost x of the ellipse at height y,
// x_r(y) = (-B y + sqrt(tau A - det y^2)) / A (det = AC - B^2), is concave in y with its
// peak at the ellipse's rightmost point y_r = -B e_x / C, so xr = x_r(y_r clamped to the
// band); xl is symmetric.  A band beyond the ellipse's vertical extent keeps nothing.
//
// The projection computes the runs once per Gaussian and stores them in the tile record
// that the emission expands (for rectangles too large for the record, the emission
// computes them again from the render record).  Float contraction is off so that the
// float64 evaluation rounds as written.
#pragma once

#include "gs_device.h"

namespace gs {

struct TileEllipse {
  double u, v, B, det, tauA, iA, yr;  // det = AC - B^2, tauA = tau A, iA = 1 / A
  int px0, px1, py0, py1;             // pixel box
  bool whole;                         // degenerate float32 conic: keep the whole rectangle
};

// tau = 2 ln(opacity / (1/255)), the support level of the record's opacity.
__device__ __forceinline__ TileEllipse tile_ellipse(float u, float v, float A, float B, float C, double tau,
                                                    uint32_t bx, uint32_t by) {
#pragma clang fp contract(off)
  TileEllipse e;
  const double a = A, b = B, c = C;
  e.u = u; e.v = v; e.B = b;
  e.px0 = (int)(bx & 0xFFFFu); e.px1 = (int)(bx >> 16);
  e.py0 = (int)(by & 0xFFFFu); e.py1 = (int)(by >> 16);
  e.det = a * c - b * b;
  e.whole = !(e.det > 0.0 && a > 0.0 && c > 0.0);
  e.tauA = tau * a;
  e.iA = 1.0 / a;
  e.yr = e.whole ? 0.0 : -b * sqrt(tau * c / e.det) / c;
  return e;
}

// Record form of tile_ellipse: the render record as gs_project stores it (u, v, A, B | C,
// opacity, r, g | b, pixel box x, pixel box y, 0), with tau = 2 ln(opacity / (1/255))
// evaluated as the projection evaluates it.
__device__ __forceinline__ TileEllipse tile_ellipse_rec(const float4 r0, const float4 r1, const float4 r2) {
  const double tau = 2.0 * log((double)r1.y / (double)kAlphaMin);
  return tile_ellipse(r0.x, r0.y, r0.z, r0.w, r1.x, tau, __float_as_uint(r2.y), __float_as_uint(r2.z));
}

// Kept columns [lo, hi] of tile row ty inside [tx0, tx1] (hi < lo: none).  The half-width
// of the ellipse at height y is sqrt(tau A - det y^2) / A around its centre line -B y / A.
// A column stays when its pixel-centre x-range meets [xl, xr]: its right edge
// min(16 c + 15, px1) + 0.5 - u is at least xl and its left edge max(16 c, px0) + 0.5 - u at
// most xr.  Both edges are nondecreasing in c, so lo is the first column passing the first
// test and hi the last passing the second; each is found from a guess by the exact tests
// (a step or two), which gives the columns a walk from tx0 and from tx1 would give.
__device__ __forceinline__ void tile_row_span(const TileEllipse& e, int ty, int tx0, int tx1, int& lo, int& hi) {
#pragma clang fp contract(off)
  lo = tx0;
  hi = tx1;
  if (e.whole) return;
  const double Y0 = (double)max(kTile * ty, e.py0) + 0.5 - e.v;
  const double Y1 = (double)min(kTile * ty + kTile - 1, e.py1) + 0.5 - e.v;
  const double yc = fmin(fmax(e.yr, Y0), Y1);
  const double yl = fmin(fmax(-e.yr, Y0), Y1);
  const double Dr = e.tauA - e.det * (yc * yc);
  const double Dl = e.tauA - e.det * (yl * yl);
  if (!(Dr >= 0.0) || !(Dl >= 0.0)) {  // the band misses the ellipse
    hi = tx0 - 1;
    return;
  }
  const double xr = (sqrt(Dr) - e.B * yc) * e.iA;
  const double xl = (-sqrt(Dl) - e.B * yl) * e.iA;
  auto right_edge = [&](int c) { return (double)min(kTile * c + kTile - 1, e.px1) + 0.5 - e.u; };
  auto left_edge = [&](int c) { return (double)max(kTile * c, e.px0) + 0.5 - e.u; };
  lo = (int)fmin(fmax(ceil((xl + e.u - 15.5) * 0.0625), (double)tx0), (double)(tx1 + 1));
  while (lo > tx0 && right_edge(lo - 1) >= xl) --lo;
  while (lo <= tx1 && right_edge(lo) < xl) ++lo;
  hi = (int)fmin(fmax(floor((xr + e.u - 0.5) * 0.0625), (double)(lo - 1)), (double)tx1);
  while (hi < tx1 && left_edge(hi + 1) <= xr) ++hi;
  while (hi >= lo && left_edge(hi) > xr) --hi;
}

// Tile record (32 bytes per Gaussian, written by the projection, expanded by the
// emission): words 0-3 the kept runs of a rectangle of at most kSpanRows tile rows and
// kSpanCols tile columns, two bytes per row (first kept column - tx0, count); then the
// rectangle (tx0 | tx1 << 16, ty0 | ty1 << 16) and the tile count.  A larger rectangle
// stores kTableSpans and the index of its first row in the projection's row table (an
// entry per row: first kept column | count << 16, kept tiles of the earlier rows), or,
// when its block's region of the table is full, kNoSpans: the emission then computes its
// rows from the render record with tile_row_span, the same test, so the same tiles.
constexpr int kSpanRows = 8;
constexpr int kSpanCols = 255;
constexpr uint32_t kNoSpans = 0xFFFFFFFFu;
constexpr uint32_t kTableSpans = 0xFFFFFFFEu;

__device__ __forceinline__ bool spans_fit(int tx0, int tx1, int ty0, int ty1) {
  return ty1 - ty0 + 1 <= kSpanRows && tx1 - tx0 + 1 <= kSpanCols;
}

__device__ __forceinline__ bool spans_packed(const uint4 sp) { return sp.x < kTableSpans; }

// Kept columns [c0, c1] of row k (0-based from ty0) of packed spans.
__device__ __forceinline__ void packed_row(const uint4 sp, int k, int tx0, int& c0, int& c1) {
  const uint32_t word = k < 2 ? sp.x : k < 4 ? sp.y : k < 6 ? sp.z : sp.w;
  const uint32_t half = (word >> (16 * (k & 1))) & 0xFFFFu;
  c0 = tx0 + (int)(half & 0xFFu);
  c1 = c0 + (int)(half >> 8) - 1;
}

}  // namespace gs
