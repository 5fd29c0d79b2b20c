/*
 * gs_oracle.c -- plain float64 CPU oracle for tile-based 3D Gaussian splatting.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the slow, obviously-correct reference that
 * the HIP path is checked against.  Only the tests, the smoke entry and the CPU-baseline
 * leg of the benchmark load it.  It shares no code, header, table or constant with the
 * HIP library; both are written independently from the same pages.
 *
 * Sources (the pages' titles; sections as the pages number them):
 *  [JULIA-1]  "Implementing Better Gaussian Splatting in Julia: principles, optimisation
 *             and practice" (pwwt.cn) -- s1.1 the pipeline, s3.1 the Gaussian record,
 *             s3.2 projection, s3.3 compositing, s4.3 tiles and influence radius.
 *  [JULIA-2]  "Better Gaussian Splatting in Julia" (lshu.cn) -- s3.1 parameter table
 *             (SH coefficients per degree), s3.2 the rasterize pipeline.
 *  [ABSGRAD]  "Enabling the absolute-gradient strategy in 3D Gaussian Splatting"
 *             (jsqmd.com) -- s1 densification statistics, s2 the two gradient norms.
 *  [SPIRULA]  "Training 10M Gaussians in 8 GB: Spirula Studio's VRAM efficiency"
 *             (mhpq.cn) -- the 16-bit AABB section: a conservative screen box followed by
 *             an ellipse test as a second cull leaves the rendered image unchanged.
 *
 * The pages omit the covariance and SH formulas ([JULIA-1] s3.2 points at "the original
 * paper's Jacobian approximation").  The readings used here are the textbook ones:
 * EWA splatting (Zwicker et al. 2002) for the 2D covariance, the real spherical harmonics
 * with the Condon-Shortley phase for colour, and the Hamilton unit-quaternion rotation.
 *
 * Everything is float64.  Thresholds are the exact float32 constants of the configs
 * lifted to float64, so both implementations test against the same numbers.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* Threads the OpenMP loops use (1 without OpenMP). */
int orc_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/* Thread count of the OpenMP loops from now on (timing the oracle single-threaded). */
void orc_set_threads(int n) {
#ifdef _OPENMP
  if (n > 0) omp_set_num_threads(n);
#else
  (void)n;
#endif
}

#define ORC_AMAX ((double)0.99f)              /* alpha clamp                         */
#define ORC_AMIN ((double)(float)(1.0 / 255.0)) /* skip contributions below this alpha */
#define ORC_TMIN ((double)1e-4f)              /* stop a pixel below this transmittance */
#define ORC_TILE 16                          /* 16x16 tiles, [JULIA-1] s4.3           */
#define ORC_EPS32 (1.0 / 16777216.0)          /* 2^-24: unit roundoff of float32        */

typedef struct {
  double R[9];   /* world -> camera rotation, row major: x_cam = R x_world + t */
  double t[3];
  double fx, fy, cx, cy;
  double near_z;
  int64_t width, height;
} orc_camera;

/* ------------------------------------------------------------------------------------ */
/* Real spherical harmonics, degree <= 3, Condon-Shortley phase, index l*l + l + m.       */
/* Written as polynomials of the unit direction (x, y, z).                               */
/* ------------------------------------------------------------------------------------ */
static void sh_constants(double c[16]) {
  const double pi = M_PI;
  c[0] = 0.5 * sqrt(1.0 / pi);
  c[1] = sqrt(3.0 / (4.0 * pi));
  c[2] = 0.5 * sqrt(15.0 / pi);
  c[3] = 0.25 * sqrt(5.0 / pi);
  c[4] = 0.25 * sqrt(15.0 / pi);
  c[5] = 0.25 * sqrt(35.0 / (2.0 * pi));
  c[6] = 0.5 * sqrt(105.0 / pi);
  c[7] = 0.25 * sqrt(21.0 / (2.0 * pi));
  c[8] = 0.25 * sqrt(7.0 / pi);
  c[9] = 0.25 * sqrt(105.0 / pi);
}

/* Y[k] for k < (L+1)^2; dY[k][3] = gradient of the polynomial w.r.t. (x, y, z) if dY. */
void orc_sh_basis(int L, const double d[3], double* Y, double* dY) {
  double c[16];
  sh_constants(c);
  const double x = d[0], y = d[1], z = d[2];
  double g[16][3];
  memset(g, 0, sizeof g);
  double v[16];
  v[0] = c[0];
  if (L >= 1) {
    v[1] = -c[1] * y;  g[1][1] = -c[1];
    v[2] = c[1] * z;   g[2][2] = c[1];
    v[3] = -c[1] * x;  g[3][0] = -c[1];
  }
  if (L >= 2) {
    v[4] = c[2] * x * y;            g[4][0] = c[2] * y;  g[4][1] = c[2] * x;
    v[5] = -c[2] * y * z;           g[5][1] = -c[2] * z; g[5][2] = -c[2] * y;
    v[6] = c[3] * (3 * z * z - 1);  g[6][2] = c[3] * 6 * z;
    v[7] = -c[2] * x * z;           g[7][0] = -c[2] * z; g[7][2] = -c[2] * x;
    v[8] = c[4] * (x * x - y * y);  g[8][0] = c[4] * 2 * x; g[8][1] = -c[4] * 2 * y;
  }
  if (L >= 3) {
    v[9] = -c[5] * y * (3 * x * x - y * y);
    g[9][0] = -c[5] * 6 * x * y;
    g[9][1] = -c[5] * (3 * x * x - 3 * y * y);
    v[10] = c[6] * x * y * z;
    g[10][0] = c[6] * y * z; g[10][1] = c[6] * x * z; g[10][2] = c[6] * x * y;
    v[11] = -c[7] * y * (5 * z * z - 1);
    g[11][1] = -c[7] * (5 * z * z - 1); g[11][2] = -c[7] * 10 * y * z;
    v[12] = c[8] * z * (5 * z * z - 3);
    g[12][2] = c[8] * (15 * z * z - 3);
    v[13] = -c[7] * x * (5 * z * z - 1);
    g[13][0] = -c[7] * (5 * z * z - 1); g[13][2] = -c[7] * 10 * x * z;
    v[14] = c[9] * z * (x * x - y * y);
    g[14][0] = c[9] * 2 * x * z; g[14][1] = -c[9] * 2 * y * z; g[14][2] = c[9] * (x * x - y * y);
    v[15] = -c[5] * x * (x * x - 3 * y * y);
    g[15][0] = -c[5] * (3 * x * x - 3 * y * y); g[15][1] = c[5] * 6 * x * y;
  }
  const int K = (L + 1) * (L + 1);
  for (int k = 0; k < K; ++k) {
    Y[k] = v[k];
    if (dY) { dY[3 * k] = g[k][0]; dY[3 * k + 1] = g[k][1]; dY[3 * k + 2] = g[k][2]; }
  }
}

/* Hamilton rotation matrix of the unit quaternion (w, x, y, z), row major. */
static void quat_to_rot(const double q[4], double R[9]) {
  const double w = q[0], x = q[1], y = q[2], z = q[3];
  R[0] = 1 - 2 * (y * y + z * z); R[1] = 2 * (x * y - w * z);     R[2] = 2 * (x * z + w * y);
  R[3] = 2 * (x * y + w * z);     R[4] = 1 - 2 * (x * x + z * z); R[5] = 2 * (y * z - w * x);
  R[6] = 2 * (x * z - w * y);     R[7] = 2 * (y * z + w * x);     R[8] = 1 - 2 * (x * x + y * y);
}

/* dR/dq_c for c = w, x, y, z at the unit quaternion q (each a 3x3 row-major block). */
static void quat_rot_jac(const double q[4], double dR[4][9]) {
  const double w = q[0], x = q[1], y = q[2], z = q[3];
  /* d/dw */
  double Dw[9] = {0, -2 * z, 2 * y, 2 * z, 0, -2 * x, -2 * y, 2 * x, 0};
  /* d/dx */
  double Dx[9] = {0, 2 * y, 2 * z, 2 * y, -4 * x, -2 * w, 2 * z, 2 * w, -4 * x};
  /* d/dy */
  double Dy[9] = {-4 * y, 2 * x, 2 * w, 2 * x, 0, 2 * z, -2 * w, 2 * z, -4 * y};
  /* d/dz */
  double Dz[9] = {-4 * z, -2 * w, 2 * x, 2 * w, -4 * z, 2 * y, 2 * x, 2 * y, 0};
  memcpy(dR[0], Dw, sizeof Dw);
  memcpy(dR[1], Dx, sizeof Dx);
  memcpy(dR[2], Dy, sizeof Dy);
  memcpy(dR[3], Dz, sizeof Dz);
}

/* 3D covariance (R(q/|q|) diag(s))(R diag(s))^T, row major (for the invariants tests). */
void orc_cov3d(const double s[3], const double q[4], double Sig[9]) {
  double qn[4], R[9], M[9];
  const double len = sqrt(q[0] * q[0] + q[1] * q[1] + q[2] * q[2] + q[3] * q[3]);
  for (int i = 0; i < 4; ++i) qn[i] = q[i] / len;
  quat_to_rot(qn, R);
  for (int i = 0; i < 3; ++i)
    for (int j = 0; j < 3; ++j) M[3 * i + j] = R[3 * i + j] * s[j];
  for (int i = 0; i < 3; ++i)
    for (int j = 0; j < 3; ++j) {
      double acc = 0;
      for (int k = 0; k < 3; ++k) acc += M[3 * i + k] * M[3 * j + k];
      Sig[3 * i + j] = acc;
    }
}

/* Round to the nearest float32 and return its bit pattern. */
static uint32_t f32_bits(double x) {
  float f = (float)x;
  uint32_t u;
  memcpy(&u, &f, 4);
  return u;
}

/* Everything the forward computes for one Gaussian; the backward reuses it. */
typedef struct {
  int visible;
  double tc[3];          /* camera-space mean                                   */
  double u, v;           /* 2D mean in pixels                                   */
  uint32_t depth_bits;   /* bits of RN_f32(z)                                   */
  double qn[4], qlen;    /* unit quaternion and the input's norm                */
  double Rq[9], M[9];    /* rotation, M = Rq diag(s)                            */
  double Sig[9];         /* 3D covariance                                       */
  double J[6];           /* 2x3 projection Jacobian at tc                       */
  double T[6];           /* J * W                                               */
  double a, b, c, det;   /* 2D covariance [[a, b], [b, c]]                      */
  double A, B, C;        /* conic = inverse 2D covariance                       */
  double tau, ex, ey;    /* support level and half extents                      */
  int64_t px0, px1, py0, py1; /* pixel-centre bounding box, clamped            */
  int64_t tx0, tx1, ty0, ty1; /* tile rectangle                                 */
  int64_t n_tiles;
  double dir[3], dist;   /* unit view direction and camera distance             */
  double raw[3], rgb[3];
  int clamp[3];
  int flags;             /* bit0 depth rounding tie, bit1 rect edge, bit2 colour sign,
                            bit3 a tile-ellipse decision near its threshold,
                            bit4 the line cull near its threshold                   */
} orc_gauss;

/* Is x within tol of an integer? */
static int near_integer(double x, double tol) {
  double r = x - floor(x + 0.5);
  return fabs(r) <= tol;
}

/*
 * Smallest value of the positive-definite form q = A x^2 + 2 B x y + C y^2 over the box
 * [X0, X1] x [Y0, Y1]: 0 when the box holds the origin; otherwise it lies on the boundary,
 * and on each edge q is a convex quadratic in one variable, smallest at its vertex clamped
 * to the edge.  (xm, ym) receive the minimising point.
 */
static double clampd(double x, double lo, double hi) { return x < lo ? lo : x > hi ? hi : x; }

double orc_box_min_q(double A, double B, double C, double X0, double X1, double Y0, double Y1,
                     double* xm, double* ym) {
  if (X0 <= 0 && 0 <= X1 && Y0 <= 0 && 0 <= Y1) {
    if (xm) { *xm = 0; *ym = 0; }
    return 0.0;
  }
  double best = INFINITY, bx = 0, by = 0;
  for (int e = 0; e < 2; ++e) {
    const double X = e ? X1 : X0;             /* edge x = X */
    const double y = clampd(-B * X / C, Y0, Y1);
    const double qx = A * X * X + 2 * B * X * y + C * y * y;
    if (qx < best) { best = qx; bx = X; by = y; }
    const double Y = e ? Y1 : Y0;             /* edge y = Y */
    const double x = clampd(-B * Y / A, X0, X1);
    const double qy = A * x * x + 2 * B * x * Y + C * Y * Y;
    if (qy < best) { best = qy; bx = x; by = Y; }
  }
  if (xm) { *xm = bx; *ym = by; }
  return best;
}

/*
 * The ellipse test of [SPIRULA] (16-bit AABB section), read as an exact test: tile (tx, ty)
 * of the rectangle stays in the Gaussian's list iff the box spanned by its pixel centres
 * (inside the Gaussian's pixel box) meets the support ellipse {q <= tau} around (u, v).
 * A pixel of a dropped tile has q > tau, so alpha < 1/255: the list only loses Gaussians
 * that cannot contribute.  With margin_flag non-NULL it is set when q's minimum lies
 * within the bound on how far rounding the record to float32 (the 2D mean and the conic)
 * can move it: such decisions may legitimately go either way in an implementation that
 * tests the rounded record.
 */
int orc_tile_keeps(double u, double v, double A, double B, double C, double tau, const int64_t px[4],
                   int64_t tx, int64_t ty, int* margin_flag) {
  const double X0 = (double)(tx * ORC_TILE > px[0] ? tx * ORC_TILE : px[0]) + 0.5 - u;
  const double X1 = (double)(tx * ORC_TILE + ORC_TILE - 1 < px[1] ? tx * ORC_TILE + ORC_TILE - 1 : px[1]) + 0.5 - u;
  const double Y0 = (double)(ty * ORC_TILE > px[2] ? ty * ORC_TILE : px[2]) + 0.5 - v;
  const double Y1 = (double)(ty * ORC_TILE + ORC_TILE - 1 < px[3] ? ty * ORC_TILE + ORC_TILE - 1 : px[3]) + 0.5 - v;
  double x, y;
  const double qmin = orc_box_min_q(A, B, C, X0, X1, Y0, Y1, &x, &y);
  if (margin_flag) {
    const double terms = fabs(A) * x * x + 2 * fabs(B * x * y) + fabs(C) * y * y;
    const double grad = 2 * fabs(A * x + B * y) * (fabs(u) + 1) + 2 * fabs(B * x + C * y) * (fabs(v) + 1);
    const double bound = 8 * ORC_EPS32 * (terms + grad + tau) + 1e-12 * tau;
    if (fabs(qmin - tau) <= bound) *margin_flag = 1;
  }
  return qmin <= tau;
}

/*
 * The forward projection of one Gaussian ([JULIA-1] s3.1-3.2; [JULIA-2] s3.1-3.2).
 * Culled Gaussians get visible = 0 and n_tiles = 0.
 */
static void project_one(const orc_camera* cam, const double mu[3], const double s[3],
                        const double q[4], double o, const double* sh, int L,
                        orc_gauss* g) {
  memset(g, 0, sizeof *g);
  const double* W = cam->R;
  /* view transform */
  for (int i = 0; i < 3; ++i)
    g->tc[i] = W[3 * i] * mu[0] + W[3 * i + 1] * mu[1] + W[3 * i + 2] * mu[2] + cam->t[i];
  const double x = g->tc[0], y = g->tc[1], z = g->tc[2];
  g->depth_bits = f32_bits(z);
  {
    /* flag a depth whose float32 rounding sits on a tie (double rounding could flip it) */
    float f = (float)z;
    double lo = nextafterf(f, -INFINITY), hi = nextafterf(f, INFINITY);
    double mid_lo = 0.5 * ((double)f + lo), mid_hi = 0.5 * ((double)f + hi);
    /* an exact tie is computed exactly by any float64 evaluation, so only near ties count */
    double tol = 8 * fabs(z) * 1.1102230246251565e-16;
    double e_lo = fabs(z - mid_lo), e_hi = fabs(z - mid_hi);
    if ((e_lo > 0 && e_lo <= tol) || (e_hi > 0 && e_hi <= tol)) g->flags |= 1;
  }

  /* colour: view direction from the camera centre -R^T t to the mean */
  double campos[3];
  for (int i = 0; i < 3; ++i)
    campos[i] = -(W[i] * cam->t[0] + W[3 + i] * cam->t[1] + W[6 + i] * cam->t[2]);
  double dv[3] = {mu[0] - campos[0], mu[1] - campos[1], mu[2] - campos[2]};
  g->dist = sqrt(dv[0] * dv[0] + dv[1] * dv[1] + dv[2] * dv[2]);
  for (int i = 0; i < 3; ++i) g->dir[i] = dv[i] / g->dist;
  const int K = (L + 1) * (L + 1);
  double Y[16];
  orc_sh_basis(L, g->dir, Y, NULL);
  for (int ch = 0; ch < 3; ++ch) {
    double acc = 0.5;
    for (int k = 0; k < K; ++k) acc += Y[k] * sh[3 * k + ch];
    g->raw[ch] = acc;
    g->clamp[ch] = acc < 0;
    g->rgb[ch] = acc < 0 ? 0.0 : acc;
    if (fabs(acc) <= 1e-6) g->flags |= 4;
  }

  /* 3D covariance from scale and quaternion: Sigma = (R S)(R S)^T */
  g->qlen = sqrt(q[0] * q[0] + q[1] * q[1] + q[2] * q[2] + q[3] * q[3]);
  for (int i = 0; i < 4; ++i) g->qn[i] = q[i] / g->qlen;
  quat_to_rot(g->qn, g->Rq);
  for (int i = 0; i < 3; ++i)
    for (int j = 0; j < 3; ++j) g->M[3 * i + j] = g->Rq[3 * i + j] * s[j];
  for (int i = 0; i < 3; ++i)
    for (int j = 0; j < 3; ++j) {
      double acc = 0;
      for (int k = 0; k < 3; ++k) acc += g->M[3 * i + k] * g->M[3 * j + k];
      g->Sig[3 * i + j] = acc;
    }

  if (!(z > cam->near_z)) return; /* near cull; NaN fails this test */

  /* EWA: Jacobian of the perspective map at the camera-space mean */
  g->J[0] = cam->fx / z; g->J[1] = 0;            g->J[2] = -cam->fx * x / (z * z);
  g->J[3] = 0;           g->J[4] = cam->fy / z;  g->J[5] = -cam->fy * y / (z * z);
  for (int r = 0; r < 2; ++r)
    for (int j = 0; j < 3; ++j) {
      double acc = 0;
      for (int k = 0; k < 3; ++k) acc += g->J[3 * r + k] * W[3 * k + j];
      g->T[3 * r + j] = acc;
    }
  double TS[6];
  for (int r = 0; r < 2; ++r)
    for (int j = 0; j < 3; ++j) {
      double acc = 0;
      for (int k = 0; k < 3; ++k) acc += g->T[3 * r + k] * g->Sig[3 * k + j];
      TS[3 * r + j] = acc;
    }
  double cov[4];
  for (int r = 0; r < 2; ++r)
    for (int cc = 0; cc < 2; ++cc) {
      double acc = 0;
      for (int k = 0; k < 3; ++k) acc += TS[3 * r + k] * g->T[3 * cc + k];
      cov[2 * r + cc] = acc;
    }
  g->a = cov[0]; g->b = 0.5 * (cov[1] + cov[2]); g->c = cov[3];
  g->det = g->a * g->c - g->b * g->b;
  g->u = cam->fx * x / z + cam->cx;
  g->v = cam->fy * y / z + cam->cy;
  /* the conic exists for det > 0; a 2D covariance that is a line to working precision is
     culled too: det <= 1e-9 (a + c)^2.  det / (a + c)^2 = l1 l2 / (l1 + l2)^2 for the
     eigenvalues l1 >= l2, so this is a screen-space axis ratio below ~3e-5, whatever the
     rotation.  A covariance of rank one (a zero scale) has det = 0 in exact arithmetic and
     rounding noise of either sign in practice, far below the threshold, where the sign of det
     alone would be decided by rounding.  A decision within 1e-11 (a + c)^2 of the threshold
     is flagged. */
  const double tr2 = (g->a + g->c) * (g->a + g->c);
  if (tr2 > 0 && fabs(g->det - 1e-9 * tr2) <= 1e-11 * tr2) g->flags |= 16;
  if (!(g->det > 1e-9 * tr2)) return;
  g->A = g->c / g->det; g->B = -g->b / g->det; g->C = g->a / g->det;

  /* support: alpha >= AMIN  <=>  q <= tau = 2 ln(o / AMIN) */
  if (!(o >= ORC_AMIN)) return;
  g->tau = 2.0 * log(o / ORC_AMIN);
  g->ex = sqrt(g->tau * g->a);
  g->ey = sqrt(g->tau * g->c);
  /* pixel (i, j) has its centre at (i + 0.5, j + 0.5) */
  double lx = ceil(g->u - g->ex - 0.5), hx = floor(g->u + g->ex - 0.5);
  double ly = ceil(g->v - g->ey - 0.5), hy = floor(g->v + g->ey - 0.5);
  double tol = 1e-9 * (fabs(g->u) + fabs(g->v) + g->ex + g->ey + 1.0);
  if (near_integer(g->u - g->ex - 0.5, tol) || near_integer(g->u + g->ex - 0.5, tol) ||
      near_integer(g->v - g->ey - 0.5, tol) || near_integer(g->v + g->ey - 0.5, tol))
    g->flags |= 2;
  if (lx < 0) lx = 0;
  if (ly < 0) ly = 0;
  if (hx > (double)(cam->width - 1)) hx = (double)(cam->width - 1);
  if (hy > (double)(cam->height - 1)) hy = (double)(cam->height - 1);
  if (!(lx <= hx) || !(ly <= hy)) return;
  g->px0 = (int64_t)lx; g->px1 = (int64_t)hx;
  g->py0 = (int64_t)ly; g->py1 = (int64_t)hy;
  g->tx0 = g->px0 / ORC_TILE; g->tx1 = g->px1 / ORC_TILE;
  g->ty0 = g->py0 / ORC_TILE; g->ty1 = g->py1 / ORC_TILE;
  /* the tiles of the rectangle that pass the ellipse test ([SPIRULA], 16-bit AABB section),
     applied to every rectangle whatever its size: the page sets no limit */
  const int64_t px[4] = {g->px0, g->px1, g->py0, g->py1};
  int near = 0;
  g->n_tiles = 0;
  for (int64_t ty = g->ty0; ty <= g->ty1; ++ty)
    for (int64_t tx = g->tx0; tx <= g->tx1; ++tx)
      g->n_tiles += orc_tile_keeps(g->u, g->v, g->A, g->B, g->C, g->tau, px, tx, ty, &near);
  if (near) g->flags |= 8;
  g->visible = g->n_tiles > 0;
}

/*
 * Project n Gaussians.  Outputs (all optional except n_tiles):
 *  uv[n][2], z[n], depth_bits[n], cov2d[n][3] (a, b, c), conic[n][3] (A, B, C),
 *  rgb[n][3], clamp[n] (bit per channel), pxrect[n][4] (px0, px1, py0, py1),
 *  trect[n][4] (tx0, tx1, ty0, ty1), n_tiles[n], flags[n].
 */
void orc_project(int64_t n, const double* means, const double* scales, const double* quats,
                 const double* opac, const double* sh, int L, const orc_camera* cam,
                 double* uv, double* zout, uint32_t* depth_bits, double* cov2d,
                 double* conic, double* rgb, uint8_t* clamp, int32_t* pxrect,
                 int32_t* trect, int64_t* n_tiles, uint8_t* flags) {
  const int K = (L + 1) * (L + 1);
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) {
    orc_gauss g;
    project_one(cam, means + 3 * i, scales + 3 * i, quats + 4 * i, opac[i], sh + 3 * K * i, L, &g);
    if (uv) { uv[2 * i] = g.u; uv[2 * i + 1] = g.v; }
    if (zout) zout[i] = g.tc[2];
    if (depth_bits) depth_bits[i] = g.depth_bits;
    if (cov2d) { cov2d[3 * i] = g.a; cov2d[3 * i + 1] = g.b; cov2d[3 * i + 2] = g.c; }
    if (conic) { conic[3 * i] = g.A; conic[3 * i + 1] = g.B; conic[3 * i + 2] = g.C; }
    if (rgb) for (int ch = 0; ch < 3; ++ch) rgb[3 * i + ch] = g.rgb[ch];
    if (clamp) clamp[i] = (uint8_t)(g.clamp[0] | (g.clamp[1] << 1) | (g.clamp[2] << 2));
    if (pxrect) {
      pxrect[4 * i] = (int32_t)g.px0; pxrect[4 * i + 1] = (int32_t)g.px1;
      pxrect[4 * i + 2] = (int32_t)g.py0; pxrect[4 * i + 3] = (int32_t)g.py1;
    }
    if (trect) {
      trect[4 * i] = (int32_t)g.tx0; trect[4 * i + 1] = (int32_t)g.tx1;
      trect[4 * i + 2] = (int32_t)g.ty0; trect[4 * i + 3] = (int32_t)g.ty1;
    }
    n_tiles[i] = g.visible ? g.n_tiles : 0;
    if (flags) flags[i] = (uint8_t)g.flags;
  }
}

/* ------------------------------------------------------------------------------------ */
/* Binning and sorting ([JULIA-2] s3.2: assign_to_tiles, sort_by_depth!)                */
/* ------------------------------------------------------------------------------------ */

/* Total pair count = sum of n_tiles. */
int64_t orc_count_pairs(int64_t n, const int64_t* n_tiles) {
  int64_t p = 0;
  for (int64_t i = 0; i < n; ++i) p += n_tiles[i];
  return p;
}

/*
 * Emit one (key, id) pair per kept tile, Gaussians in id order, rows (ty) outer and
 * columns (tx) inner.  key = tile_id * 2^32 + float32 depth bits, tile_id = ty*tiles_x+tx.
 * A tile of the rectangle is kept when it passes the ellipse test for the Gaussian's
 * ell[i] = (u, v, A, B, C, tau) and pixel box pxrect[i] (every tile when ell is NULL, for
 * hand-built lists); Gaussians with
 * n_tiles = 0 are skipped.  Writes at most capacity pairs; returns the number of kept tiles.
 */
int64_t orc_emit_pairs(int64_t n, const int32_t* trect, const int32_t* pxrect, const double* ell,
                       const int64_t* n_tiles, const uint32_t* depth_bits, int64_t tiles_x, uint64_t* keys,
                       uint32_t* vals, int64_t capacity) {
  int64_t p = 0;
  for (int64_t i = 0; i < n; ++i) {
    if (n_tiles[i] <= 0) continue;
    const double* e = ell ? ell + 6 * i : NULL;
    const int64_t px[4] = {pxrect ? pxrect[4 * i] : 0, pxrect ? pxrect[4 * i + 1] : 0,
                           pxrect ? pxrect[4 * i + 2] : 0, pxrect ? pxrect[4 * i + 3] : 0};
    for (int64_t ty = trect[4 * i + 2]; ty <= trect[4 * i + 3]; ++ty)
      for (int64_t tx = trect[4 * i]; tx <= trect[4 * i + 1]; ++tx) {
        if (e && !orc_tile_keeps(e[0], e[1], e[2], e[3], e[4], e[5], px, tx, ty, NULL)) continue;
        if (p < capacity) {
          uint64_t tile = (uint64_t)(ty * tiles_x + tx);
          keys[p] = (tile << 32) | (uint64_t)depth_bits[i];
          vals[p] = (uint32_t)i;
        }
        ++p;
      }
  }
  return p;
}

/* orc_tile_keeps for n Gaussians and one tile: keep[i], and near[i] the margin flag. */
void orc_tile_keeps_batch(int64_t n, const double* ell, const int64_t* pxrect, int64_t tx, int64_t ty,
                          int32_t* keep, int32_t* near) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) {
    const double* e = ell + 6 * i;
    int f = 0;
    keep[i] = orc_tile_keeps(e[0], e[1], e[2], e[3], e[4], e[5], pxrect + 4 * i, tx, ty, &f);
    near[i] = f;
  }
}

/* ell[i] = (u, v, A, B, C, tau) from 2D means, conics and opacities, with the support level
 * tau = 2 ln(o / AMIN) of project_one. */
void orc_ellipses(int64_t n, const double* uv, const double* conic, const double* opac, double* ell) {
  for (int64_t i = 0; i < n; ++i) {
    ell[6 * i] = uv[2 * i]; ell[6 * i + 1] = uv[2 * i + 1];
    for (int k = 0; k < 3; ++k) ell[6 * i + 2 + k] = conic[3 * i + k];
    ell[6 * i + 5] = opac[i] >= ORC_AMIN ? 2.0 * log(opac[i] / ORC_AMIN) : 0.0;
  }
}

/* Tiles kept, per Gaussian, as orc_emit_pairs counts them. */
void orc_count_kept(int64_t n, const int32_t* trect, const int32_t* pxrect, const double* ell, int64_t* out) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) {
    const double* e = ell + 6 * i;
    const int64_t px[4] = {pxrect[4 * i], pxrect[4 * i + 1], pxrect[4 * i + 2], pxrect[4 * i + 3]};
    int64_t c = 0;
    for (int64_t ty = trect[4 * i + 2]; ty <= trect[4 * i + 3]; ++ty)
      for (int64_t tx = trect[4 * i]; tx <= trect[4 * i + 1]; ++tx)
        c += orc_tile_keeps(e[0], e[1], e[2], e[3], e[4], e[5], px, tx, ty, NULL);
    out[i] = c;
  }
}

typedef struct { uint64_t key; uint32_t val; } orc_pair;

static int cmp_pair(const void* pa, const void* pb) {
  const orc_pair* a = (const orc_pair*)pa;
  const orc_pair* b = (const orc_pair*)pb;
  if (a->key != b->key) return a->key < b->key ? -1 : 1;
  if (a->val != b->val) return a->val < b->val ? -1 : 1;
  return 0;
}

/* Sort pairs by (key, id): the depth order inside each tile, ties broken by id. */
void orc_sort_pairs(int64_t p, uint64_t* keys, uint32_t* vals) {
  orc_pair* buf = (orc_pair*)malloc(sizeof(orc_pair) * (size_t)(p > 0 ? p : 1));
  for (int64_t i = 0; i < p; ++i) { buf[i].key = keys[i]; buf[i].val = vals[i]; }
  qsort(buf, (size_t)p, sizeof(orc_pair), cmp_pair);
  for (int64_t i = 0; i < p; ++i) { keys[i] = buf[i].key; vals[i] = buf[i].val; }
  free(buf);
}

/* ranges[t] = [first, last + 1) of tile t in the sorted keys; empty tiles get [0, 0). */
void orc_tile_ranges(int64_t p, const uint64_t* keys, int64_t num_tiles, int64_t* ranges) {
  for (int64_t t = 0; t < 2 * num_tiles; ++t) ranges[t] = 0;
  for (int64_t i = 0; i < p; ++i) {
    int64_t t = (int64_t)(keys[i] >> 32);
    if (i == 0 || (int64_t)(keys[i - 1] >> 32) != t) ranges[2 * t] = i;
    if (i == p - 1 || (int64_t)(keys[i + 1] >> 32) != t) ranges[2 * t + 1] = i + 1;
  }
}

/* ------------------------------------------------------------------------------------ */
/* Compositing ([JULIA-1] s3.3): front to back with transmittance.                      */
/* A record is (u, v, A, B, C, opacity, r, g, b) per Gaussian.                          */
/* ------------------------------------------------------------------------------------ */

#define ORC_REC 9
#define ORC_MAXBR 8

typedef struct {
  double col[3], T;
  int64_t n;          /* list position + 1 of the last contributor */
  int n_amb;          /* ambiguous decisions met on this run        */
  int n_clamp_amb;    /* alpha-clamp decisions near 0.99 (gradient only) */
} orc_pix;

/*
 * Composite one pixel over a list of Gaussian ids.  flip_mask flips the i-th ambiguous
 * decision met (bit i), so a caller can enumerate the results every correct evaluation
 * of the thresholds could give.  A decision is ambiguous when float32 rounding of the
 * same formula could land on the other side of its threshold.
 */
static void composite(const double* rec, const uint32_t* list, int64_t len, double px,
                      double py, const double bg[3], unsigned flip_mask, orc_pix* out) {
  double T = 1.0, col[3] = {0, 0, 0}, relT = 0.0;
  int64_t n = 0;
  int amb = 0, camb = 0;
  for (int64_t k = 0; k < len; ++k) {
    const double* r = rec + (size_t)ORC_REC * list[k];
    const double dx = px - r[0], dy = py - r[1];
    const double A = r[2], B = r[3], C = r[4], o = r[5];
    const double q = A * dx * dx + 2.0 * B * dx * dy + C * dy * dy;
    const double G = exp(-0.5 * q);
    double alpha = o * G;
    if (alpha > ORC_AMAX) alpha = ORC_AMAX;
    int take = !(alpha < ORC_AMIN);
    /* float32 error scale of q as the GPU evaluates it (inputs rounded to float32) */
    const double eq = ORC_EPS32 * (fabs(A) * dx * dx + 2 * fabs(B * dx * dy) + fabs(C) * dy * dy +
                                   2 * fabs(A * dx + B * dy) * (fabs(dx) + fabs(r[0]) + 1) +
                                   2 * fabs(B * dx + C * dy) * (fabs(dy) + fabs(r[1]) + 1) + 2);
    const double tau = o > 0 ? 2.0 * log(o / ORC_AMIN) : -INFINITY;
    const double relA = 0.5 * eq + ORC_EPS32 * (4 + fabs(q));
    if (fabs(q - tau) <= 16 * (eq + ORC_EPS32 * (4 + fabs(tau)))) {
      if (flip_mask & (1u << amb)) take = !take;
      ++amb;
    }
    if (!take) continue;
    if (fabs(o * G / ORC_AMAX - 1.0) <= 16 * relA) ++camb;
    for (int ch = 0; ch < 3; ++ch) col[ch] += r[6 + ch] * alpha * T;
    T *= (1.0 - alpha);
    relT += 2 * ORC_EPS32 + relA * alpha / (1.0 - alpha);
    n = k + 1;
    int stop = T < ORC_TMIN;
    if (fabs(T / ORC_TMIN - 1.0) <= 16 * relT) {
      if (flip_mask & (1u << amb)) stop = !stop;
      ++amb;
    }
    if (stop) break;
  }
  for (int ch = 0; ch < 3; ++ch) out->col[ch] = col[ch] + T * bg[ch];
  out->T = T;
  out->n = n;
  out->n_amb = amb;
  out->n_clamp_amb = camb;
}

/* Pixel list = the tile's slice of the sorted ids. */
static void tile_list(int64_t i, int64_t j, int64_t tiles_x, const int64_t* ranges,
                      const uint32_t* vals, const uint32_t** list, int64_t* len) {
  const int64_t t = (j / ORC_TILE) * tiles_x + (i / ORC_TILE);
  *list = vals + ranges[2 * t];
  *len = ranges[2 * t + 1] - ranges[2 * t];
}

/*
 * Tiled render of the pixels in pix[] (linear index j*W + i), or of every pixel when
 * pix == NULL (then npix must be W*H).  Per pixel it writes the natural result
 * (out_col[3], out_T, out_n) and, in branches[npix][ORC_MAXBR][5] (r, g, b, T, n), the
 * results of all flips of up to three ambiguous decisions; nbranch = 1, 2, 4 or 8, or 0
 * when the pixel has more than three ambiguous decisions.  amb_flags: bit0 any ambiguous
 * threshold decision, bit1 an alpha near the 0.99 clamp.
 * Output arrays are indexed by position in pix[] (or by the pixel when pix == NULL).
 */
void orc_render_pixels(int64_t W, int64_t H, const double bg[3], const double* rec,
                       const uint32_t* vals, const int64_t* ranges, int64_t npix,
                       const int64_t* pix, double* out_col, double* out_T, int64_t* out_n,
                       double* branches, int32_t* nbranch, uint8_t* amb_flags) {
  const int64_t tiles_x = (W + ORC_TILE - 1) / ORC_TILE;
  (void)H;
#pragma omp parallel for schedule(dynamic, 256)
  for (int64_t p = 0; p < npix; ++p) {
    const int64_t lin = pix ? pix[p] : p;
    const int64_t i = lin % W, j = lin / W;
    const uint32_t* list;
    int64_t len;
    tile_list(i, j, tiles_x, ranges, vals, &list, &len);
    orc_pix r0;
    composite(rec, list, len, i + 0.5, j + 0.5, bg, 0u, &r0);
    out_col[3 * p] = r0.col[0]; out_col[3 * p + 1] = r0.col[1]; out_col[3 * p + 2] = r0.col[2];
    out_T[p] = r0.T;
    out_n[p] = r0.n;
    if (amb_flags) amb_flags[p] = (uint8_t)((r0.n_amb > 0) | ((r0.n_clamp_amb > 0) << 1));
    if (branches) {
      int nb = r0.n_amb <= 3 ? 1 << r0.n_amb : 0;
      nbranch[p] = nb;
      double* br = branches + (size_t)p * ORC_MAXBR * 5;
      for (int m = 0; m < ORC_MAXBR; ++m)
        for (int e = 0; e < 5; ++e) br[5 * m + e] = NAN;
      for (int m = 0; m < nb; ++m) {
        orc_pix rb;
        composite(rec, list, len, i + 0.5, j + 0.5, bg, (unsigned)m, &rb);
        br[5 * m] = rb.col[0]; br[5 * m + 1] = rb.col[1]; br[5 * m + 2] = rb.col[2];
        br[5 * m + 3] = rb.T; br[5 * m + 4] = (double)rb.n;
      }
    }
  }
}

/*
 * Brute-force render: every pixel composites the given order of ids (all visible
 * Gaussians sorted by (depth bits, id)), with no tiles.  image[3][H][W], T[H][W].
 */
void orc_render_brute(int64_t W, int64_t H, const double bg[3], const double* rec,
                      const uint32_t* order, int64_t len, double* image, double* Tout) {
#pragma omp parallel for schedule(dynamic, 16)
  for (int64_t lin = 0; lin < W * H; ++lin) {
    const int64_t i = lin % W, j = lin / W;
    orc_pix r;
    composite(rec, order, len, i + 0.5, j + 0.5, bg, 0u, &r);
    for (int ch = 0; ch < 3; ++ch) image[ch * W * H + lin] = r.col[ch];
    Tout[lin] = r.T;
  }
}

/* ------------------------------------------------------------------------------------ */
/* Backward through compositing: exact derivative of the forward above.                  */
/* grad_screen[n][10] = dL/d(u, v, A, B, C, opacity, r, g, b) and sum_p ||dL_p/d(u, v)||. */
/* ------------------------------------------------------------------------------------ */
void orc_render_bwd(int64_t W, int64_t H, const double bg[3], const double* rec,
                    const uint32_t* vals, const int64_t* ranges, int64_t n,
                    const double* dL_dimg, double* grad_screen, double* grad_abs,
                    double* grad_err, int64_t npix, const int64_t* pix) {
  /* pix (optional): only these pixels (linear j*W + i) contribute; NULL = all W*H. */
  /* grad_abs (optional): per element, the sum of |per-pixel terms|, so a caller can tell
   * an ill-conditioned sum (|sum| << sum |terms|) from a wrong one. */
  /* grad_err (optional): per element, a scale of the rounding that a float32 reverse walk
   * carries into the terms: the walk recovers T by dividing by (1 - alpha) and sums the
   * colour behind one contributor at a time, so at the contributor with s contributors
   * behind it both carry about s roundings, and they enter the term through dL/dalpha =
   * T dC.c - dC.behind / (1 - alpha), whose parts may cancel.  Each term adds
   * (s + 1) * sum_ch |dC_ch| (c_ch T + behind_ch / (1 - alpha)) * |d term / d dL/dalpha|
   * (for the colour terms, (s + 1) * |term|). */
  const int64_t tiles_x = (W + ORC_TILE - 1) / ORC_TILE;
  memset(grad_screen, 0, sizeof(double) * 10 * (size_t)n);
  if (grad_abs) memset(grad_abs, 0, sizeof(double) * 10 * (size_t)n);
  if (grad_err) memset(grad_err, 0, sizeof(double) * 10 * (size_t)n);
#pragma omp parallel
  {
    int64_t cap = 1024;
    uint32_t* ids = (uint32_t*)malloc(sizeof(uint32_t) * cap);
    double* st = (double*)malloc(sizeof(double) * 6 * cap);
    const int64_t count = pix ? npix : W * H;
#pragma omp for schedule(dynamic, 64)
    for (int64_t pi = 0; pi < count; ++pi) {
      const int64_t lin = pix ? pix[pi] : pi;
      const int64_t i = lin % W, j = lin / W;
      const double px = i + 0.5, py = j + 0.5;
      const uint32_t* list;
      int64_t len;
      tile_list(i, j, tiles_x, ranges, vals, &list, &len);
      /* forward, keeping every contributor's state */
      double T = 1.0;
      int64_t m = 0;
      for (int64_t k = 0; k < len; ++k) {
        const double* r = rec + (size_t)ORC_REC * list[k];
        const double dx = px - r[0], dy = py - r[1];
        const double q = r[2] * dx * dx + 2.0 * r[3] * dx * dy + r[4] * dy * dy;
        const double G = exp(-0.5 * q);
        const double oG = r[5] * G;
        const double alpha = oG > ORC_AMAX ? ORC_AMAX : oG;
        if (alpha < ORC_AMIN) continue;
        if (m == cap) {
          cap *= 2;
          ids = (uint32_t*)realloc(ids, sizeof(uint32_t) * cap);
          st = (double*)realloc(st, sizeof(double) * 6 * cap);
        }
        ids[m] = list[k];
        st[6 * m] = alpha; st[6 * m + 1] = T; st[6 * m + 2] = G;
        st[6 * m + 3] = dx; st[6 * m + 4] = dy; st[6 * m + 5] = oG > ORC_AMAX ? 1.0 : 0.0;
        ++m;
        T *= (1.0 - alpha);
        if (T < ORC_TMIN) break;
      }
      const double dC[3] = {dL_dimg[lin], dL_dimg[W * H + lin], dL_dimg[2 * W * H + lin]};
      /* colour behind contributor k: sum_{j>k} c_j alpha_j T_j + bg T_final */
      double behind[3] = {bg[0] * T, bg[1] * T, bg[2] * T};
      for (int64_t k = m - 1; k >= 0; --k) {
        const uint32_t id = ids[k];
        const double* r = rec + (size_t)ORC_REC * id;
        const double alpha = st[6 * k], Tk = st[6 * k + 1], G = st[6 * k + 2];
        const double dx = st[6 * k + 3], dy = st[6 * k + 4];
        const int clamped = st[6 * k + 5] != 0.0;
        double g[10] = {0};
        double dL_dalpha = 0, parts = 0;
        for (int ch = 0; ch < 3; ++ch) {
          g[6 + ch] = dC[ch] * alpha * Tk;
          dL_dalpha += dC[ch] * (r[6 + ch] * Tk - behind[ch] / (1.0 - alpha));
          parts += fabs(dC[ch]) * (r[6 + ch] * Tk + behind[ch] / (1.0 - alpha));
        }
        double es[10] = {0};  /* |d term / d dL/dalpha|, the colour terms' own size */
        const double steps = (double)(m - k);
        for (int ch = 0; ch < 3; ++ch) behind[ch] += r[6 + ch] * alpha * Tk;
        if (!clamped) {
          const double o = r[5];
          const double dL_dq = dL_dalpha * (-0.5 * o * G);
          g[5] = dL_dalpha * G;
          g[2] = dL_dq * dx * dx;
          g[3] = dL_dq * 2.0 * dx * dy;
          g[4] = dL_dq * dy * dy;
          /* dx = px - u, so dq/du = -(2 A dx + 2 B dy) */
          g[0] = dL_dq * (-2.0 * (r[2] * dx + r[3] * dy));
          g[1] = dL_dq * (-2.0 * (r[3] * dx + r[4] * dy));
          g[9] = sqrt(g[0] * g[0] + g[1] * g[1]);
          const double h = 0.5 * o * G, mu = 2.0 * fabs(r[2] * dx + r[3] * dy), mv = 2.0 * fabs(r[3] * dx + r[4] * dy);
          es[5] = parts * G;
          es[2] = parts * h * dx * dx;
          es[3] = parts * h * 2.0 * fabs(dx * dy);
          es[4] = parts * h * dy * dy;
          es[0] = parts * h * mu;
          es[1] = parts * h * mv;
          es[9] = parts * h * sqrt(mu * mu + mv * mv);
        }
        for (int ch = 0; ch < 3; ++ch) es[6 + ch] = fabs(g[6 + ch]);
        double* out = grad_screen + 10 * (size_t)id;
        for (int e = 0; e < 10; ++e) {
#pragma omp atomic
          out[e] += g[e];
        }
        if (grad_abs) {
          double* oa = grad_abs + 10 * (size_t)id;
          for (int c = 0; c < 10; ++c) {
#pragma omp atomic
            oa[c] += fabs(g[c]);
          }
        }
        if (grad_err) {
          double* oe = grad_err + 10 * (size_t)id;
          for (int c = 0; c < 10; ++c) {
#pragma omp atomic
            oe[c] += steps * es[c];
          }
        }
      }
    }
    free(ids);
    free(st);
  }
}

/* ------------------------------------------------------------------------------------ */
/* Backward through the projection, per Gaussian, and densification statistics          */
/* ([ABSGRAD] s1-s3: accum[:,0] += ||dL/d(u,v)||, accum[:,1] += sum_p ||g_p||, denom).  */
/* ------------------------------------------------------------------------------------ */
void orc_project_bwd(int64_t n, const double* means, const double* scales, const double* quats,
                     const double* opac, const double* sh, int L, const orc_camera* cam,
                     const double* grad_screen, double* dmeans, double* dscales,
                     double* dquats, double* dopac, double* dsh, double* accum,
                     int64_t* denom) {
  const int K = (L + 1) * (L + 1);
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) {
    orc_gauss g;
    const double* s = scales + 3 * i;
    project_one(cam, means + 3 * i, s, quats + 4 * i, opac[i], sh + 3 * K * i, L, &g);
    const double* gs = grad_screen + 10 * i;
    double dmu[3] = {0, 0, 0}, ds[3] = {0, 0, 0}, dq[4] = {0, 0, 0, 0};
    double* dshi = dsh + 3 * (size_t)K * i;
    for (int k = 0; k < 3 * K; ++k) dshi[k] = 0;
    dopac[i] = g.visible ? gs[5] : 0.0;
    if (g.visible) {
      const double* W = cam->R;
      /* colour: rgb = max(raw, 0), raw = 0.5 + sum_k Y_k(d) sh_k */
      double draw[3];
      for (int ch = 0; ch < 3; ++ch) draw[ch] = g.raw[ch] < 0 ? 0.0 : gs[6 + ch];
      double Y[16], dY[48];
      orc_sh_basis(L, g.dir, Y, dY);
      double ddir[3] = {0, 0, 0};
      for (int k = 0; k < K; ++k)
        for (int ch = 0; ch < 3; ++ch) {
          dshi[3 * k + ch] = Y[k] * draw[ch];
          for (int e = 0; e < 3; ++e) ddir[e] += sh[3 * K * i + 3 * k + ch] * draw[ch] * dY[3 * k + e];
        }
      /* d = (mu - campos)/|mu - campos|: dd/dmu = (I - d d^T)/|mu - campos| */
      double dd = ddir[0] * g.dir[0] + ddir[1] * g.dir[1] + ddir[2] * g.dir[2];
      for (int e = 0; e < 3; ++e) dmu[e] += (ddir[e] - dd * g.dir[e]) / g.dist;

      /* conic (A, B, C) = (c, -b, a)/det, det = a c - b^2 */
      const double a = g.a, b = g.b, c = g.c, det = g.det, d2 = det * det;
      const double dA = gs[2], dB = gs[3], dC = gs[4];
      const double dAda = -c * c / d2, dAdb = 2 * b * c / d2, dAdc = (det - a * c) / d2;
      const double dBda = b * c / d2, dBdb = -(det + 2 * b * b) / d2, dBdc = a * b / d2;
      const double dCda = (det - a * c) / d2, dCdb = 2 * a * b / d2, dCdc = -a * a / d2;
      const double da = dA * dAda + dB * dBda + dC * dCda;
      const double db = dA * dAdb + dB * dBdb + dC * dCdb;
      const double dc = dA * dAdc + dB * dBdc + dC * dCdc;
      /* a = t0^T S t0, b = t0^T S t1, c = t1^T S t1 with t0, t1 the rows of T = J W */
      const double* t0 = g.T;
      const double* t1 = g.T + 3;
      double St0[3], St1[3];
      for (int r = 0; r < 3; ++r) {
        St0[r] = g.Sig[3 * r] * t0[0] + g.Sig[3 * r + 1] * t0[1] + g.Sig[3 * r + 2] * t0[2];
        St1[r] = g.Sig[3 * r] * t1[0] + g.Sig[3 * r + 1] * t1[1] + g.Sig[3 * r + 2] * t1[2];
      }
      /* dL/dSigma (full 3x3, entries treated as independent) */
      double dSig[9];
      for (int r = 0; r < 3; ++r)
        for (int cc = 0; cc < 3; ++cc)
          dSig[3 * r + cc] = da * t0[r] * t0[cc] + db * t0[r] * t1[cc] + dc * t1[r] * t1[cc];
      double dT[6];
      for (int e = 0; e < 3; ++e) {
        dT[e] = 2 * da * St0[e] + db * St1[e];
        dT[3 + e] = db * St0[e] + 2 * dc * St1[e];
      }
      /* T = J W  ->  dJ = dT W^T */
      double dJ[6];
      for (int r = 0; r < 2; ++r)
        for (int k = 0; k < 3; ++k)
          dJ[3 * r + k] = dT[3 * r] * W[3 * k] + dT[3 * r + 1] * W[3 * k + 1] + dT[3 * r + 2] * W[3 * k + 2];
      const double x = g.tc[0], y = g.tc[1], z = g.tc[2];
      const double fx = cam->fx, fy = cam->fy;
      double dt[3] = {0, 0, 0};
      /* J = [[fx/z, 0, -fx x/z^2], [0, fy/z, -fy y/z^2]] */
      dt[0] += dJ[2] * (-fx / (z * z));
      dt[1] += dJ[5] * (-fy / (z * z));
      dt[2] += dJ[0] * (-fx / (z * z)) + dJ[2] * (2 * fx * x / (z * z * z)) +
               dJ[4] * (-fy / (z * z)) + dJ[5] * (2 * fy * y / (z * z * z));
      /* u = fx x/z + cx, v = fy y/z + cy */
      const double du = gs[0], dv = gs[1];
      dt[0] += du * fx / z;
      dt[1] += dv * fy / z;
      dt[2] += du * (-fx * x / (z * z)) + dv * (-fy * y / (z * z));
      /* t = W mu + t_cam */
      for (int e = 0; e < 3; ++e) dmu[e] += W[e] * dt[0] + W[3 + e] * dt[1] + W[6 + e] * dt[2];
      /* Sigma = M M^T, M = Rq diag(s) */
      double dM[9];
      for (int r = 0; r < 3; ++r)
        for (int cc = 0; cc < 3; ++cc) {
          double acc = 0;
          for (int k = 0; k < 3; ++k) acc += (dSig[3 * r + k] + dSig[3 * k + r]) * g.M[3 * k + cc];
          dM[3 * r + cc] = acc;
        }
      double dR[9];
      for (int r = 0; r < 3; ++r)
        for (int cc = 0; cc < 3; ++cc) {
          ds[cc] += dM[3 * r + cc] * g.Rq[3 * r + cc];
          dR[3 * r + cc] = dM[3 * r + cc] * s[cc];
        }
      double J4[4][9];
      quat_rot_jac(g.qn, J4);
      double dqn[4];
      for (int e = 0; e < 4; ++e) {
        double acc = 0;
        for (int k = 0; k < 9; ++k) acc += dR[k] * J4[e][k];
        dqn[e] = acc;
      }
      /* qn = q/|q|: dq = (I - qn qn^T) dqn / |q| */
      double proj = dqn[0] * g.qn[0] + dqn[1] * g.qn[1] + dqn[2] * g.qn[2] + dqn[3] * g.qn[3];
      for (int e = 0; e < 4; ++e) dq[e] = (dqn[e] - proj * g.qn[e]) / g.qlen;
      if (accum) {
        accum[2 * i] += sqrt(du * du + dv * dv);
        accum[2 * i + 1] += gs[9];
      }
      if (denom) denom[i] += 1;
    }
    for (int e = 0; e < 3; ++e) { dmeans[3 * i + e] = dmu[e]; dscales[3 * i + e] = ds[e]; }
    for (int e = 0; e < 4; ++e) dquats[4 * i + e] = dq[e];
  }
}

/* ------------------------------------------------------------------------------------ */
/* Whole forward from raw parameters (for finite differences and end-to-end checks).     */
/* ------------------------------------------------------------------------------------ */

/* records from an orc_project run: (u, v, A, B, C, o, r, g, b) */
void orc_make_records(int64_t n, const double* uv, const double* conic, const double* opac,
                      const double* rgb, double* rec) {
  for (int64_t i = 0; i < n; ++i) {
    double* r = rec + ORC_REC * i;
    r[0] = uv[2 * i]; r[1] = uv[2 * i + 1];
    r[2] = conic[3 * i]; r[3] = conic[3 * i + 1]; r[4] = conic[3 * i + 2];
    r[5] = opac[i];
    r[6] = rgb[3 * i]; r[7] = rgb[3 * i + 1]; r[8] = rgb[3 * i + 2];
  }
}

/*
 * Project, bin, sort and composite every pixel.  Writes image[3][H][W], T[H][W],
 * n_contrib[H][W] and returns a hash of the discrete decisions (the sorted (tile, id)
 * list and every pixel's contributor sequence), so a finite-difference probe can tell
 * whether a perturbation crossed a threshold.
 */
uint64_t orc_forward(int64_t n, const double* means, const double* scales, const double* quats,
                     const double* opac, const double* sh, int L, const orc_camera* cam,
                     const double bg[3], double* image, double* Tout, int64_t* ncontrib) {
  const int K = (L + 1) * (L + 1);
  (void)K;
  const int64_t W = cam->width, H = cam->height;
  const int64_t tiles_x = (W + ORC_TILE - 1) / ORC_TILE, tiles_y = (H + ORC_TILE - 1) / ORC_TILE;
  double* uv = (double*)malloc(sizeof(double) * 2 * n);
  double* conic = (double*)malloc(sizeof(double) * 3 * n);
  double* rgb = (double*)malloc(sizeof(double) * 3 * n);
  uint32_t* db = (uint32_t*)malloc(sizeof(uint32_t) * n);
  int32_t* trect = (int32_t*)malloc(sizeof(int32_t) * 4 * n);
  int32_t* pxrect = (int32_t*)malloc(sizeof(int32_t) * 4 * n);
  int64_t* nt = (int64_t*)malloc(sizeof(int64_t) * n);
  double* rec = (double*)malloc(sizeof(double) * ORC_REC * n);
  double* ell = (double*)malloc(sizeof(double) * 6 * n);
  orc_project(n, means, scales, quats, opac, sh, L, cam, uv, NULL, db, NULL, conic, rgb, NULL,
              pxrect, trect, nt, NULL);
  orc_make_records(n, uv, conic, opac, rgb, rec);
  orc_ellipses(n, uv, conic, opac, ell);
  const int64_t P = orc_count_pairs(n, nt);
  uint64_t* keys = (uint64_t*)malloc(sizeof(uint64_t) * (P > 0 ? P : 1));
  uint32_t* vals = (uint32_t*)malloc(sizeof(uint32_t) * (P > 0 ? P : 1));
  orc_emit_pairs(n, trect, pxrect, ell, nt, db, tiles_x, keys, vals, P);
  orc_sort_pairs(P, keys, vals);
  int64_t* ranges = (int64_t*)malloc(sizeof(int64_t) * 2 * tiles_x * tiles_y);
  orc_tile_ranges(P, keys, tiles_x * tiles_y, ranges);
  double* col = (double*)malloc(sizeof(double) * 3 * W * H);
  orc_render_pixels(W, H, bg, rec, vals, ranges, W * H, NULL, col, Tout, ncontrib, NULL, NULL,
                    NULL);
  for (int64_t p = 0; p < W * H; ++p)
    for (int ch = 0; ch < 3; ++ch) image[ch * W * H + p] = col[3 * p + ch];
  /* decision hash (FNV-1a) */
  uint64_t h = 1469598103934665603ull;
#define ORC_MIX(x) do { h ^= (uint64_t)(x); h *= 1099511628211ull; } while (0)
  for (int64_t i = 0; i < P; ++i) { ORC_MIX(keys[i] >> 32); ORC_MIX(vals[i]); }
  for (int64_t p = 0; p < W * H; ++p) {
    const int64_t i = p % W, j = p / W;
    const uint32_t* list;
    int64_t len;
    tile_list(i, j, tiles_x, ranges, vals, &list, &len);
    ORC_MIX(ncontrib[p]);
    for (int64_t k = 0; k < ncontrib[p]; ++k) {
      const double* r = rec + ORC_REC * list[k];
      const double dx = i + 0.5 - r[0], dy = j + 0.5 - r[1];
      const double q = r[2] * dx * dx + 2 * r[3] * dx * dy + r[4] * dy * dy;
      const double oG = r[5] * exp(-0.5 * q);
      const double a = oG > ORC_AMAX ? ORC_AMAX : oG;
      ORC_MIX((a < ORC_AMIN ? 0u : 1u) | (oG > ORC_AMAX ? 2u : 0u));
    }
  }
#undef ORC_MIX
  free(uv); free(conic); free(rgb); free(db); free(trect); free(pxrect); free(nt); free(rec); free(ell);
  free(keys); free(vals); free(ranges); free(col);
  return h;
}
