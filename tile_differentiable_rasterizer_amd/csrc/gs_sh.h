// gs_sh.h -- real spherical harmonics up to degree 3 (Condon-Shortley phase, index
// l*l + l + m) as polynomials of a unit direction, for view-dependent colour.
// "Better Gaussian Splatting in Julia" (lshu.cn) s3.1: the number of SH coefficients per
// Gaussian grows with the degree; the basis is the standard real one.
#pragma once

#include <hip/hip_runtime.h>

namespace gs {

// Normalisation constants of the real SH basis.
constexpr float kY00 = 0.28209479177387814f;   // 1 / (2 sqrt(pi))
constexpr float kY1 = 0.4886025119029199f;     // sqrt(3 / (4 pi))
constexpr float kY2a = 1.0925484305920792f;    // sqrt(15 / pi) / 2
constexpr float kY2b = 0.31539156525252005f;   // sqrt(5 / pi) / 4
constexpr float kY2c = 0.5462742152960396f;    // sqrt(15 / pi) / 4
constexpr float kY3a = 0.5900435899266435f;    // sqrt(35 / (2 pi)) / 4
constexpr float kY3b = 2.890611442640554f;     // sqrt(105 / pi) / 2
constexpr float kY3c = 0.4570457994644658f;    // sqrt(21 / (2 pi)) / 4
constexpr float kY3d = 0.3731763325901154f;    // sqrt(7 / pi) / 4
constexpr float kY3e = 1.445305721320277f;     // sqrt(105 / pi) / 4

// Basis values Y[0 .. (L+1)^2) at the unit direction (x, y, z).
template <int L>
__device__ __forceinline__ void sh_basis(float x, float y, float z, float* Y) {
  Y[0] = kY00;
  if constexpr (L >= 1) {
    Y[1] = -kY1 * y;
    Y[2] = kY1 * z;
    Y[3] = -kY1 * x;
  }
  if constexpr (L >= 2) {
    const float xx = x * x, yy = y * y, zz = z * z;
    Y[4] = kY2a * x * y;
    Y[5] = -kY2a * y * z;
    Y[6] = kY2b * (3.0f * zz - 1.0f);
    Y[7] = -kY2a * x * z;
    Y[8] = kY2c * (xx - yy);
    if constexpr (L >= 3) {
      Y[9] = -kY3a * y * (3.0f * xx - yy);
      Y[10] = kY3b * x * y * z;
      Y[11] = -kY3c * y * (5.0f * zz - 1.0f);
      Y[12] = kY3d * z * (5.0f * zz - 3.0f);
      Y[13] = -kY3c * x * (5.0f * zz - 1.0f);
      Y[14] = kY3e * z * (xx - yy);
      Y[15] = -kY3a * x * (xx - 3.0f * yy);
    }
  }
}

// Gradient of each basis polynomial with respect to (x, y, z): dY[k][0..2].
template <int L>
__device__ __forceinline__ void sh_basis_grad(float x, float y, float z, float (*dY)[3]) {
  dY[0][0] = dY[0][1] = dY[0][2] = 0.0f;
  if constexpr (L >= 1) {
    dY[1][0] = 0.0f;  dY[1][1] = -kY1; dY[1][2] = 0.0f;
    dY[2][0] = 0.0f;  dY[2][1] = 0.0f; dY[2][2] = kY1;
    dY[3][0] = -kY1;  dY[3][1] = 0.0f; dY[3][2] = 0.0f;
  }
  if constexpr (L >= 2) {
    const float xx = x * x, yy = y * y, zz = z * z;
    dY[4][0] = kY2a * y;         dY[4][1] = kY2a * x;          dY[4][2] = 0.0f;
    dY[5][0] = 0.0f;             dY[5][1] = -kY2a * z;         dY[5][2] = -kY2a * y;
    dY[6][0] = 0.0f;             dY[6][1] = 0.0f;              dY[6][2] = 6.0f * kY2b * z;
    dY[7][0] = -kY2a * z;        dY[7][1] = 0.0f;              dY[7][2] = -kY2a * x;
    dY[8][0] = 2.0f * kY2c * x;  dY[8][1] = -2.0f * kY2c * y;  dY[8][2] = 0.0f;
    if constexpr (L >= 3) {
      dY[9][0] = -6.0f * kY3a * x * y;
      dY[9][1] = -3.0f * kY3a * (xx - yy);
      dY[9][2] = 0.0f;
      dY[10][0] = kY3b * y * z;
      dY[10][1] = kY3b * x * z;
      dY[10][2] = kY3b * x * y;
      dY[11][0] = 0.0f;
      dY[11][1] = -kY3c * (5.0f * zz - 1.0f);
      dY[11][2] = -10.0f * kY3c * y * z;
      dY[12][0] = 0.0f;
      dY[12][1] = 0.0f;
      dY[12][2] = kY3d * (15.0f * zz - 3.0f);
      dY[13][0] = -kY3c * (5.0f * zz - 1.0f);
      dY[13][1] = 0.0f;
      dY[13][2] = -10.0f * kY3c * x * z;
      dY[14][0] = 2.0f * kY3e * x * z;
      dY[14][1] = -2.0f * kY3e * y * z;
      dY[14][2] = kY3e * (xx - yy);
      dY[15][0] = -3.0f * kY3a * (xx - yy);
      dY[15][1] = 6.0f * kY3a * x * y;
      dY[15][2] = 0.0f;
    }
  }
}

}  // namespace gs
