"""Pins for the oracle's spherical harmonics (colour up to degree 3).

"Better Gaussian Splatting in Julia" (lshu.cn) s3.1 lists SH coefficients whose count
depends on the degree; the reading is the real SH basis with the Condon-Shortley phase,
pinned here by the addition theorem, orthonormality on the sphere and SciPy's complex
spherical harmonics (a library routine independent of the oracle).
"""
import math

import numpy as np
import pytest
from scipy import special

DIRS = np.random.default_rng(11).normal(size=(64, 3))
DIRS /= np.linalg.norm(DIRS, axis=1, keepdims=True)


def test_addition_theorem(orc):
    for d in DIRS:
        Y, _ = orc.sh_basis(3, d)
        for l in range(4):
            band = Y[l * l:(l + 1) * (l + 1)]
            assert np.sum(band * band) == pytest.approx((2 * l + 1) / (4 * math.pi), rel=1e-12)


def test_orthonormal_by_quadrature(orc):
    # Gauss-Legendre in cos(theta) x trapezoid in phi: exact for degree <= 6 products
    xs, ws = np.polynomial.legendre.leggauss(8)
    nphi = 16
    G = np.zeros((16, 16))
    for ct, w in zip(xs, ws):
        st = math.sqrt(1 - ct * ct)
        for k in range(nphi):
            ph = 2 * math.pi * k / nphi
            Y, _ = orc.sh_basis(3, (st * math.cos(ph), st * math.sin(ph), ct))
            G += w * (2 * math.pi / nphi) * np.outer(Y, Y)
    assert np.allclose(G, np.eye(16), atol=1e-12)


def _real_sh_scipy(l, m, d):
    x, y, z = d
    theta = math.acos(max(-1.0, min(1.0, z)))
    phi = math.atan2(y, x)
    Ylm = special.sph_harm_y(l, abs(m), theta, phi)  # includes the Condon-Shortley phase
    if m > 0:
        return math.sqrt(2) * Ylm.real
    if m < 0:
        return math.sqrt(2) * Ylm.imag
    return Ylm.real


def test_matches_scipy_real_basis(orc):
    for d in DIRS[:16]:
        Y, _ = orc.sh_basis(3, d)
        for l in range(4):
            for m in range(-l, l + 1):
                assert Y[l * l + l + m] == pytest.approx(_real_sh_scipy(l, m, d), abs=1e-12)


def test_gradient_tangential_part_matches_finite_differences(orc):
    """The polynomial gradient, projected on the sphere's tangent plane, is the derivative
    along the sphere (what the colour backward uses)."""
    rng = np.random.default_rng(5)
    for d in DIRS[:8]:
        Y, dY = orc.sh_basis(3, d)
        for _ in range(3):
            t = rng.normal(size=3)
            t -= t.dot(d) * d
            t /= np.linalg.norm(t)
            h = 1e-6
            dp = (d + h * t) / np.linalg.norm(d + h * t)
            dm = (d - h * t) / np.linalg.norm(d - h * t)
            fd = (orc.sh_basis(3, dp)[0] - orc.sh_basis(3, dm)[0]) / (2 * h)
            assert np.allclose(dY @ t, fd, atol=1e-8)


def test_degree0_colour_is_view_independent(orc):
    from tile_differentiable_rasterizer_amd.scenes import Scene, orbit_camera

    sc = Scene(np.array([[0.1, 0.2, 0.3]], np.float32), np.full((1, 3), 0.05, np.float32),
               np.array([[1, 0, 0, 0]], np.float32), np.array([0.9], np.float32),
               np.array([[[0.3, -0.2, 1.1]]], np.float32), 0)
    cols = [orc.project(sc, orbit_camera(th, 200, 200))["rgb"][0] for th in (0.0, 1.0, 2.5)]
    c0 = 0.5 / math.sqrt(math.pi)
    k = np.array([0.3, -0.2, 1.1], np.float32).astype(np.float64)
    for c in cols:
        assert np.allclose(c, 0.5 + c0 * k, atol=1e-14)
