"""Pins for the oracle's tile test (the ellipse test after the screen box).

"Training 10M Gaussians in 8 GB: Spirula Studio's VRAM efficiency" (mhpq.cn), 16-bit AABB
section: a conservative box followed by an ellipse test as a second cull leaves the image
unchanged.  Read as an exact test: a tile stays in a Gaussian's list iff the box spanned by
its pixel centres (inside the Gaussian's pixel box) meets the support ellipse q <= tau.

The box minimum is checked against dense sampling, the tile test against the closed form
for circles (distance from the centre to the box), the lists against brute force over
pixel centres (every pixel with q <= tau lies in a kept tile), and a thin diagonal ellipse
against the tiles its axis crosses.
"""
import math

import numpy as np
import pytest

from tile_differentiable_rasterizer_amd import scenes


def _q(A, B, C, x, y):
    return A * x * x + 2 * B * x * y + C * y * y


def test_box_min_matches_dense_sampling(orc):
    rng = np.random.default_rng(11)
    for _ in range(300):
        th = rng.uniform(0, math.pi)
        l1, l2 = np.exp(rng.uniform(-4, 2, 2))
        R = np.array([[math.cos(th), -math.sin(th)], [math.sin(th), math.cos(th)]])
        M = R @ np.diag([l1, l2]) @ R.T
        A, B, C = M[0, 0], M[0, 1], M[1, 1]
        X0, Y0 = rng.uniform(-20, 20, 2)
        X1, Y1 = X0 + rng.uniform(0, 15), Y0 + rng.uniform(0, 15)
        q, (xm, ym) = orc.box_min_q(A, B, C, X0, X1, Y0, Y1)
        xs, ys = np.meshgrid(np.linspace(X0, X1, 401), np.linspace(Y0, Y1, 401))
        grid = _q(A, B, C, xs, ys).min()
        # sampled values can only be larger; the grid spacing bounds how much larger
        assert grid >= q - 1e-9 * (1 + abs(q))
        h = max(X1 - X0, Y1 - Y0) / 400
        slope = 2 * (abs(A) + abs(B) + abs(C)) * (abs(X0) + abs(X1) + abs(Y0) + abs(Y1) + 1)
        assert grid - q <= slope * h + 1e-9
        assert X0 - 1e-12 <= xm <= X1 + 1e-12 and Y0 - 1e-12 <= ym <= Y1 + 1e-12
        assert _q(A, B, C, xm, ym) == pytest.approx(q, rel=1e-12, abs=1e-12)
    assert orc.box_min_q(2.0, 0.5, 1.0, -1.0, 3.0, -2.0, 0.5)[0] == 0.0  # the box holds the centre


def test_circle_keeps_tiles_within_its_radius(orc):
    """For A = C = 1/s^2, B = 0 the box minimum is dist^2 / s^2: a tile is kept iff the
    distance from the centre to its pixel-centre box is at most s * sqrt(tau)."""
    rng = np.random.default_rng(12)
    for _ in range(400):
        s = math.exp(rng.uniform(-1, 3))
        u, v = rng.uniform(0, 200, 2)
        tau = rng.uniform(0.5, 11)
        r = s * math.sqrt(tau)
        px = np.array([max(0, math.ceil(u - r - 0.5)), math.floor(u + r - 0.5),
                       max(0, math.ceil(v - r - 0.5)), math.floor(v + r - 0.5)])
        if px[0] > px[1] or px[2] > px[3]:
            continue
        ell = np.array([u, v, 1 / s ** 2, 0.0, 1 / s ** 2, tau])
        for ty in range(px[2] // 16, px[3] // 16 + 1):
            for tx in range(px[0] // 16, px[1] // 16 + 1):
                X0, X1 = max(16 * tx, px[0]) + 0.5, min(16 * tx + 15, px[1]) + 0.5
                Y0, Y1 = max(16 * ty, px[2]) + 0.5, min(16 * ty + 15, px[3]) + 0.5
                dx = max(X0 - u, 0.0, u - X1)
                dy = max(Y0 - v, 0.0, v - Y1)
                d = math.hypot(dx, dy)
                if abs(d - r) < 1e-9 * (1 + r):
                    continue
                keep, _ = orc.tile_keeps(ell, px, tx, ty)
                assert bool(keep[0]) == (d <= r), (u, v, s, tau, tx, ty)


@pytest.mark.parametrize("name,n", [("tiny_1k_sh0_64", None), ("spheres_100k_sh3_800", 3000)])
def test_kept_tiles_hold_every_supporting_pixel(orc, name, n):
    """Brute force over pixel centres: a pixel with q <= tau always lies in a kept tile, and
    the kept tiles are a subset of the rectangle."""
    sc, cams, _ = scenes.workload(name, n)
    cam = cams[0]
    p = orc.project(sc, cam)
    ell = orc.ellipses(p["uv"], p["conic"], p["opacity"])
    vis = np.nonzero(p["n_tiles"] > 0)[0]
    dropped_some = False
    for g in vis:
        u, v, A, B, C, tau = ell[g]
        x0, x1, y0, y1 = p["pxrect"][g]
        xs, ys = np.meshgrid(np.arange(x0, x1 + 1) + 0.5, np.arange(y0, y1 + 1) + 0.5)
        inside = _q(A, B, C, xs - u, ys - v) <= tau
        need = set(zip((ys[inside] // 16).astype(int), (xs[inside] // 16).astype(int)))
        tx0, tx1, ty0, ty1 = p["trect"][g]
        kept = {(ty, tx) for ty in range(ty0, ty1 + 1) for tx in range(tx0, tx1 + 1)
                if orc.tile_keeps(ell[g], p["pxrect"][g], tx, ty)[0][0]}
        assert need <= kept, g
        assert len(kept) == p["n_tiles"][g]
        dropped_some |= len(kept) < (tx1 - tx0 + 1) * (ty1 - ty0 + 1)
    if name != "tiny_1k_sh0_64":
        assert dropped_some


def test_thin_diagonal_ellipse_keeps_the_tiles_its_axis_crosses(orc):
    """An ellipse of half-length 60 px along the diagonal and half-width 0.5 px, centred on
    a tile corner: its 8x8-tile rectangle keeps only tiles near the diagonal."""
    u = v = 64.0
    t = math.pi / 4
    R = np.array([[math.cos(t), -math.sin(t)], [math.sin(t), math.cos(t)]])
    tau = 9.0
    sig = np.diag([(60 / 3) ** 2, (0.5 / 3) ** 2])  # q = 9 at the tips and sides
    Cov = R @ sig @ R.T
    M = np.linalg.inv(Cov)
    ell = np.array([u, v, M[0, 0], M[0, 1], M[1, 1], tau])
    ex, ey = math.sqrt(tau * Cov[0, 0]), math.sqrt(tau * Cov[1, 1])
    px = np.array([math.ceil(u - ex - 0.5), math.floor(u + ex - 0.5), math.ceil(v - ey - 0.5),
                   math.floor(v + ey - 0.5)])
    kept = {(ty, tx) for ty in range(px[2] // 16, px[3] // 16 + 1) for tx in range(px[0] // 16, px[1] // 16 + 1)
            if orc.tile_keeps(ell, px, tx, ty)[0][0]}
    # the axis runs through tiles (k, k) and grazes the neighbours across the shared corners
    assert {(k, k) for k in range(1, 7)} <= kept
    assert all(abs(ty - tx) <= 1 for ty, tx in kept)
    assert (1, 6) not in kept and (6, 1) not in kept


def _brute_tiles(ell, px):
    """Tiles holding a pixel centre with q <= tau (brute force over the pixel box)."""
    u, v, A, B, C, tau = ell
    xs, ys = np.meshgrid(np.arange(px[0], px[1] + 1) + 0.5, np.arange(px[2], px[3] + 1) + 0.5)
    inside = _q(A, B, C, xs - u, ys - v) <= tau
    return set(zip((ys[inside] // 16).astype(int).tolist(), (xs[inside] // 16).astype(int).tolist()))


@pytest.mark.parametrize("half_len,angle,center", [(75.0, math.pi / 3, 96.0), (300.0, 0.4, 400.0),
                                                    (2600.0, 0.02, 2400.0)])
def test_ellipse_test_applies_to_rectangles_of_any_size(orc, half_len, angle, center):
    """The page sets no size limit on the ellipse test: a thin tilted ellipse whose rectangle
    spans 10 to 40 tile rows, or more than 255 tile columns, keeps only the tiles near its
    axis.  Every tile holding a supporting pixel centre is kept (brute force); every kept tile
    is within one tile of the axis's path, and the count is well below the rectangle's area."""
    u = v = center
    R = np.array([[math.cos(angle), -math.sin(angle)], [math.sin(angle), math.cos(angle)]])
    Cov = R @ np.diag([(half_len / 3) ** 2, (0.6 / 3) ** 2]) @ R.T
    M = np.linalg.inv(Cov)
    ell = np.array([u, v, M[0, 0], M[0, 1], M[1, 1], 9.0])
    ex, ey = math.sqrt(9.0 * Cov[0, 0]), math.sqrt(9.0 * Cov[1, 1])
    px = np.array([max(0, math.ceil(u - ex - 0.5)), math.floor(u + ex - 0.5), max(0, math.ceil(v - ey - 0.5)),
                   math.floor(v + ey - 0.5)], np.int32)
    tr = (px // 16).astype(np.int32)
    rows, cols = int(tr[3] - tr[2] + 1), int(tr[1] - tr[0] + 1)
    assert rows > 8 or cols > 255
    kept = {(ty, tx) for ty in range(tr[2], tr[3] + 1) for tx in range(tr[0], tr[1] + 1)
            if orc.tile_keeps(ell, px, tx, ty)[0][0]}
    assert _brute_tiles(ell, px) <= kept
    assert int(orc.count_kept(tr[None], px[None], ell[None])[0]) == len(kept)
    # the axis through (u, v) along (cos, sin): a kept tile's centre lies within a tile
    # diagonal plus the ellipse's half-width of it
    d = np.array([math.cos(angle), math.sin(angle)])
    for ty, tx in kept:
        cx, cy = 16 * tx + 8.0 - u, 16 * ty + 8.0 - v
        assert abs(-d[1] * cx + d[0] * cy) <= 8 * math.sqrt(2) + 1.0
    assert len(kept) < rows * cols // 2
