"""Pins for the oracle's quantised SH (q8 / q16, bounds per 256 units).

"Training 10M Gaussians in 8 GB: Spirula Studio's VRAM efficiency" (mhpq.cn), quantised
training section.  Checked by hand at the code endpoints and a midpoint, by the half-step
error bound, and by the colour bound sum_k |Y_k| step_k / 2 after projection.
"""
import numpy as np

import oracle
import oracle.qsh as Q
from tile_differentiable_rasterizer_amd import scenes


def test_endpoints_and_midpoint():
    x = np.array([0.0, 1.0, 0.5, 0.25], np.float32)
    c8, b8 = Q.quantize(x, 8)
    # rint(0.5 * 255) = rint(127.5) = 128 (ties to even); rint(63.75) = 64
    assert list(c8) == [0, 255, 128, 64] and tuple(b8[0]) == (0.0, 1.0)
    c16, b16 = Q.quantize(x, 16)
    assert list(c16) == [0, 65535, 32768, 16384]
    d8 = Q.dequantize(c8, b8, 8)
    assert d8[0] == 0.0 and abs(d8[1] - 1.0) < 1e-6 and abs(d8[2] - 128 / 255) < 1e-7
    # a constant block stores code 0 and decodes exactly
    c, b = Q.quantize(np.full(300, -0.75, np.float32), 16)
    assert np.all(c == 0) and np.all(Q.dequantize(c, b, 16) == np.float32(-0.75))


def test_error_within_half_a_step():
    rng = np.random.default_rng(4)
    x = (rng.normal(size=(1000, 16, 3)) * np.exp(rng.uniform(-4, 1, (1000, 1, 1)))).astype(np.float32)
    for bits in (8, 16):
        c, b = Q.quantize(x, bits)
        d = Q.dequantize(c, b, bits)
        flat = x.reshape(-1)
        blk = np.arange(flat.size) // 256
        step = (b[blk, 1].astype(np.float64) - b[blk, 0]) / Q.qmax(bits)
        err = np.abs(d.reshape(-1).astype(np.float64) - flat)
        # half a code step, plus the float32 rounding of the decode: its step carries ~3
        # roundings (x code <= qmax) and its last addition rounds at the bounds' magnitude
        mag = np.maximum(np.abs(b[blk, 0]), np.abs(b[blk, 1]))
        assert np.all(err <= 0.5 * step * (1 + 1e-3) + 2 * np.spacing(mag)), bits
        # the block extremes are exact codes
        assert np.all(c.reshape(-1)[np.argmin(flat[:256])] == 0)


def test_projected_colour_within_the_quantisation_bound():
    sc, cams, _ = scenes.workload("spheres_100k_sh3_800", 5000)
    cam = cams[0]
    for bits in (8, 16):
        c, b = Q.quantize(sc.sh, bits)
        sq = scenes.Scene(sc.means, sc.scales, sc.quats, sc.opacities, Q.dequantize(c, b, bits), sc.sh_degree)
        p0 = oracle.project(sc, cam)
        p1 = oracle.project(sq, cam)
        vis = p0["n_tiles"] > 0
        # |d colour| <= sum_k |Y_k(d)| * |d coefficient_k| (the clamp at 0 only shrinks it),
        # d the unit direction from the camera centre -R^T t to the mean
        campos = -cam.R.astype(np.float64).T @ cam.t.astype(np.float64)
        v = sc.means[vis].astype(np.float64) - campos
        dirs = v / np.linalg.norm(v, axis=1, keepdims=True)
        Y = np.stack([oracle.sh_basis(3, d)[0] for d in dirs])
        dc = np.abs(sq.sh.astype(np.float64) - sc.sh)[vis]  # [v][16][3]
        bound = np.einsum("vk,vkc->vc", np.abs(Y), dc)
        diff = np.abs(p1["rgb"][vis] - p0["rgb"][vis])
        assert np.all(diff <= bound + 1e-9), bits
        assert diff.max() > 0  # quantisation did change something
