"""Pins for the oracle's densify-and-prune.

"Enabling the absolute-gradient strategy in 3D Gaussian Splatting" (jsqmd.com) s1, s3.3:
average gradient = accumulated gradient / views, column 1 with the absolute-gradient
strategy; above the threshold, clone small Gaussians and split large ones; prune low
opacity or abnormal scale.  The expected outputs below are worked by hand; the split
geometry is checked against SciPy's rotations and against the sample covariance of many
children.
"""
import numpy as np
from scipy.spatial.transform import Rotation

import oracle

P = dict(grad_threshold=0.5, use_abs=False, scale_threshold=0.1, split_n=2, split_shrink=1.6, min_opacity=0.05,
         max_scale=0.0)


def _five():
    """Five Gaussians, one per case (values chosen so every decision is far from its edge)."""
    means = np.array([[0, 0, 1], [1, 0, 1], [2, 0, 1], [3, 0, 1], [4, 0, 1]], np.float32)
    scales = np.array([[0.05, 0.05, 0.05],   # small
                       [0.05, 0.02, 0.01],   # small
                       [0.2, 0.1, 0.1],      # large
                       [0.05, 0.05, 0.05],
                       [0.3, 0.3, 0.3]], np.float32)
    quats = np.tile(np.array([1, 0, 0, 0], np.float32), (5, 1))
    opac = np.array([0.9, 0.8, 0.7, 0.01, 0.6], np.float32)
    sh = np.arange(5 * 4 * 3, dtype=np.float32).reshape(5, 4, 3)
    # averages (col 0): 0.2 below, 1.0 above (clone), 2.0 above (split), 3.0 above but pruned,
    # and no views at all (denom 0) for the last one
    accum = np.array([[0.4, 9.0], [2.0, 0.0], [6.0, 0.0], [3.0, 0.0], [5.0, 0.0]], np.float32)
    denom = np.array([2, 2, 3, 1, 0], np.int32)
    z = np.zeros((5, 2, 3), np.float32)
    z[2, 0] = (1.0, 0.0, 0.0)
    z[2, 1] = (0.0, -1.0, 2.0)
    return means, scales, quats, opac, sh, accum, denom, z


def test_each_case_by_hand():
    means, scales, quats, opac, sh, accum, denom, z = _five()
    out = oracle.densify(means, scales, quats, opac, sh, accum, denom, z, **P)
    # 0 kept; 1 cloned (2 rows); 2 split (2 children); 3 cloned but pruned (opacity 0.01); 4 kept
    assert list(out["kind"]) == [0, 1, 2, 1, 0]
    assert list(out["src"]) == [0, 1, 1, 2, 2, 4]
    assert out["n_out"] == 6 and out["n_clone"] == 2 and out["n_split"] == 1
    # the kept Gaussian and the clones are exact copies of their inputs
    inputs = dict(means=means, scales=scales, quats=quats, opacities=opac, sh=sh)
    for k, a in inputs.items():
        assert np.array_equal(out[k][0], a[0])
        assert np.array_equal(out[k][1], a[1]) and np.array_equal(out[k][2], a[1])
        assert np.array_equal(out[k][5], a[4])
    # children of Gaussian 2 (identity rotation): centre + scale * z, scales / 1.6
    assert np.allclose(out["means"][3], [2 + 0.2, 0, 1], atol=1e-7)
    assert np.allclose(out["means"][4], [2, -0.1, 1 + 0.2], atol=1e-7)
    assert np.array_equal(out["scales"][3], np.float32([0.2, 0.1, 0.1]) / np.float32(1.6))
    assert np.array_equal(out["sh"][3], sh[2]) and np.array_equal(out["sh"][4], sh[2])
    assert out["opacities"][3] == np.float32(0.7)


def test_absolute_gradient_column():
    means, scales, quats, opac, sh, accum, denom, z = _five()
    # column 1: only Gaussian 0 (9 / 2 = 4.5) is above the threshold, and it is small
    out = oracle.densify(means, scales, quats, opac, sh, accum, denom, z, **dict(P, use_abs=True))
    assert list(out["kind"]) == [1, 0, 0, 0, 0]
    assert list(out["src"]) == [0, 0, 1, 2, 4]


def test_threshold_is_strict_and_max_scale_prunes():
    means, scales, quats, opac, sh, accum, denom, z = _five()
    accum = accum.copy()
    accum[1, 0] = 1.0  # average exactly 0.5: not above
    out = oracle.densify(means, scales, quats, opac, sh, accum, denom, z, **dict(P, max_scale=0.2))
    assert out["kind"][1] == 0
    # max scale 0.2: Gaussian 4 (0.3) is pruned; Gaussian 2's children (0.125) stay
    assert list(out["src"]) == [0, 1, 2, 2]


def test_split_offsets_match_scipy_rotation():
    rng = np.random.default_rng(3)
    n = 50
    q = rng.normal(size=(n, 4)).astype(np.float32)
    s = np.exp(rng.uniform(-2, 0, (n, 3))).astype(np.float32)
    mu = rng.normal(size=(n, 3)).astype(np.float32)
    z = rng.normal(size=(n, 3, 3)).astype(np.float32)
    out = oracle.densify(mu, s, q, np.full(n, 0.5, np.float32), np.zeros((n, 1, 3), np.float32),
                         np.full((n, 2), 10.0, np.float32), np.ones(n, np.int32), z,
                         **dict(P, split_n=3, scale_threshold=0.0))
    assert out["n_split"] == n and out["n_out"] == 3 * n
    R = Rotation.from_quat(q[:, [1, 2, 3, 0]].astype(np.float64)).as_matrix()  # SciPy takes (x, y, z, w)
    for i in range(n):
        for j in range(3):
            want = mu[i].astype(np.float64) + R[i] @ (s[i].astype(np.float64) * z[i, j].astype(np.float64))
            assert np.allclose(out["means"][3 * i + j], want, rtol=0, atol=1e-6)


def test_children_follow_the_parent_distribution():
    """Many children of one Gaussian: their sample covariance is R diag(s^2) R^T."""
    rng = np.random.default_rng(8)
    m = 20000
    q = np.array([[0.8, 0.3, -0.4, 0.2]], np.float32)
    s = np.array([[0.5, 0.2, 0.05]], np.float32)
    z = rng.normal(size=(1, m, 3)).astype(np.float32)
    out = oracle.densify(np.zeros((1, 3), np.float32), s, q, np.ones(1, np.float32), np.zeros((1, 1, 3), np.float32),
                         np.ones((1, 2), np.float32), np.ones(1, np.int32), z, **dict(P, split_n=m, scale_threshold=0.0))
    R = Rotation.from_quat(q[0, [1, 2, 3, 0]].astype(np.float64)).as_matrix()
    sigma = R @ np.diag(s[0].astype(np.float64) ** 2) @ R.T
    emp = np.cov(out["means"].astype(np.float64).T)
    # sampling error of 20000 draws is ~1% of the largest entry; a transposed rotation
    # would be off by ~100%
    assert np.abs(emp - sigma).max() < 0.04 * sigma.max()


def test_empty_and_all_pruned():
    e = np.zeros((0, 3), np.float32)
    out = oracle.densify(e, e, np.zeros((0, 4), np.float32), np.zeros(0, np.float32), np.zeros((0, 1, 3), np.float32),
                         np.zeros((0, 2), np.float32), np.zeros(0, np.int32), np.zeros((0, 2, 3), np.float32), **P)
    assert out["n_out"] == 0 and out["src"].shape == (0,)
    means, scales, quats, opac, sh, accum, denom, z = _five()
    out = oracle.densify(means, scales, quats, np.full(5, 0.01, np.float32), sh, accum, denom, z, **P)
    assert out["n_out"] == 0
