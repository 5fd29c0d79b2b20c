"""GPU parity of gs_densify against the float64 oracle (oracle/densify.py), through the C ABI.

Decisions, sources, scales, quaternions, opacities, SH rows and copied centres must be
bit-exact.  Children's centres are rounded once from float64 on both sides, by sums taken
in different orders, so they may differ in the last float32 bit: tolerance 1e-6 absolute +
1e-6 relative (an ulp of the centres here is at most 2.4e-7).
"""
import ctypes as C

import numpy as np
import pytest
import torch

import oracle
from tile_differentiable_rasterizer_amd import raster

from gpu_util import say

pytestmark = pytest.mark.gpu


def inputs(n, L, seed, split_n=2):
    """Seeded synthetic Gaussians and statistics with every case present: averages spread
    over decades around the threshold, a third of the Gaussians unseen or barely seen,
    scales on both sides of the clone/split boundary, some opacities below the prune level."""
    rng = np.random.default_rng(seed)
    K = (L + 1) ** 2
    means = rng.uniform(-2, 2, (n, 3)).astype(np.float32)
    scales = np.exp(rng.uniform(-5, -1, (n, 3))).astype(np.float32)
    quats = rng.normal(size=(n, 4)).astype(np.float32)
    opac = rng.uniform(0.0, 1.0, n).astype(np.float32)
    sh = rng.normal(0, 0.3, (n, K, 3)).astype(np.float32)
    denom = rng.integers(0, 8, n).astype(np.int32)
    accum = (np.exp(rng.uniform(-12, -4, (n, 2))) * np.maximum(denom, 1)[:, None]).astype(np.float32)
    normals = rng.normal(size=(n, split_n, 3)).astype(np.float32)
    return means, scales, quats, opac, sh, accum, denom, normals


def run_gpu(arrs, L, params):
    dev = torch.device("cuda")
    t = [torch.from_numpy(a).to(dev) for a in arrs]
    out = raster.densify(t[0], t[1], t[2], t[3], t[4], L, t[5], t[6], t[7], params)
    torch.cuda.synchronize()
    return {k: (v.cpu().numpy() if torch.is_tensor(v) else v) for k, v in out.items()}


def compare(arrs, L, kw, label):
    params = raster.densify_params(**kw)
    g = run_gpu(arrs, L, params)
    o = oracle.densify(*arrs, **dict(kw, use_abs=bool(kw.get("use_abs", False)),
                                     split_n=kw.get("split_n", 2), split_shrink=kw.get("split_shrink", 1.6),
                                     min_opacity=kw.get("min_opacity", 0.005), max_scale=kw.get("max_scale", 0.0)))
    say(f"{label}: n={arrs[0].shape[0]} -> {o['n_out']} (clone {o['n_clone']}, split {o['n_split']})")
    assert g["n_out"] == o["n_out"], label
    assert np.array_equal(g["src"].view(np.uint32), o["src"]), label
    for k in ("scales", "quats", "opacities", "sh"):
        assert np.array_equal(g[k], o[k]), f"{label}: {k}"
    child = o["kind"][o["src"]] == 2
    assert np.array_equal(g["means"][~child], o["means"][~child]), label
    assert np.allclose(g["means"][child], o["means"][child], rtol=1e-6, atol=1e-6), label
    return o


@pytest.mark.parametrize("L", [0, 1, 2, 3])
def test_parity_per_degree(L):
    arrs = inputs(3000 + 17 * L, L, 11 + L)
    o = compare(arrs, L, dict(grad_threshold=2e-4, scale_threshold=0.05), f"L={L}")
    assert o["n_clone"] > 0 and o["n_split"] > 0 and o["n_out"] < arrs[0].shape[0] + o["n_clone"] + o["n_split"]


@pytest.mark.parametrize("kw", [
    dict(grad_threshold=5e-4, scale_threshold=0.02, use_abs=True),
    dict(grad_threshold=1e-4, scale_threshold=0.1, split_n=3, split_shrink=2.4),
    dict(grad_threshold=2e-4, scale_threshold=0.03, split_n=4, split_shrink=3.2, max_scale=0.1, min_opacity=0.3),
])
def test_parity_parameters(kw):
    arrs = inputs(20000, 3, 23, split_n=kw.get("split_n", 2))
    compare(arrs, 3, kw, str(kw))


def test_parity_one_million():
    arrs = inputs(1_000_000, 3, 5)
    o = compare(arrs, 3, dict(grad_threshold=2e-4, scale_threshold=0.05), "1M")
    assert o["n_out"] > 900_000


def test_count_only_capacity_and_errors():
    arrs = inputs(5000, 3, 2)
    dev = torch.device("cuda")
    t = [torch.from_numpy(a).to(dev) for a in arrs]
    p = raster.densify_params(2e-4, 0.05)
    full = raster.densify(t[0], t[1], t[2], t[3], t[4], 3, t[5], t[6], t[7], p)
    m = full["n_out"]
    small = dict(means=torch.empty((m - 1, 3), device=dev), scales=torch.empty((m - 1, 3), device=dev),
                 quats=torch.empty((m - 1, 4), device=dev), opacities=torch.empty(m - 1, device=dev),
                 sh=torch.empty((m - 1, 16, 3), device=dev), src=torch.empty(m - 1, dtype=torch.int32, device=dev))
    r = raster.densify(t[0], t[1], t[2], t[3], t[4], 3, t[5], t[6], t[7], p, out=small)
    assert r["status"] == raster.GS_ERR_CAPACITY and r["n_out"] == m
    L_ = raster.lib()
    cnt = C.c_int64(0)
    ws = torch.empty(L_.gs_densify_workspace_bytes(5000), dtype=torch.uint8, device=dev)
    bad = raster.densify_params(2e-4, 0.05, split_n=5)
    args = [5000] + [x.data_ptr() for x in t[:5]] + [3] + [x.data_ptr() for x in t[5:]]
    assert L_.gs_densify(*args, C.byref(bad), None, None, None, None, None, None, 0, C.byref(cnt), ws.data_ptr(),
                         ws.numel(), None) == raster.GS_ERR_INVALID_ARG
    bad = raster.densify_params(2e-4, 0.05, split_shrink=0.0)
    assert L_.gs_densify(*args, C.byref(bad), None, None, None, None, None, None, 0, C.byref(cnt), ws.data_ptr(),
                         ws.numel(), None) == raster.GS_ERR_INVALID_ARG
    assert L_.gs_densify(*args, C.byref(p), None, None, None, None, None, None, 0, C.byref(cnt), ws.data_ptr(), 8,
                         None) == raster.GS_ERR_WORKSPACE
    torch.cuda.synchronize()


def test_empty_and_all_pruned():
    arrs = inputs(0, 3, 1)
    g = run_gpu(arrs, 3, raster.densify_params(2e-4, 0.05))
    assert g["n_out"] == 0
    arrs = list(inputs(4000, 3, 4))
    arrs[3] = np.full(4000, 0.001, np.float32)
    g = run_gpu(arrs, 3, raster.densify_params(2e-4, 0.05))
    assert g["n_out"] == 0
