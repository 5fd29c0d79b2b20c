"""GPU parity of gs_adam_q16 against the float64 oracle (oracle/adam.py), through the C ABI.

Parameters, packed moment codes and block bounds must be bit-exact after every step: both
sides evaluate the definition in float64 in the same order, decide the codes in float64 and
round the parameters once.
"""
import ctypes as C

import numpy as np
import pytest
import torch

import oracle.adam as A
from tile_differentiable_rasterizer_amd import raster

from gpu_util import say

pytestmark = pytest.mark.gpu


def grads_for(rng, U, step):
    """Gradient magnitudes over six decades with random signs; every 7th block all zero
    (its moments stay constant: equal bounds) on odd steps."""
    g = (np.exp(rng.uniform(-10, 3, U)) * rng.choice([-1.0, 1.0], U)).astype(np.float32)
    if step % 2:
        blk = np.arange(U) // 256
        g[blk % 7 == 3] = 0.0
    return g


def run(U, steps, seed, **hyper):
    rng = np.random.default_rng(seed)
    dev = torch.device("cuda")
    p = rng.normal(size=U).astype(np.float32)
    nb = (U + 255) // 256
    w = np.zeros(U, np.uint32)
    b = np.zeros((nb, 4), np.float32)
    tp = torch.from_numpy(p.copy()).to(dev)
    ts, tb = raster.adam_state(U, dev)
    h = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8)
    h.update(hyper)
    for t in range(1, steps + 1):
        g = grads_for(rng, U, t)
        raster.adam_q16(tp, torch.from_numpy(g).to(dev), ts, tb, step=t, **h)
        p, w, b = A.adam_q16(p, g, w, b, step=t, **h)
        torch.cuda.synchronize()
        gp = tp.cpu().numpy()
        gw = ts.cpu().numpy().view(np.uint32)
        gb = tb.cpu().numpy()
        assert np.array_equal(gb, b), f"U={U} step {t}: bounds"
        assert np.array_equal(gw, w), f"U={U} step {t}: codes ({int((gw != w).sum())} differ)"
        assert np.array_equal(gp, p), f"U={U} step {t}: params ({int((gp != p).sum())} differ)"
    say(f"adam U={U}: {steps} steps bit-exact")


@pytest.mark.parametrize("U", [1, 255, 256, 257, 100_003])
def test_parity_steps(U):
    run(U, 4, 40 + U % 97)


def test_parity_hyperparameters():
    run(50_000, 3, 7, lr=0.05, beta1=0.5, beta2=0.9, eps=1e-4)
    run(50_000, 3, 8, lr=1e-4, beta1=0.0, beta2=0.0, eps=1e-12)


def test_parity_ten_million_units():
    run(10_000_000, 2, 9)


def test_empty_and_errors():
    dev = torch.device("cuda")
    e = torch.zeros(0, device=dev)
    raster.adam_q16(e, e, torch.zeros(0, dtype=torch.int32, device=dev), torch.zeros((0, 4), device=dev), lr=1e-3,
                    step=1)
    L = raster.lib()
    p = torch.zeros(10, device=dev)
    s, b = raster.adam_state(10, dev)
    for h in (raster.GsAdamParams(1e-3, 0.9, 0.999, 1e-8, 0), raster.GsAdamParams(1e-3, 1.0, 0.999, 1e-8, 1),
              raster.GsAdamParams(1e-3, 0.9, -0.5, 1e-8, 1)):
        assert L.gs_adam_q16(10, p.data_ptr(), p.data_ptr(), s.data_ptr(), b.data_ptr(), C.byref(h),
                             None) == raster.GS_ERR_INVALID_ARG
    h = raster.GsAdamParams(1e-3, 0.9, 0.999, 1e-8, 1)
    assert L.gs_adam_q16(10, None, p.data_ptr(), s.data_ptr(), b.data_ptr(), C.byref(h), None) == \
        raster.GS_ERR_INVALID_ARG
    torch.cuda.synchronize()
