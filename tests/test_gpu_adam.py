"""GPU parity of gs_adam_q16 against the float64 oracle (oracle/adam.py, Adam in its defining
form), through the C ABI.  Each step is chained: the oracle takes the GPU's state after the
previous step.

The kernel updates the moments in float64 along a different rounding path (it decodes with
(hi - lo) * (1/65535) and scales by precomputed reciprocals), and the parameter's step in
float32.  Derived rule:

* moments differ from the oracle's by at most DX = 16 * 2^-53 * (|lo| + |hi| + |x| + |g|)
  (|g|^2 for the second moment): a few float64 roundings of the operands;
* a block bound (the float32 rounding of the block's extreme) must equal the oracle's, or
  lie between the float32 roundings of the oracle's extreme -/+ DX; blocks where it
  differs are counted, capped, and their codes not compared;
* a code equals the oracle's, or differs by one where the oracle's scaled value
  (x - lo) / (hi - lo) * 65535 lies within 65535 DX / (hi - lo) + 1e-9 of a rounding
  boundary (k + 1/2); such units are counted and capped;
* a parameter is within one float32 spacing of the oracle's plus 1e-6 of its step
  (the float32 step's error is below 4.3 float32 ulps, 5e-7 relative).
Caps: at most max(4, 1e-6 U) ambiguous units and max(1, 1e-5 blocks) ambiguous blocks.
"""
import ctypes as C

import numpy as np
import pytest
import torch

import oracle.adam as A
from tile_differentiable_rasterizer_amd import raster

from gpu_util import say

pytestmark = pytest.mark.gpu

EPS64 = 2.0 ** -53


def grads_for(rng, U, step):
    """Gradient magnitudes over six decades with random signs; every 7th block all zero
    (its moments stay constant: equal bounds) on odd steps."""
    g = (np.exp(rng.uniform(-10, 3, U)) * rng.choice([-1.0, 1.0], U)).astype(np.float32)
    if step % 2:
        blk = np.arange(U) // 256
        g[blk % 7 == 3] = 0.0
    return g


def _block_extremes(x, U):
    nb = (U + 255) // 256
    pad = np.full(nb * 256, np.nan)
    pad[:U] = x
    pad = pad.reshape(nb, 256)
    return np.nanmin(pad, axis=1), np.nanmax(pad, axis=1), np.nanargmin(pad, axis=1), np.nanargmax(pad, axis=1)


def check_step(U, gpu, orc, prev_b, g, label):
    """gpu, orc: (params, state, bounds); orc carries the oracle's float64 moments and steps."""
    gp, gw, gb = gpu
    op, ow, ob, x = orc
    blk = np.arange(U) // 256
    g = g.astype(np.float64)
    lo_m, hi_m = prev_b[blk, 0].astype(np.float64), prev_b[blk, 1].astype(np.float64)
    lo_v, hi_v = prev_b[blk, 2].astype(np.float64), prev_b[blk, 3].astype(np.float64)
    dx = {0: 16 * EPS64 * (np.abs(lo_m) + np.abs(hi_m) + np.abs(x["m"]) + np.abs(g)),
          1: 16 * EPS64 * (np.abs(lo_v) + np.abs(hi_v) + np.abs(x["v"]) + g * g)}
    amb_units = 0
    amb_blocks = np.zeros(ob.shape[0], bool)
    for k, key in ((0, "m"), (1, "v")):
        xv = x[key]
        mn, mx, imn, imx = _block_extremes(xv, U)
        for col, ext, idx in ((2 * k, mn, imn), (2 * k + 1, mx, imx)):
            d = np.array([dx[k][b * 256 + i] for b, i in enumerate(idx)])
            lo32, hi32 = (ext - d).astype(np.float32), (ext + d).astype(np.float32)
            same = gb[:, col] == ob[:, col]
            ok = same | ((gb[:, col] >= lo32) & (gb[:, col] <= hi32))
            assert np.all(ok), f"{label}: bounds column {col}, blocks {np.nonzero(~ok)[0][:5]}"
            amb_blocks |= ~same
        sh = 16 * k
        gc = ((gw >> sh) & 0xFFFF).astype(np.int64)
        oc = ((ow >> sh) & 0xFFFF).astype(np.int64)
        lo, hi = ob[blk, 2 * k].astype(np.float64), ob[blk, 2 * k + 1].astype(np.float64)
        span = np.where(hi > lo, hi - lo, 1.0)
        scaled = (xv - lo) / span * 65535.0
        eta = 65535.0 * dx[k] / span + 1e-9
        near_half = np.abs(scaled - np.floor(scaled) - 0.5) <= eta
        cmp = ~amb_blocks[blk]
        diff = np.abs(gc - oc)
        bad = cmp & ~((diff == 0) | ((diff == 1) & near_half))
        assert not bad.any(), f"{label}: {key} codes differ at {np.nonzero(bad)[0][:5]}"
        amb_units += int((cmp & (diff == 1)).sum())
    nblocks = ob.shape[0]
    assert amb_units <= max(4, 1e-6 * U), f"{label}: {amb_units} codes decided within rounding of a boundary"
    assert amb_blocks.sum() <= max(1, 1e-5 * nblocks), f"{label}: {int(amb_blocks.sum())} ambiguous blocks"
    tol = np.spacing(np.abs(op)).astype(np.float64) + 1e-6 * np.abs(x["update"])
    err = np.abs(gp.astype(np.float64) - op.astype(np.float64))
    assert np.all(err <= tol), f"{label}: params, worst {np.max(err / tol):.3g} of the tolerance"
    return amb_units, int(amb_blocks.sum()), float(np.max(err / tol, initial=0.0))


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
        orc = A.adam_q16(p, g, w, b, step=t, full=True, **h)
        torch.cuda.synchronize()
        gp = tp.cpu().numpy()
        gw = ts.cpu().numpy().view(np.uint32)
        gb = tb.cpu().numpy()
        info = check_step(U, (gp, gw, gb), orc, b, g, f"U={U} step {t}")
        say(f"adam U={U} step {t}: ambiguous codes {info[0]}, blocks {info[1]}, worst param {info[2]:.3g} of tol")
        p, w, b = gp.copy(), gw.copy(), gb.copy()  # the next step starts from the GPU's state


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
