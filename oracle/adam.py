"""float64 oracle of the fused Adam step with 16-bit packed moments -- TEST INFRASTRUCTURE
ONLY (see oracle/__init__.py).

"Training 10M Gaussians in 8 GB: Spirula Studio's VRAM efficiency" (mhpq.cn), quantised
training section: the Adam moments are kept as 16-bit codes packed next to each other, in a
transposed (unit-major) layout, with one (min, max) bounds pair per 256 units; gradients stay
float32.  The update itself is Adam (Kingma and Ba): m = b1 m + (1 - b1) g,
v = b2 v + (1 - b2) g^2, theta -= lr * (m / (1 - b1^t)) / (sqrt(v / (1 - b2^t)) + eps).

Readings (the page leaves the code format and the precision open):
  * a unit is one float32 parameter; word[u] = m code | v code << 16;
  * bounds[b] = (m_lo, m_hi, v_lo, v_hi), float32, for units [256 b, 256 b + 256);
  * decode: x = lo + code * ((hi - lo) * (1 / 65535)), in float64;
  * the update runs in float64, with the bias corrections applied as the reciprocals
    1 / (1 - b^t) (b^t from the host's pow); the new parameter is rounded once to float32;
  * encode: the block's new bounds are the float32 roundings of its min and max; code =
    rint((x - lo) * (65535 / (hi - lo))) clamped to [0, 65535] (0 when hi == lo).
  Scaling by reciprocals computed once keeps the device pass to one division per unit.
"""
from __future__ import annotations

import math

import numpy as np

BLOCK = 256
QMAX = 65535.0
INV_QMAX = 1.0 / QMAX


def decode(codes, lo, hi):
    """Codes (per unit) with the bounds of their block (per unit) -> float64 values."""
    lo = np.asarray(lo, np.float64)
    hi = np.asarray(hi, np.float64)
    return lo + np.asarray(codes, np.float64) * ((hi - lo) * INV_QMAX)


def encode_blocks(x):
    """float64 values [U] -> (codes uint16 [U], lo float32 [nb], hi float32 [nb]) per 256-unit block."""
    x = np.asarray(x, np.float64)
    U = x.shape[0]
    nb = (U + BLOCK - 1) // BLOCK
    lo = np.empty(nb, np.float32)
    hi = np.empty(nb, np.float32)
    codes = np.empty(U, np.uint16)
    for b in range(nb):
        seg = x[b * BLOCK:(b + 1) * BLOCK]
        lo[b] = np.float32(seg.min())
        hi[b] = np.float32(seg.max())
        l, h = np.float64(lo[b]), np.float64(hi[b])
        if h == l:
            c = np.zeros(seg.shape[0])
        else:
            c = np.rint((seg - l) * (QMAX / (h - l)))
        codes[b * BLOCK:(b + 1) * BLOCK] = np.clip(c, 0.0, QMAX).astype(np.uint16)
    return codes, lo, hi


def adam_q16(params, grads, state, bounds, *, lr: float, beta1: float, beta2: float, eps: float, step: int):
    """One Adam step.  params float32 [U], grads float32 [U], state uint32 [U], bounds float32
    [nb][4].  Returns (params, state, bounds) after the step (new arrays)."""
    p = np.asarray(params, np.float32)
    g = np.asarray(grads, np.float32).astype(np.float64)
    w = np.asarray(state, np.uint32)
    bd = np.asarray(bounds, np.float32).reshape(-1, 4)
    U = p.shape[0]
    blk = np.arange(U) // BLOCK
    m = decode(w & 0xFFFF, bd[blk, 0], bd[blk, 1])
    v = decode(w >> 16, bd[blk, 2], bd[blk, 3])
    b1, b2 = np.float64(np.float32(beta1)), np.float64(np.float32(beta2))
    m = b1 * m + (1.0 - b1) * g
    v = b2 * v + (1.0 - b2) * (g * g)
    ib1 = 1.0 / (1.0 - math.pow(float(b1), step))
    ib2 = 1.0 / (1.0 - math.pow(float(b2), step))
    upd = np.float64(np.float32(lr)) * (m * ib1) / (np.sqrt(v * ib2) + np.float64(np.float32(eps)))
    new_p = (p.astype(np.float64) - upd).astype(np.float32)
    mc, mlo, mhi = encode_blocks(m)
    vc, vlo, vhi = encode_blocks(v)
    new_w = mc.astype(np.uint32) | (vc.astype(np.uint32) << np.uint32(16))
    new_b = np.stack([mlo, mhi, vlo, vhi], axis=1).astype(np.float32)
    return new_p, new_w, new_b
