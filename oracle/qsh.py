"""Quantised SH coefficients (q8 / q16) -- TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).

"Training 10M Gaussians in 8 GB: Spirula Studio's VRAM efficiency" (mhpq.cn), quantised
training section: SH coefficients are stored as 8- or 16-bit fixed-point codes with a
(min, max) bounds table for decoding, one bounds pair per 256 units.

Readings (the page leaves the code arithmetic open):
  * units are the coefficients in their [n][K][3] order; block b holds units [256 b, 256 b + 256);
  * bounds[b] = (min, max) of the block's float32 values;
  * code = rint((x - lo) * (qmax / (hi - lo))) in float64, clamped to [0, qmax]
    (0 when hi == lo), qmax = 2^bits - 1;
  * decode, in float32 with each operation rounded: lo + code * ((hi - lo) * (1 / qmax)).
The projection of quantised SH is the float32 projection of the decoded coefficients.
"""
from __future__ import annotations

import numpy as np

BLOCK = 256


def qmax(bits: int) -> int:
    assert bits in (8, 16)
    return (1 << bits) - 1


def quantize(values, bits: int):
    """float32 values (any shape; flattened in C order) -> (codes uint8/uint16 of that shape,
    bounds float32 [nb][2])."""
    x = np.asarray(values, np.float32)
    flat = x.reshape(-1)
    U = flat.shape[0]
    nb = (U + BLOCK - 1) // BLOCK
    q = float(qmax(bits))
    codes = np.empty(U, np.uint16 if bits == 16 else np.uint8)
    bounds = np.empty((nb, 2), np.float32)
    for b in range(nb):
        seg = flat[b * BLOCK:(b + 1) * BLOCK]
        lo, hi = seg.min(), seg.max()
        bounds[b] = (lo, hi)
        if hi == lo:
            c = np.zeros(seg.shape[0])
        else:
            c = np.rint((seg.astype(np.float64) - np.float64(lo)) * (q / (np.float64(hi) - np.float64(lo))))
        codes[b * BLOCK:(b + 1) * BLOCK] = np.clip(c, 0.0, q).astype(codes.dtype)
    return codes.reshape(x.shape), bounds


def dequantize(codes, bounds, bits: int):
    """Codes (any shape) and their block bounds -> float32 values of that shape."""
    c = np.asarray(codes)
    flat = c.reshape(-1)
    blk = np.arange(flat.shape[0]) // BLOCK
    bd = np.asarray(bounds, np.float32).reshape(-1, 2)
    lo, hi = bd[blk, 0], bd[blk, 1]
    step = (hi - lo) * np.float32(1.0 / qmax(bits))  # float32 operations, each rounded
    return (lo + flat.astype(np.float32) * step).astype(np.float32).reshape(c.shape)
