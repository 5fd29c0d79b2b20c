"""float64 oracle of the fused Adam step with 16-bit packed moments (and, in its second form,
16-bit packed parameters too) -- TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).

"Training 10M Gaussians in 8 GB: Spirula Studio's VRAM efficiency" (mhpq.cn), quantised
training section: the Adam moments are kept as 16-bit codes packed next to each other, in a
transposed (unit-major) layout, with one (min, max) bounds pair per 256 units; gradients stay
float32.  The update itself is Adam (Kingma and Ba): m = b1 m + (1 - b1) g,
v = b2 v + (1 - b2) g^2, theta -= lr * (m / (1 - b1^t)) / (sqrt(v / (1 - b2^t)) + eps).

Readings (the page leaves the code format and the precision open); every formula is the
defining one, written as it reads, in float64:
  * a unit is one float32 parameter; word[u] = m code | v code << 16;
  * bounds[b] = (m_lo, m_hi, v_lo, v_hi), float32, for units [256 b, 256 b + 256);
  * decode: x = lo + code (hi - lo) / 65535;
  * update: m = b1 m + (1 - b1) g, v = b2 v + (1 - b2) g^2, m_hat = m / (1 - b1^t),
    v_hat = v / (1 - b2^t), theta = theta - lr m_hat / (sqrt(v_hat) + eps); the new
    parameter is rounded once to float32;
  * encode: the block's new bounds are the float32 roundings of its min and max; code =
    rint((x - lo) / (hi - lo) * 65535) clamped to [0, 65535] (0 when hi == lo).
"""
from __future__ import annotations

import math

import numpy as np

BLOCK = 256
QMAX = 65535.0


def decode(codes, lo, hi):
    """Codes (per unit) with the bounds of their block (per unit) -> float64 values."""
    lo = np.asarray(lo, np.float64)
    hi = np.asarray(hi, np.float64)
    return lo + np.asarray(codes, np.float64) * (hi - lo) / QMAX


def encode(x, lo, hi):
    """float64 values with the float32 bounds of their blocks (per value) -> uint16 codes:
    rint((x - lo) / (hi - lo) * 65535) clamped to [0, 65535], 0 where hi == lo."""
    x = np.asarray(x, np.float64)
    lo = np.asarray(lo, np.float32).astype(np.float64)
    hi = np.asarray(hi, np.float32).astype(np.float64)
    span = hi - lo
    c = np.where(span != 0.0, np.rint((x - lo) / np.where(span != 0.0, span, 1.0) * QMAX), 0.0)
    return np.clip(c, 0.0, QMAX).astype(np.uint16)


def encode_blocks(x):
    """float64 values [U] -> (codes uint16 [U], lo float32 [nb], hi float32 [nb]) per 256-unit block."""
    x = np.asarray(x, np.float64)
    U = x.shape[0]
    nb = (U + BLOCK - 1) // BLOCK
    lo = np.empty(nb, np.float32)
    hi = np.empty(nb, np.float32)
    for b in range(nb):
        seg = x[b * BLOCK:(b + 1) * BLOCK]
        lo[b] = np.float32(seg.min())
        hi[b] = np.float32(seg.max())
    blk = np.arange(U) // BLOCK
    return encode(x, lo[blk], hi[blk]), lo, hi


def adam_q16(params, grads, state, bounds, *, lr: float, beta1: float, beta2: float, eps: float, step: int,
             full: bool = False):
    """One Adam step.  params float32 [U], grads float32 [U], state uint32 [U], bounds float32
    [nb][4].  Returns (params, state, bounds) after the step (new arrays); with ``full`` also a
    dict of the float64 moments m, v and the update of each parameter (for tolerances)."""
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
    m_hat = m / (1.0 - math.pow(float(b1), step))
    v_hat = v / (1.0 - math.pow(float(b2), step))
    upd = np.float64(np.float32(lr)) * m_hat / (np.sqrt(v_hat) + np.float64(np.float32(eps)))
    new_p = (p.astype(np.float64) - upd).astype(np.float32)
    mc, mlo, mhi = encode_blocks(m)
    vc, vlo, vhi = encode_blocks(v)
    new_w = mc.astype(np.uint32) | (vc.astype(np.uint32) << np.uint32(16))
    new_b = np.stack([mlo, mhi, vlo, vhi], axis=1).astype(np.float32)
    if full:
        return new_p, new_w, new_b, dict(m=m, v=v, update=upd)
    return new_p, new_w, new_b


# --- parameters packed too ("FPBO") ------------------------------------------------------------
# The same page packs the parameters into 16-bit words together with both moments.  Readings
# (the page gives neither the word layout nor the arithmetic):
#   * a block of 256 units is stored transposed: three planes of 256 uint16 codes, the
#     parameters' codes, then the first moments', then the second moments'; state has shape
#     [nb][3][256] and the codes past the last unit of the last block are 0;
#   * bounds[b] = (p_lo, p_hi, m_lo, m_hi, v_lo, v_hi), float32, with the encoding and decoding
#     above for all three quantities;
#   * a step decodes the parameter, takes Adam's update in float64 (no float32 rounding of the
#     parameter in between: its storage is the 16-bit code) and encodes the new parameter with
#     its block's new bounds, as the moments are; the float32 parameters a renderer reads are
#     the decoded new codes, lo + code (hi - lo) / 65535 rounded once to float32.


def fpbo_pack(params):
    """float32 params [U] -> (state uint16 [nb][3][256], bounds float32 [nb][6]): the parameters
    encoded per block, both moments zero (codes 0, bounds 0)."""
    p = np.asarray(params, np.float32).astype(np.float64)
    U = p.shape[0]
    nb = (U + BLOCK - 1) // BLOCK
    state = np.zeros((nb, 3, BLOCK), np.uint16)
    bounds = np.zeros((nb, 6), np.float32)
    codes, lo, hi = encode_blocks(p)
    pad = np.zeros(nb * BLOCK, np.uint16)
    pad[:U] = codes
    state[:, 0, :] = pad.reshape(nb, BLOCK)
    bounds[:, 0], bounds[:, 1] = lo, hi
    return state, bounds


def fpbo_decode_params(state, bounds, U: int):
    """The float32 parameters held by a packed state: lo + code (hi - lo) / 65535, rounded once."""
    st = np.asarray(state, np.uint16).reshape(-1, 3, BLOCK)
    bd = np.asarray(bounds, np.float32).reshape(-1, 6)
    blk = np.arange(U) // BLOCK
    return decode(st[:, 0, :].reshape(-1)[:U], bd[blk, 0], bd[blk, 1]).astype(np.float32)


def adam_fpbo(state, bounds, grads, *, lr: float, beta1: float, beta2: float, eps: float, step: int,
              full: bool = False):
    """One Adam step on a packed state (see fpbo_pack).  grads float32 [U].  Returns (state,
    bounds, params) after the step, params being the decoded float32 parameters; with ``full``
    also a dict of the float64 parameters, moments and updates (for tolerances)."""
    g = np.asarray(grads, np.float32).astype(np.float64)
    U = g.shape[0]
    st = np.asarray(state, np.uint16).reshape(-1, 3, BLOCK)
    bd = np.asarray(bounds, np.float32).reshape(-1, 6)
    nb = st.shape[0]
    blk = np.arange(U) // BLOCK
    theta = decode(st[:, 0, :].reshape(-1)[:U], bd[blk, 0], bd[blk, 1])
    m = decode(st[:, 1, :].reshape(-1)[:U], bd[blk, 2], bd[blk, 3])
    v = decode(st[:, 2, :].reshape(-1)[:U], bd[blk, 4], bd[blk, 5])
    b1, b2 = np.float64(np.float32(beta1)), np.float64(np.float32(beta2))
    m = b1 * m + (1.0 - b1) * g
    v = b2 * v + (1.0 - b2) * (g * g)
    m_hat = m / (1.0 - math.pow(float(b1), step))
    v_hat = v / (1.0 - math.pow(float(b2), step))
    upd = np.float64(np.float32(lr)) * m_hat / (np.sqrt(v_hat) + np.float64(np.float32(eps)))
    theta = theta - upd
    new_st = np.zeros((nb, 3, BLOCK), np.uint16)
    new_bd = np.zeros((nb, 6), np.float32)
    for plane, x in enumerate((theta, m, v)):
        codes, lo, hi = encode_blocks(x)
        pad = np.zeros(nb * BLOCK, np.uint16)
        pad[:U] = codes
        new_st[:, plane, :] = pad.reshape(nb, BLOCK)
        new_bd[:, 2 * plane], new_bd[:, 2 * plane + 1] = lo, hi
    params = fpbo_decode_params(new_st, new_bd, U)
    if full:
        return new_st, new_bd, params, dict(theta=theta, m=m, v=v, update=upd)
    return new_st, new_bd, params
