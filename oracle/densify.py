"""float64 oracle of densify-and-prune -- TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).

"Enabling the absolute-gradient strategy in 3D Gaussian Splatting" (jsqmd.com) s1: each
Gaussian's average view-space gradient is its accumulated gradient divided by the number of
views that saw it, from the first accumulator column, or from the second (the absolute
gradient) when that strategy is switched on (s3.3).  A Gaussian whose average exceeds the
threshold is cloned when its scale is small and split when it is large; Gaussians with too
low an opacity or an abnormal scale are pruned.  "Better Gaussian Splatting in Julia"
(lshu.cn) s3.4 and "Implementing Better Gaussian Splatting in Julia" (pwwt.cn) s4.2 describe
the same control: clone where detail is missing, split where one Gaussian covers too much,
delete what is small and contributes little.

The pages leave the geometry open; the readings taken here:
  * the average gradient is accum[col] / denom in float64; denom = 0 never densifies;
  * densify iff average > threshold; "small" scale = largest axis scale <= scale_threshold;
  * a clone is an exact copy, placed right after the original;
  * a split replaces the Gaussian by split_n children drawn from the Gaussian itself:
    child j's centre is mean + R(q / |q|) (scale * z_j) with z_j a caller-supplied standard
    normal sample, its scales are scale / split_shrink (float32 division), and its
    quaternion, opacity and SH coefficients are the parent's;
  * pruning applies to every output: it is dropped when opacity < min_opacity or, with
    max_scale > 0, when its largest scale exceeds max_scale;
  * outputs keep input order, each input's outputs contiguous (children in j order); src
    gives each output's input index.
"""
from __future__ import annotations

import numpy as np


def quat_to_rot(q) -> np.ndarray:
    """Rotation matrices [n][3][3] of quaternions (w, x, y, z) after normalisation."""
    q = np.asarray(q, np.float64)
    q = q / np.linalg.norm(q, axis=-1, keepdims=True)
    w, x, y, z = q[..., 0], q[..., 1], q[..., 2], q[..., 3]
    R = np.empty(q.shape[:-1] + (3, 3), np.float64)
    R[..., 0, 0] = 1 - 2 * (y * y + z * z)
    R[..., 0, 1] = 2 * (x * y - w * z)
    R[..., 0, 2] = 2 * (x * z + w * y)
    R[..., 1, 0] = 2 * (x * y + w * z)
    R[..., 1, 1] = 1 - 2 * (x * x + z * z)
    R[..., 1, 2] = 2 * (y * z - w * x)
    R[..., 2, 0] = 2 * (x * z - w * y)
    R[..., 2, 1] = 2 * (y * z + w * x)
    R[..., 2, 2] = 1 - 2 * (x * x + y * y)
    return R


def decide(scales, opacities, accum, denom, *, grad_threshold, use_abs, scale_threshold):
    """Per input: 0 keep as is, 1 clone, 2 split (before pruning)."""
    col = 1 if use_abs else 0
    a = np.asarray(accum, np.float64)[:, col]
    d = np.asarray(denom, np.int64)
    avg = np.zeros_like(a)
    seen = d > 0
    avg[seen] = a[seen] / d[seen].astype(np.float64)
    dens = avg > np.float64(np.float32(grad_threshold))
    smax = np.asarray(scales, np.float32).max(axis=1)
    small = smax <= np.float32(scale_threshold)
    return np.where(dens & small, 1, np.where(dens, 2, 0)).astype(np.int8)


def densify(means, scales, quats, opacities, sh, accum, denom, normals, *, grad_threshold: float,
            use_abs: bool, scale_threshold: float, split_n: int, split_shrink: float, min_opacity: float,
            max_scale: float) -> dict:
    """Densify and prune one set of Gaussians.  normals: [n][split_n][3] standard normal
    samples (only split inputs use theirs).  Returns the output arrays (float32, the centres
    of split children rounded once from float64), src (uint32) and the decision per input."""
    means = np.asarray(means, np.float32)
    scales = np.asarray(scales, np.float32)
    quats = np.asarray(quats, np.float32)
    opacities = np.asarray(opacities, np.float32)
    sh = np.asarray(sh, np.float32)
    n = means.shape[0]
    kind = decide(scales, opacities, accum, denom, grad_threshold=grad_threshold, use_abs=use_abs,
                  scale_threshold=scale_threshold)
    per = np.where(kind == 2, split_n, np.where(kind == 1, 2, 1))
    src = np.repeat(np.arange(n, dtype=np.int64), per)
    # position of each output inside its input's group: 0, 1, ... per - 1
    first = np.repeat(np.cumsum(per) - per, per)
    j = np.arange(src.shape[0], dtype=np.int64) - first
    child = kind[src] == 2

    out_means = means[src].copy()
    out_scales = scales[src].copy()
    if child.any():
        s = src[child]
        R = quat_to_rot(quats[s])
        z = np.asarray(normals, np.float64)[s, j[child]]
        offset = np.einsum("nij,nj->ni", R, scales[s].astype(np.float64) * z)
        out_means[child] = (means[s].astype(np.float64) + offset).astype(np.float32)
        out_scales[child] = scales[s] / np.float32(split_shrink)
    out_opac = opacities[src]
    keep = out_opac >= np.float32(min_opacity)
    if max_scale > 0:
        keep &= out_scales.max(axis=1) <= np.float32(max_scale)
    return dict(means=out_means[keep], scales=out_scales[keep], quats=quats[src][keep], opacities=out_opac[keep],
                sh=sh[src][keep], src=src[keep].astype(np.uint32), kind=kind,
                n_clone=int((kind == 1).sum()), n_split=int((kind == 2).sum()), n_out=int(keep.sum()))
