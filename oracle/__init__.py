"""float64 CPU oracle for the tile Gaussian rasteriser -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, the smoke entry and the benchmark's CPU-baseline leg may import this
package.  The product path never calls it.  It loads ``liboracle.so``, built from
``gs_oracle.c`` with plain gcc (``build()``); nothing here is shared with the HIP library.

Every function lifts float32 inputs to float64 exactly and returns float64 (or integer)
NumPy arrays.  See ``gs_oracle.c`` for the definitions and the passages they follow;
densify-and-prune, the fused Adam step with 16-bit moments and the q8/q16 SH codes, plain
array logic, are NumPy in ``densify.py``, ``adam.py`` and ``qsh.py``.

Parity pins (tests/test_oracle_*.py) tie each stage to something outside the oracle:
closed forms of single and paired Gaussians, the SH addition theorem and SciPy's
spherical harmonics, brute force over every Gaussian and pixel, and finite differences
for the backward.  No function here is "parity unpinned".
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gs_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (float64, no fast-math, OpenMP)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-fno-fast-math",
               "-ffp-contract=off", "-D_DEFAULT_SOURCE", "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


class _Cam(C.Structure):
    _fields_ = [("R", C.c_double * 9), ("t", C.c_double * 3), ("fx", C.c_double),
                ("fy", C.c_double), ("cx", C.c_double), ("cy", C.c_double),
                ("near_z", C.c_double), ("width", C.c_int64), ("height", C.c_int64)]


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=True)
        _lib = C.CDLL(_LIB)
        _lib.orc_count_pairs.restype = C.c_int64
        _lib.orc_emit_pairs.restype = C.c_int64
        _lib.orc_box_min_q.restype = C.c_double
        _lib.orc_forward.restype = C.c_uint64
    return _lib


def _p(a):
    return a.ctypes.data_as(C.c_void_p) if a is not None else None


def _d(x):
    return np.ascontiguousarray(np.asarray(x, dtype=np.float32).astype(np.float64))


def camera(cam) -> _Cam:
    c = _Cam()
    R = np.asarray(cam.R, dtype=np.float32).astype(np.float64).reshape(9)
    t = np.asarray(cam.t, dtype=np.float32).astype(np.float64).reshape(3)
    for i in range(9):
        c.R[i] = R[i]
    for i in range(3):
        c.t[i] = t[i]
    c.fx, c.fy = float(np.float32(cam.fx)), float(np.float32(cam.fy))
    c.cx, c.cy = float(np.float32(cam.cx)), float(np.float32(cam.cy))
    c.near_z = float(np.float32(cam.near))
    c.width, c.height = int(cam.width), int(cam.height)
    return c


def _scene_arrays(scene):
    return (_d(scene.means), _d(scene.scales), _d(scene.quats), _d(scene.opacities),
            _d(scene.sh).reshape(scene.n, -1), int(scene.sh_degree))


def sh_basis(L: int, d) -> tuple[np.ndarray, np.ndarray]:
    """Real SH basis values and polynomial gradients at one direction."""
    lib = _load()
    K = (L + 1) ** 2
    d = np.ascontiguousarray(np.asarray(d, dtype=np.float64).reshape(3))
    Y = np.zeros(K)
    dY = np.zeros((K, 3))
    lib.orc_sh_basis(C.c_int(L), _p(d), _p(Y), _p(dY))
    return Y, dY


def project(scene, cam) -> dict:
    """Projection of every Gaussian: 2D mean, depth, 2D covariance, conic, colour, rects.

    flags marks decisions that lie within rounding of their thresholds and may go either way:
    bit 0 a depth whose float32 rounding sits on a tie, bit 1 a pixel-box edge, bit 2 a
    colour channel near 0 (the clamp), bit 3 a tile test near tau, bit 4 a 2D determinant
    within rounding of 0 (a covariance of rank one: whether the conic exists)."""
    lib = _load()
    means, scales, quats, opac, sh, L = _scene_arrays(scene)
    n = scene.n
    out = dict(uv=np.zeros((n, 2)), z=np.zeros(n), depth_bits=np.zeros(n, np.uint32),
               cov2d=np.zeros((n, 3)), conic=np.zeros((n, 3)), rgb=np.zeros((n, 3)),
               clamp=np.zeros(n, np.uint8), pxrect=np.zeros((n, 4), np.int32),
               trect=np.zeros((n, 4), np.int32), n_tiles=np.zeros(n, np.int64),
               flags=np.zeros(n, np.uint8))
    c = camera(cam)
    lib.orc_project(C.c_int64(n), _p(means), _p(scales), _p(quats), _p(opac), _p(sh), C.c_int(L),
                    C.byref(c), _p(out["uv"]), _p(out["z"]), _p(out["depth_bits"]),
                    _p(out["cov2d"]), _p(out["conic"]), _p(out["rgb"]), _p(out["clamp"]),
                    _p(out["pxrect"]), _p(out["trect"]), _p(out["n_tiles"]), _p(out["flags"]))
    out["opacity"] = opac
    return out


def records(proj: dict) -> np.ndarray:
    """(u, v, A, B, C, opacity, r, g, b) per Gaussian from an oracle projection."""
    return np.ascontiguousarray(np.concatenate(
        [proj["uv"], proj["conic"], proj["opacity"][:, None], proj["rgb"]], axis=1))


def ellipses(uv, conic, opacity):
    """Per Gaussian (u, v, A, B, C, tau): the support ellipse the tile test uses."""
    lib = _load()
    uv = np.ascontiguousarray(uv, dtype=np.float64)
    conic = np.ascontiguousarray(conic, dtype=np.float64)
    opacity = np.ascontiguousarray(opacity, dtype=np.float64)
    n = opacity.shape[0]
    ell = np.zeros((n, 6))
    lib.orc_ellipses(C.c_int64(n), _p(uv), _p(conic), _p(opacity), _p(ell))
    return ell


def box_min_q(A, B, C_, X0, X1, Y0, Y1):
    """Smallest A x^2 + 2 B x y + C y^2 over [X0, X1] x [Y0, Y1], and its minimiser."""
    lib = _load()
    xm, ym = C.c_double(), C.c_double()
    q = lib.orc_box_min_q(C.c_double(A), C.c_double(B), C.c_double(C_), C.c_double(X0), C.c_double(X1),
                          C.c_double(Y0), C.c_double(Y1), C.byref(xm), C.byref(ym))
    return q, (xm.value, ym.value)


def tile_keeps(ell, pxrect, tx: int, ty: int):
    """Ellipse test of one tile for each Gaussian: (keeps, near-threshold flag) arrays."""
    lib = _load()
    ell = np.ascontiguousarray(ell, dtype=np.float64).reshape(-1, 6)
    pxrect = np.ascontiguousarray(pxrect, dtype=np.int64).reshape(-1, 4)
    n = ell.shape[0]
    keep = np.zeros(n, np.int32)
    near = np.zeros(n, np.int32)
    lib.orc_tile_keeps_batch(C.c_int64(n), _p(ell), _p(pxrect), C.c_int64(tx), C.c_int64(ty), _p(keep), _p(near))
    return keep.astype(bool), near.astype(bool)


def count_kept(trect, pxrect, ell):
    """Tiles of each rectangle kept by the ellipse test."""
    lib = _load()
    trect = np.ascontiguousarray(trect, dtype=np.int32)
    pxrect = np.ascontiguousarray(pxrect, dtype=np.int32)
    ell = np.ascontiguousarray(ell, dtype=np.float64)
    n = trect.shape[0]
    out = np.zeros(n, np.int64)
    lib.orc_count_kept(C.c_int64(n), _p(trect), _p(pxrect), _p(ell), _p(out))
    return out


def emit_pairs(trect, n_tiles, depth_bits, tiles_x: int, pxrect=None, ell=None):
    """Pairs in id order: key = tile_id << 32 | depth bits, value = Gaussian id, for every
    tile of each rectangle that passes the ellipse test of ell (u, v, A, B, C, tau) inside
    the pixel box pxrect; every tile of the rectangle when ell is None."""
    lib = _load()
    trect = np.ascontiguousarray(trect, dtype=np.int32)
    n_tiles = np.ascontiguousarray(n_tiles, dtype=np.int64)
    depth_bits = np.ascontiguousarray(depth_bits, dtype=np.uint32)
    n = n_tiles.shape[0]
    if ell is not None:
        pxrect = np.ascontiguousarray(pxrect, dtype=np.int32)
        ell = np.ascontiguousarray(ell, dtype=np.float64)
    P = int(lib.orc_count_pairs(C.c_int64(n), _p(n_tiles)))
    keys = np.zeros(max(P, 1), np.uint64)
    vals = np.zeros(max(P, 1), np.uint32)
    got = lib.orc_emit_pairs(C.c_int64(n), _p(trect), _p(pxrect), _p(ell), _p(n_tiles), _p(depth_bits),
                             C.c_int64(tiles_x), _p(keys), _p(vals), C.c_int64(P))
    assert got == P, f"{got} tiles kept for {P} counted"
    return keys[:P], vals[:P]


def emit_projected(proj: dict, tiles_x: int):
    """emit_pairs for an oracle projection (its rectangles, pixel boxes and ellipses)."""
    ell = ellipses(proj["uv"], proj["conic"], proj["opacity"])
    return emit_pairs(proj["trect"], proj["n_tiles"], proj["depth_bits"], tiles_x, proj["pxrect"], ell)


def sort_pairs(keys, vals):
    """Sort by (key, id)."""
    lib = _load()
    keys = np.array(keys, dtype=np.uint64, copy=True)
    vals = np.array(vals, dtype=np.uint32, copy=True)
    lib.orc_sort_pairs(C.c_int64(keys.shape[0]), _p(keys), _p(vals))
    return keys, vals


def tile_ranges(keys, num_tiles: int) -> np.ndarray:
    lib = _load()
    keys = np.ascontiguousarray(keys, dtype=np.uint64)
    ranges = np.zeros((num_tiles, 2), np.int64)
    lib.orc_tile_ranges(C.c_int64(keys.shape[0]), _p(keys), C.c_int64(num_tiles), _p(ranges))
    return ranges


def render_pixels(W: int, H: int, bg, rec, vals, ranges, pix=None) -> dict:
    """Tiled compositing of the listed pixels (all when ``pix`` is None).

    Returns col (npix, 3), T, n, branches (npix, 8, 5) = (r, g, b, T, n) per branch,
    nbranch (1, 2, 4, 8, or 0 with more than three near-threshold decisions) and amb flags.
    """
    lib = _load()
    rec = np.ascontiguousarray(rec, dtype=np.float64)
    vals = np.ascontiguousarray(vals, dtype=np.uint32)
    ranges = np.ascontiguousarray(ranges, dtype=np.int64)
    bg = np.ascontiguousarray(bg, dtype=np.float64)
    if pix is None:
        npix = W * H
        pixa = None
    else:
        pixa = np.ascontiguousarray(pix, dtype=np.int64)
        npix = pixa.shape[0]
    out = dict(col=np.zeros((npix, 3)), T=np.zeros(npix), n=np.zeros(npix, np.int64),
               branches=np.zeros((npix, 8, 5)), nbranch=np.zeros(npix, np.int32),
               amb=np.zeros(npix, np.uint8))
    lib.orc_render_pixels(C.c_int64(W), C.c_int64(H), _p(bg), _p(rec), _p(vals), _p(ranges),
                          C.c_int64(npix), _p(pixa), _p(out["col"]), _p(out["T"]), _p(out["n"]),
                          _p(out["branches"]), _p(out["nbranch"]), _p(out["amb"]))
    return out


def render_brute(W: int, H: int, bg, rec, order):
    lib = _load()
    rec = np.ascontiguousarray(rec, dtype=np.float64)
    order = np.ascontiguousarray(order, dtype=np.uint32)
    bg = np.ascontiguousarray(bg, dtype=np.float64)
    image = np.zeros((3, H, W))
    T = np.zeros((H, W))
    lib.orc_render_brute(C.c_int64(W), C.c_int64(H), _p(bg), _p(rec), _p(order),
                         C.c_int64(order.shape[0]), _p(image), _p(T))
    return image, T


def num_threads() -> int:
    return int(_load().orc_num_threads())


def set_threads(n: int) -> None:
    """Thread count of the oracle's OpenMP loops from now on."""
    _load().orc_set_threads(C.c_int(int(n)))


def render_bwd(W: int, H: int, bg, rec, vals, ranges, n: int, dL_dimg, with_abs: bool = False, pix=None,
               with_err: bool = False):
    """grad_screen (n, 10): dL/d(u, v, A, B, C, opacity, r, g, b), sum_p ||dL_p/d(u, v)||.

    With ``with_abs`` also returns the per-element sum of |per-pixel terms|; with
    ``with_err`` (and with_abs) also the per-element scale of the rounding a float32 reverse
    walk carries into its terms (see orc_render_bwd): (grad, abs, err)."""
    lib = _load()
    rec = np.ascontiguousarray(rec, dtype=np.float64)
    vals = np.ascontiguousarray(vals, dtype=np.uint32)
    ranges = np.ascontiguousarray(ranges, dtype=np.int64)
    bg = np.ascontiguousarray(bg, dtype=np.float64)
    dL = np.ascontiguousarray(np.asarray(dL_dimg, dtype=np.float64).reshape(3, H, W))
    gs = np.zeros((n, 10))
    ga = np.zeros((n, 10)) if with_abs else None
    ge = np.zeros((n, 10)) if with_err else None
    pixa = None if pix is None else np.ascontiguousarray(pix, dtype=np.int64)
    lib.orc_render_bwd(C.c_int64(W), C.c_int64(H), _p(bg), _p(rec), _p(vals), _p(ranges),
                       C.c_int64(n), _p(dL), _p(gs), _p(ga), _p(ge),
                       C.c_int64(0 if pixa is None else pixa.shape[0]), _p(pixa))
    if with_err:
        return gs, ga, ge
    return (gs, ga) if with_abs else gs


def project_bwd(scene, cam, grad_screen, accum=None, denom=None) -> dict:
    """Chain rule to means, scales, quaternions, opacity and SH; densification stats."""
    lib = _load()
    means, scales, quats, opac, sh, L = _scene_arrays(scene)
    n = scene.n
    K = (L + 1) ** 2
    gs = np.ascontiguousarray(grad_screen, dtype=np.float64).reshape(n, 10)
    out = dict(dmeans=np.zeros((n, 3)), dscales=np.zeros((n, 3)), dquats=np.zeros((n, 4)),
               dopacity=np.zeros(n), dsh=np.zeros((n, K, 3)),
               accum=np.zeros((n, 2)) if accum is None else np.array(accum, np.float64),
               denom=np.zeros(n, np.int64) if denom is None else np.array(denom, np.int64))
    c = camera(cam)
    lib.orc_project_bwd(C.c_int64(n), _p(means), _p(scales), _p(quats), _p(opac), _p(sh),
                        C.c_int(L), C.byref(c), _p(gs), _p(out["dmeans"]), _p(out["dscales"]),
                        _p(out["dquats"]), _p(out["dopacity"]), _p(out["dsh"]), _p(out["accum"]),
                        _p(out["denom"]))
    return out


def forward(scene, cam, bg=(0.0, 0.0, 0.0)):
    """Whole forward from raw parameters; returns (image[3][H][W], T, n_contrib, hash)."""
    lib = _load()
    means, scales, quats, opac, sh, L = _scene_arrays(scene)
    return forward_raw(means, scales, quats, opac, sh, L, cam, bg)


def forward_raw(means, scales, quats, opac, sh, L, cam, bg=(0.0, 0.0, 0.0)):
    """``forward`` on float64 parameter arrays (used by finite differences)."""
    lib = _load()
    W, H = int(cam.width), int(cam.height)
    c = cam if isinstance(cam, _Cam) else camera(cam)
    image = np.zeros((3, H, W))
    T = np.zeros((H, W))
    ncon = np.zeros((H, W), np.int64)
    bgv = np.ascontiguousarray(bg, dtype=np.float64)
    arrs = [np.ascontiguousarray(a, dtype=np.float64) for a in (means, scales, quats, opac, sh)]
    h = lib.orc_forward(C.c_int64(arrs[0].shape[0]), *[_p(a) for a in arrs], C.c_int(L), C.byref(c),
                        _p(bgv), _p(image), _p(T), _p(ncon))
    return image, T, ncon, int(h)


def end_to_end(scene, cam, bg=(0.0, 0.0, 0.0), pix=None) -> dict:
    """Project, bin, sort and composite from raw parameters; keeps every stage's output."""
    proj = project(scene, cam)
    keys, vals = emit_projected(proj, cam.tiles_x)
    skeys, svals = sort_pairs(keys, vals)
    ranges = tile_ranges(skeys, cam.num_tiles)
    rec = records(proj)
    pixr = render_pixels(cam.width, cam.height, bg, rec, svals, ranges, pix)
    return dict(proj=proj, keys=keys, vals=vals, skeys=skeys, svals=svals, ranges=ranges,
                rec=rec, render=pixr)


def cov3d(scale, quat) -> np.ndarray:
    """3D covariance of one Gaussian (3x3)."""
    lib = _load()
    s = np.ascontiguousarray(np.asarray(scale, dtype=np.float64).reshape(3))
    q = np.ascontiguousarray(np.asarray(quat, dtype=np.float64).reshape(4))
    out = np.zeros(9)
    lib.orc_cov3d(_p(s), _p(q), _p(out))
    return out.reshape(3, 3)


from .adam import adam_q16  # noqa: E402,F401
from .densify import densify, quat_to_rot  # noqa: E402,F401
