"""Helpers for the GPU parity tests: run each C-ABI stage, bring results to the host, and
compare them with the float64 oracle under the acceptance rules:

* projection: same visibility, tile rect, pixel box, tile count and depth bits; 2D mean
  within 1e-4 px, or half a float32 spacing of the coordinate where that is coarser (the
  kernel rounds a float64 value once; beyond 2048 px half a spacing exceeds 1e-4); conic
  within 1e-5 relative, colour within 1e-5 (absolute or relative to 1).  A Gaussian whose
  pixel-box edge (flag 2) or tile-test decision (flag 8) lies within rounding of its
  threshold is exempt from the comparisons that decision feeds (visibility, tile count; the
  rect and pixel box for flag 2) and from nothing else; such Gaussians may number at most
  FLAG_CAP of the tile decisions made (the tiles of the visible Gaussians' rectangles);
* binning and sorting: bit-exact keys, ids and tile ranges;
* compositing: every channel and the final transmittance within 1e-4 of some result that a
  correct evaluation of the thresholds can give (the oracle enumerates the two sides of any
  decision that float32 rounding could flip, up to three per pixel), and the same
  contributor count; pixels with more than three such decisions are excluded and may be
  at most 1e-5 of those compared;
* gradients: |g - g_ref| <= max(1e-3 |g_ref|, 1e-5, 16 * 2^-24 * S + 4 * 2^-24 * E), where S is the sum of
  the absolute per-pixel terms that make up the element and E the oracle's rounding scale
  of the float32 reverse walk (both reported by the oracle).  The last term is float32's
  own floor for a sum whose terms cancel: each per-pixel term carries a few roundings, the
  walk's transmittance and colour behind carry one or two per contributor into the parts
  of dL/dalpha (which may cancel too), and the sum adds a few more, so a correct float32
  result can be off by that much even when |g_ref| << S.  Elements
  that pass only through that term are reported with their conditioning
  kappa = S / |g_ref|; each must have kappa >= 1e2 (a summation limit, not a wrong term),
  and there may be at most max(4, 1e-6 * elements) of them.

Each oracle stage consumes the previous GPU stage's output lifted exactly to float64, so a
mismatch names the stage that caused it.
"""
from __future__ import annotations

import math

import numpy as np
import torch

import oracle
from tile_differentiable_rasterizer_amd import raster

PIX_TOL = 1e-4
GRAD_REL, GRAD_ABS = 1e-3, 1e-5
FLAG_CAP = 1e-4        # flagged (near-threshold) Gaussians, per tile decision of the visible ones
EXCLUDED_CAP = 1e-5    # pixels with more than three near-threshold decisions, fraction
COND_KAPPA_MIN = 1e2   # conditioning of a gradient element passing through the float32 floor only
COND_CAP = 1e-6        # such elements, fraction of all elements (at least 4 allowed)


def say(msg: str):
    print(msg, flush=True)


def to_np(t):
    return t.detach().cpu().numpy()


def gpu_stages(scene, cam, bg=(0.0, 0.0, 0.0), keep_unsorted=True, digit_counts=True):
    """Run project, bin, sort, render through the C ABI; return host copies.  With
    digit_counts the sort takes the binning's tile-digit counts (the Rasterizer's path);
    without, it counts the digits itself."""
    dev = torch.device("cuda")
    means, scales, quats, opac, sh = raster.scene_to_device(scene, dev)
    n = scene.n
    tiles = cam.tiles_x * cam.tiles_y
    proj = raster.project(means, scales, quats, opac, sh, scene.sh_degree, cam)
    ws = torch.empty(max(raster.workspace_bytes(n, 1, tiles), 8), dtype=torch.uint8, device=dev)
    st, P = raster.bin_tiles(proj, cam, None, None, ws)
    assert st == raster.GS_OK
    keys = torch.empty(max(P, 1), dtype=torch.int64, device=dev)
    vals = torch.empty(max(P, 1), dtype=torch.int32, device=dev)
    ws = torch.empty(raster.workspace_bytes(n, P, tiles), dtype=torch.uint8, device=dev)
    dc = torch.full((raster.TILE_DIGIT_COUNTS,), -1, dtype=torch.int64, device=dev) if digit_counts else None
    st, P2 = raster.bin_tiles(proj, cam, keys, vals, ws, digit_counts=dc)
    assert st == raster.GS_OK and P2 == P
    torch.cuda.synchronize()
    out = dict(P=P, n=n)
    if digit_counts:
        out["digit_counts"] = to_np(dc).view(np.uint64).reshape(2, 256).copy()
    if keep_unsorted:
        out["keys_unsorted"] = to_np(keys[:P]).view(np.uint64).copy()
        out["vals_unsorted"] = to_np(vals[:P]).view(np.uint32).copy()
    ktmp = torch.empty_like(keys)
    vtmp = torch.empty_like(vals)
    ranges = torch.empty((tiles, 2), dtype=torch.int64, device=dev)
    order = torch.empty(tiles, dtype=torch.int32, device=dev)
    raster.sort_keys(P, tiles, keys, vals, ktmp, vtmp, ranges, ws, order, digit_counts=dc)
    image = torch.empty((3, cam.height, cam.width), dtype=torch.float32, device=dev)
    final_T = torch.empty((cam.height, cam.width), dtype=torch.float32, device=dev)
    n_contrib = torch.empty((cam.height, cam.width), dtype=torch.int32, device=dev)
    raster.render_fwd(proj, vals, ranges, cam, bg, image, final_T, n_contrib, order)
    torch.cuda.synchronize()
    rec = to_np(proj["rec"])
    out.update(
        rec=rec, bbox=rec[:, 9:11].view(np.uint32), depth_bits=to_np(proj["depth"]).view(np.uint32),
        rect=to_np(proj["rect"]).view(np.uint16).astype(np.int32), n_tiles=to_np(proj["n_tiles"]).view(np.uint32),
        clamp=to_np(proj["clamp"]), keys=to_np(keys[:P]).view(np.uint64).copy(),
        vals=to_np(vals[:P]).view(np.uint32).copy(), ranges=to_np(ranges), order=to_np(order), image=to_np(image),
        final_T=to_np(final_T), n_contrib=to_np(n_contrib).view(np.uint32),
        dev=dict(means=means, scales=scales, quats=quats, opac=opac, sh=sh, proj=proj, vals=vals, ranges=ranges, order=order,
                 final_T=final_T, n_contrib=n_contrib, image=image))
    return out


def rec9(g) -> np.ndarray:
    """The GPU's render records as the oracle's (u, v, A, B, C, o, r, g, b), exact in f64."""
    return np.ascontiguousarray(g["rec"][:, :9].astype(np.float64))


def uv_tolerance(uv):
    """1e-4 px, or half a float32 spacing of the coordinate (plus float64 noise) where that
    is coarser: the kernel evaluates the 2D mean in float64 and rounds it once."""
    a = np.abs(uv)
    half = 0.5 * np.spacing(a.astype(np.float32)).astype(np.float64)
    return np.maximum(PIX_TOL, half + 1e-12 * (1.0 + a))


def check_projection(scene, cam, g, label="", flag_cap=FLAG_CAP):
    p = oracle.project(scene, cam)
    flags = p["flags"]
    vis_o = p["n_tiles"] > 0
    vis_g = g["n_tiles"] > 0
    # decisions the oracle flags as within float64 / float32 rounding of their thresholds:
    # a pixel-box edge (bit 1), a tile test (bit 3) and the sign of a determinant within
    # rounding of 0 (bit 4: whether a conic exists) may go either way
    edge = (flags & 2) != 0
    degenerate = (flags & 16) != 0
    amb = edge | ((flags & 8) != 0) | degenerate
    bad_vis = np.nonzero((vis_o != vis_g) & ~amb)[0]
    assert bad_vis.size == 0, f"{label}: visibility differs for ids {bad_vis[:10]}"
    nvis = int(vis_o.sum())
    either = vis_o | vis_g
    namb = int((amb & either).sum())
    tr = p["trect"][either].astype(np.int64)
    decisions = int(((tr[:, 1] - tr[:, 0] + 1) * (tr[:, 3] - tr[:, 2] + 1)).sum())
    assert namb <= max(2, flag_cap * decisions), \
        f"{label}: {namb} of {nvis} visible Gaussians near a threshold ({decisions} tile decisions)"
    both = vis_o & vis_g
    sure = both & ~amb
    assert np.array_equal(g["n_tiles"][sure], p["n_tiles"][sure].astype(np.uint32)), f"{label}: tile counts"
    box = both & ~edge
    assert np.array_equal(g["rect"][box], p["trect"][box]), f"{label}: tile rect"
    bx, by = g["bbox"][box, 0], g["bbox"][box, 1]
    gpx = np.stack([bx & 0xFFFF, bx >> 16, by & 0xFFFF, by >> 16], 1).astype(np.int32)
    assert np.array_equal(gpx, p["pxrect"][box]), f"{label}: pixel box differs"
    tie = (flags & 1) != 0
    vis_d = both & ~tie
    assert np.array_equal(g["depth_bits"][vis_d], p["depth_bits"][vis_d]), f"{label}: depth bits differ"
    r = g["rec"][both][:, :9].astype(np.float64)  # the float words (9 and 10 hold the pixel box bits)
    uv = p["uv"][both]
    err_uv = np.abs(r[:, 0:2] - uv)
    assert np.all(err_uv <= uv_tolerance(uv)), f"{label}: 2D mean, worst {np.max(err_uv, initial=0)} px"
    # the conic divides by the determinant: compared where that is not rounding noise
    cdef = ~degenerate[both]
    cn = p["conic"][both][cdef]
    scale = np.abs(cn[:, 0]) + np.abs(cn[:, 2])
    err = np.abs(r[cdef, 2:5] - cn) / scale[:, None]
    assert np.max(err, initial=0) <= 1e-5, f"{label}: conic rel err {np.max(err, initial=0)}"
    assert np.array_equal(r[:, 5], p["opacity"][both]), f"{label}: opacity"
    cerr = np.abs(r[:, 6:9] - p["rgb"][both]) / np.maximum(1.0, np.abs(p["rgb"][both]))
    assert np.max(cerr, initial=0) <= 1e-5, f"{label}: colour err {np.max(cerr, initial=0)}"
    csure = both & ((flags & 4) == 0)
    assert np.array_equal(g["clamp"][csure], p["clamp"][csure]), f"{label}: clamp bits"
    g["oracle_proj"] = p  # for end-to-end checks that need the oracle's flags
    return dict(visible=nvis, near_threshold=namb, ties=int(tie.sum()))


def gpu_ellipses(g):
    """The oracle's tile-test ellipses (u, v, A, B, C, tau) of the GPU's records, exact in f64."""
    r = g["rec"][:, :6].astype(np.float64)
    return oracle.ellipses(r[:, 0:2], r[:, 2:5], r[:, 5])


def gpu_pxrect(g):
    bx, by = g["bbox"][:, 0], g["bbox"][:, 1]
    return np.stack([bx & 0xFFFF, bx >> 16, by & 0xFFFF, by >> 16], 1).astype(np.int32)


def check_binning(cam, g, label=""):
    """The oracle's emission from the GPU's records (rects, pixel boxes, ellipses, depths):
    its tile counts must be the GPU's, and its sorted pairs and ranges the GPU's, bit for bit."""
    trect = np.ascontiguousarray(g["rect"].astype(np.int32))
    ell, pxr = gpu_ellipses(g), gpu_pxrect(g)
    vis = g["n_tiles"] > 0
    kept = oracle.count_kept(trect[vis], pxr[vis], ell[vis])
    bad = np.nonzero(kept != g["n_tiles"][vis])[0]
    assert bad.size == 0, f"{label}: tile counts differ for {bad.size} Gaussians, e.g. {np.nonzero(vis)[0][bad[:5]]}"
    k, v = oracle.emit_pairs(trect, g["n_tiles"].astype(np.int64), g["depth_bits"], cam.tiles_x, pxr, ell)
    assert k.shape[0] == g["P"], f"{label}: pair count {g['P']} vs {k.shape[0]}"
    if "keys_unsorted" in g:
        # gs_bin_tiles emits in (tile & 255, depth bits, id) order: the oracle's id-order
        # emission, stably reordered by (tile low byte, depth), must match it pair for pair
        low = ((k >> np.uint64(32)) & np.uint64(0xFF)).astype(np.uint32)
        dbits = (k & np.uint64(0xFFFFFFFF)).astype(np.uint32)
        perm = np.lexsort((dbits, low))
        assert np.array_equal(g["keys_unsorted"], k[perm]), f"{label}: emitted keys differ"
        assert np.array_equal(g["vals_unsorted"], v[perm]), f"{label}: emitted ids differ"
    if "digit_counts" in g:
        # the binning's counts of the tile-id digits above the low byte: a histogram of the
        # oracle's pairs (rows for the passes the tile count needs; zero digit otherwise)
        tile = (k >> np.uint64(32)).astype(np.int64)
        tb = max(0, math.ceil(math.log2(cam.num_tiles))) if cam.num_tiles > 1 else 0
        for p in range(2):
            want = np.bincount((tile >> (8 + 8 * p)) & 255, minlength=256).astype(np.uint64)
            if 8 + 8 * p >= tb:  # no such pass: the row is not written beyond the clearing
                want = np.zeros(256, np.uint64)
            assert np.array_equal(g["digit_counts"][p], want), f"{label}: tile digit counts, pass {p}"
    sk, sv = oracle.sort_pairs(k, v)
    assert np.array_equal(g["keys"], sk), f"{label}: sorted keys differ"
    assert np.array_equal(g["vals"], sv), f"{label}: sorted ids differ"
    rg = oracle.tile_ranges(sk, cam.num_tiles)
    assert np.array_equal(g["ranges"], rg), f"{label}: tile ranges differ"
    # the schedule: a permutation of the tiles with non-increasing list-length buckets
    order = g["order"]
    assert np.array_equal(np.sort(order), np.arange(cam.num_tiles)), f"{label}: tile order is not a permutation"
    lens = (rg[:, 1] - rg[:, 0])[order]
    lg = np.floor(np.log2(np.maximum(lens, 1)))
    assert np.all(np.diff(lg) <= 0), f"{label}: tile order is not longest-first"


def check_end_to_end_keys(cam, g, label=""):
    """The oracle's sorted pairs from the raw inputs (its own projection, emission and sort)
    against the GPU's: identical once both lists drop the pairs of Gaussians whose depth
    rounding, pixel-box edge or tile test the oracle flags as within rounding of a threshold
    (check_projection caps how many there are).  Returns the number of pairs dropped."""
    p = g["oracle_proj"]
    amb = (p["flags"] & (1 | 2 | 8 | 16)) != 0
    k, v = oracle.emit_projected(p, cam.tiles_x)
    sk, sv = oracle.sort_pairs(k, v)
    keep_o, keep_g = ~amb[sv], ~amb[g["vals"]]
    assert np.array_equal(sk[keep_o], g["keys"][keep_g]), f"{label}: end-to-end keys differ"
    assert np.array_equal(sv[keep_o], g["vals"][keep_g]), f"{label}: end-to-end ids differ"
    return int((~keep_o).sum() + (~keep_g).sum())


def compare_pixels(gpu_col, gpu_T, gpu_n, orc, label="", tol=PIX_TOL):
    """gpu_col (npix, 3), gpu_T (npix,), gpu_n (npix,) against oracle render_pixels output."""
    nb = orc["nbranch"]
    br = orc["branches"]  # (npix, branches, 5)
    ok = np.zeros(gpu_col.shape[0], bool)
    for m in range(br.shape[1]):
        valid = nb > m
        d = np.abs(br[:, m, 0:3] - gpu_col).max(axis=1)
        dT = np.abs(br[:, m, 3] - gpu_T)
        same_n = br[:, m, 4] == gpu_n
        ok |= valid & (d <= tol) & (dT <= tol) & same_n
    excluded = nb == 0
    nex = int(excluded.sum())
    assert nex <= EXCLUDED_CAP * gpu_col.shape[0], f"{label}: {nex} pixels with more than three near-threshold decisions"
    bad = np.nonzero(~ok & ~excluded)[0]
    if bad.size:
        i = bad[0]
        raise AssertionError(
            f"{label}: {bad.size} pixels differ; first idx {i}: gpu {gpu_col[i]} T {gpu_T[i]} n {gpu_n[i]} "
            f"oracle {orc['col'][i]} T {orc['T'][i]} n {orc['n'][i]} nbranch {nb[i]}")
    return dict(pixels=int(gpu_col.shape[0]), ambiguous=int((nb > 1).sum()), excluded=int(excluded.sum()))


def check_render_chained(cam, g, bg=(0.0, 0.0, 0.0), pix=None, label=""):
    W, H = cam.width, cam.height
    orc = oracle.render_pixels(W, H, bg, rec9(g), g["vals"], g["ranges"], pix)
    img = g["image"].reshape(3, -1).T
    T = g["final_T"].reshape(-1)
    n = g["n_contrib"].reshape(-1).astype(np.int64)
    if pix is not None:
        img, T, n = img[pix], T[pix], n[pix]
    return compare_pixels(img, T, n, orc, label)


# float32's conditioning floor for a screen-space gradient sum S = sum_k t_k, in units of
# sum_k |t_k|: each term carries its own evaluation's rounding (a chain of ~10 operations),
# the wavefront's tree reduction adds 6 levels and the float32 atomics one rounding per
# (tile, quadrant) that adds into the Gaussian's total, so the first-order bound is
# (10 + 6 + visits - 1) u.  16 u covers the terms, the tree and the first accumulations; the
# elements that need it must be badly conditioned and few (check_conditioning_only)
COND_ULPS = 16.0 * 2.0 ** -24
# the rounding a float32 reverse walk carries into its terms, in units of the oracle's
# per-element scale (orc_render_bwd grad_err: at each contributor, the contributors behind it
# times the size of the parts of dL/dalpha): T recovered by a reciprocal and a product, and
# the colour behind accumulated with one fma, per contributor
ERR_ULPS = 4.0 * 2.0 ** -24


def grad_mismatch(gpu, ref, absum=None, counts=None, errscale=None):
    """Indices violating the gradient tolerance, and the worst ratio |g - ref| / tol.

    With ``absum`` (per-element sum of |terms|) the float32 conditioning floor joins the
    tolerance, with ``errscale`` (the oracle's rounding scale of the reverse walk) the walk's
    rounding too; ``counts`` (a dict) then receives how many elements needed them and the
    conditioning kappa = absum / |ref| of each."""
    gpu = np.asarray(gpu, np.float64)
    ref = np.asarray(ref, np.float64)
    tol = np.maximum(GRAD_REL * np.abs(ref), GRAD_ABS)
    if absum is not None:
        absum = np.asarray(absum, np.float64)
        cond = COND_ULPS * absum
        if errscale is not None:
            cond = cond + ERR_ULPS * np.asarray(errscale, np.float64)
        if counts is not None:
            err = np.abs(gpu - ref)
            only = (err > tol) & (err <= cond)
            counts["conditioning_only"] = int(np.sum(only))
            counts["kappa"] = absum[only] / np.maximum(np.abs(ref[only]), 1e-300)
        tol = np.maximum(tol, cond)
    r = np.abs(gpu - ref) / tol
    return np.nonzero(r > 1.0), float(np.max(r, initial=0.0))


def check_conditioning_only(counts, size, label=""):
    """Elements that passed only through the float32 conditioning floor: each must be badly
    conditioned (kappa >= COND_KAPPA_MIN) and there may be at most max(4, COND_CAP * size)."""
    k = counts["kappa"]
    say(f"{label}: {k.size} of {size} elements within the float32 conditioning floor only"
        + (f", kappa {np.array2string(np.sort(k), precision=3)}" if k.size else ""))
    assert k.size <= max(4, COND_CAP * size), f"{label}: {k.size} elements need the conditioning floor"
    assert np.all(k >= COND_KAPPA_MIN), f"{label}: an element needs the floor at kappa {k.min():.3g}"
