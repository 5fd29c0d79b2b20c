"""GPU parity: every C-ABI stage against the float64 oracle (see gpu_util for the rules).

Workloads are the seeded synthetic scenes of tile_differentiable_rasterizer_amd.scenes:
the 1k SH0 64x64 scene, the 100k SH3 sphere scene at 800x800, and the 1M anisotropic
SH3 scene at 1920x1080 (all 8 orbit cameras, every pixel, in the launch configuration the
benchmark times).
"""
import math

import numpy as np
import pytest
import torch

import oracle
from tile_differentiable_rasterizer_amd import raster, scenes

pytestmark = pytest.mark.gpu

from gpu_util import (check_binning, check_end_to_end_keys, check_projection, check_render_chained, compare_pixels,
                      gpu_stages, rec9,
                      say)


@pytest.fixture(scope="module")
def tiny():
    sc, cams, _ = scenes.workload("tiny_1k_sh0_64")
    return sc, cams[0]


@pytest.fixture(scope="module")
def spheres():
    sc, cams, _ = scenes.workload("spheres_100k_sh3_800")
    return sc, cams[0]


@pytest.fixture(scope="module")
def aniso1m():
    sc, cams, _ = scenes.workload("aniso_1m_sh3_1080p_8cam")
    return sc, cams


def test_tiny_all_stages_and_end_to_end(tiny):
    sc, cam = tiny
    say("tiny: gpu stages")
    g = gpu_stages(sc, cam)
    say(f"tiny: P={g['P']}")
    info = check_projection(sc, cam, g, "tiny")
    check_binning(cam, g, "tiny")
    r = check_render_chained(cam, g, label="tiny")
    say(f"tiny: projection {info}, render {r}")
    # end to end: the oracle from the raw inputs
    e2e = oracle.end_to_end(sc, cam)
    assert np.array_equal(e2e["skeys"], g["keys"])
    assert np.array_equal(e2e["svals"], g["vals"])
    img = g["image"].reshape(3, -1).T
    compare_pixels(img, g["final_T"].reshape(-1), g["n_contrib"].reshape(-1).astype(np.int64), e2e["render"],
                   "tiny end-to-end")


def test_spheres_100k_all_stages_and_end_to_end(spheres):
    sc, cam = spheres
    say("spheres: gpu stages")
    g = gpu_stages(sc, cam)
    say(f"spheres: P={g['P']}")
    info = check_projection(sc, cam, g, "spheres")
    check_binning(cam, g, "spheres")
    r = check_render_chained(cam, g, label="spheres")
    say(f"spheres: projection {info}, render {r}")
    e2e = oracle.end_to_end(sc, cam)
    assert np.array_equal(e2e["skeys"], g["keys"])
    assert np.array_equal(e2e["svals"], g["vals"])
    img = g["image"].reshape(3, -1).T
    r2 = compare_pixels(img, g["final_T"].reshape(-1), g["n_contrib"].reshape(-1).astype(np.int64), e2e["render"],
                        "spheres end-to-end")
    say(f"spheres end-to-end: {r2}")


@pytest.mark.parametrize("cam_index", range(8))
def test_aniso_1m_1080p_every_camera_full_frame(aniso1m, cam_index):
    """The headline workload, every one of its 8 orbit cameras, in the launch configuration
    the benchmark times: projection against the oracle's, bit-exact emission, sort and
    ranges from the GPU's records, every pixel of the frame against the oracle's compositing
    of the GPU's lists, and the sorted pairs end to end."""
    sc, cams = aniso1m
    cam = cams[cam_index]
    say(f"aniso1m cam {cam_index}: gpu stages")
    g = gpu_stages(sc, cam)
    say(f"aniso1m cam {cam_index}: P={g['P']}")
    info = check_projection(sc, cam, g, "aniso1m")
    check_binning(cam, g, "aniso1m")
    r = check_render_chained(cam, g, label="aniso1m")
    dropped = check_end_to_end_keys(cam, g, "aniso1m")
    lens = g["ranges"][:, 1] - g["ranges"][:, 0]
    say(f"aniso1m cam {cam_index}: projection {info}, render {r}, max list {lens.max()}, "
        f"end-to-end pairs dropped for flagged Gaussians {dropped}")


def test_forward_is_bitwise_repeatable(spheres):
    sc, cam = spheres
    a = gpu_stages(sc, cam, keep_unsorted=False)
    b = gpu_stages(sc, cam, keep_unsorted=False)
    for k in ("rec", "keys", "vals", "ranges", "image", "final_T", "n_contrib"):
        assert np.array_equal(a[k], b[k]), k


def test_background_and_ragged_image():
    sc, _ = scenes.tiny_scene(7, 600)
    cam = scenes.Camera(np.eye(3, dtype=np.float32), np.zeros(3, np.float32), 60.0, 60.0, 37.0, 21.5, 77, 45, 0.2)
    bg = (0.25, 0.5, 1.0)
    g = gpu_stages(sc, cam, bg)
    check_projection(sc, cam, g, "ragged")
    check_binning(cam, g, "ragged")
    check_render_chained(cam, g, bg=bg, label="ragged")
    e2e = oracle.end_to_end(sc, cam, bg)
    compare_pixels(g["image"].reshape(3, -1).T, g["final_T"].reshape(-1),
                   g["n_contrib"].reshape(-1).astype(np.int64), e2e["render"], "ragged end-to-end")


def test_dense_small_gaussians_fill_the_emission_partitions():
    """60k Gaussians of a pixel or two (one to four tiles each) at 640x480: an emission
    partition of 1024 pairs then holds ~730 Gaussians, more than the 224 whose tile records
    the scattering pass stages in LDS, so the records past them are read from memory, and a
    counting workgroup walks ~1,460 Gaussians.  Binning, sort and ranges bit-exact against
    the oracle, every pixel of the chained compositing, and the sorted pairs end to end."""
    sc, _ = scenes.tiny_scene(23, 60000)
    sc.scales[...] = sc.scales * np.float32(0.05)
    cam = scenes.Camera(np.eye(3, dtype=np.float32), np.zeros(3, np.float32), 600.0, 600.0, 320.0, 240.0, 640, 480,
                        float(np.float32(0.2)))
    g = gpu_stages(sc, cam)
    vis = int((g["n_tiles"] > 0).sum())
    per_part = vis / max(1, -(-g["P"] // 1024))
    say(f"dense small: P={g['P']}, {vis} visible, {per_part:.0f} Gaussians per emission partition")
    assert per_part > 224
    info = check_projection(sc, cam, g, "dense small")
    check_binning(cam, g, "dense small")
    r = check_render_chained(cam, g, label="dense small")
    dropped = check_end_to_end_keys(cam, g, "dense small")
    say(f"dense small: projection {info}, render {r}, end-to-end pairs dropped for flagged Gaussians {dropped}")


def test_sort_counts_its_own_digits_the_same(spheres):
    """gs_sort_keys without the binning's tile-digit counts (its own counting read) sorts to
    the same pairs and ranges as with them (the longest-first schedule may order tiles of
    one length bucket differently from run to run; the image does not depend on it)."""
    sc, cam = spheres
    a = gpu_stages(sc, cam, keep_unsorted=False, digit_counts=True)
    b = gpu_stages(sc, cam, keep_unsorted=False, digit_counts=False)
    for k in ("keys", "vals", "ranges", "image"):
        assert np.array_equal(a[k], b[k]), k


def _binned_pairs(sc, cam):
    dev = torch.device("cuda")
    means, scales, quats, opac, sh = raster.scene_to_device(sc, dev)
    proj = raster.project(means, scales, quats, opac, sh, sc.sh_degree, cam)
    tiles = cam.num_tiles
    ws = torch.empty(max(raster.workspace_bytes(sc.n, 1, tiles), 8), dtype=torch.uint8, device=dev)
    st, P = raster.bin_tiles(proj, cam, None, None, ws)
    keys = torch.empty(max(P, 1), dtype=torch.int64, device=dev)
    vals = torch.empty(max(P, 1), dtype=torch.int32, device=dev)
    ws = torch.empty(raster.workspace_bytes(sc.n, P, tiles), dtype=torch.uint8, device=dev)
    dc = torch.empty(raster.TILE_DIGIT_COUNTS, dtype=torch.int64, device=dev)
    st, P = raster.bin_tiles(proj, cam, keys, vals, ws, digit_counts=dc)
    assert st == raster.GS_OK
    return P, tiles, keys, vals, dc, ws


@pytest.mark.parametrize("case", ["spheres", "aniso1m_cam5", "large_image"])
def test_sort_ids_matches_sort_keys(case, spheres, aniso1m):
    """gs_sort_ids (the last digit pass writes the ids only) leaves the ids, ranges and
    result buffer of gs_sort_keys, bit for bit: one digit pass (800x800, 1080p) and two
    (a 4200x4150 image, whose first pass must still write the keys)."""
    if case == "spheres":
        sc, cam = spheres
    elif case == "aniso1m_cam5":
        sc, cam = aniso1m[0], aniso1m[1][5]
    else:
        sc, _ = scenes.tiny_scene(11, 2000)
        cam = scenes.Camera(np.eye(3, dtype=np.float32), np.zeros(3, np.float32), 4400.0, 4400.0, 2100.0, 2075.0,
                            4200, 4150, 0.2)
    P, tiles, keys, vals, dc, ws = _binned_pairs(sc, cam)
    out = []
    for fn in (raster.sort_keys, raster.sort_ids):
        k, v = keys.clone(), vals.clone()
        kt, vt = torch.empty_like(k), torch.empty_like(v)
        rg = torch.empty((tiles, 2), dtype=torch.int64, device=k.device)
        order = torch.empty(tiles, dtype=torch.int32, device=k.device)
        if fn is raster.sort_keys:
            in_tmp = fn(P, tiles, k, v, kt, vt, rg, ws, order, leave_in_tmp=True, digit_counts=dc)
        else:
            in_tmp = fn(P, tiles, k, v, kt, vt, rg, ws, order, digit_counts=dc)
        torch.cuda.synchronize()
        rv = (vt if in_tmp else v)[:P].cpu().numpy()
        out.append((in_tmp, rv, rg.cpu().numpy(), order.cpu().numpy()))
    (t0, v0, r0, o0), (t1, v1, r1, o1) = out
    assert t0 == t1 and np.array_equal(v0, v1) and np.array_equal(r0, r1)
    assert np.array_equal(np.sort(o1), np.arange(tiles))
    lens = (r1[:, 1] - r1[:, 0])[o1]
    assert np.all(np.diff(np.floor(np.log2(np.maximum(lens, 1)))) <= 0)
    say(f"sort_ids {case}: P={P}, result in tmp: {t1}")


def test_sort_ids_requires_the_result_word():
    import ctypes as C
    L = raster.lib()
    d = torch.zeros(8, dtype=torch.int64, device="cuda")
    st = L.gs_sort_ids(0, 16, 40, d.data_ptr(), d.data_ptr(), d.data_ptr(), d.data_ptr(), d.data_ptr(), None, None,
                       None, d.data_ptr(), 64, None)
    assert st == raster.GS_ERR_INVALID_ARG


def _needles(sc, rng, k, lo, hi, thin=None):
    """Makes the first k Gaussians long ellipses, fairly opaque: axis 0 long (scale
    e^U[lo, hi]); the other two e^U[-7, -5] (needles), or, with thin = (r0, r1), the long
    scale times e^U[ln r0, ln r1]."""
    long_ = np.exp(rng.uniform(lo, hi, k))
    sc.scales[:k, 0] = long_.astype(np.float32)
    if thin is None:
        sc.scales[:k, 1:] = np.exp(rng.uniform(-7.0, -5.0, (k, 2))).astype(np.float32)
    else:
        sc.scales[:k, 1:] = (long_[:, None] * np.exp(rng.uniform(math.log(thin[0]), math.log(thin[1]), (k, 2)))
                             ).astype(np.float32)
    sc.opacities[:k] = rng.uniform(0.3, 0.99, k).astype(np.float32)


def _rect_sizes(g):
    r = g["rect"]
    return r[:, 3] - r[:, 2] + 1, r[:, 1] - r[:, 0] + 1


def test_tall_ellipses_are_culled_by_the_ellipse_test():
    """Long ellipses whose tile rectangles span up to the whole 1080p frame: the ellipse test
    ("Training 10M Gaussians in 8 GB: Spirula Studio's VRAM efficiency", 16-bit AABB section)
    applies to every rectangle, whatever its size.  The tile counts, the emitted and sorted
    pairs and the ranges are bit-exact against the oracle's emission from the GPU's records,
    and every pixel of the frame matches the oracle's compositing.  The short axes are 1/20
    to 1/5 of the long one, the anisotropy of the anisotropic workloads (whose scales span
    e^[-6, -5] to e^[-4, -3]); far thinner needles are binned bit-exactly in the large-image
    test, but their float32 quadratic form is beyond the 1e-4 pixel bound."""
    sc, _ = scenes.tiny_scene(13, 3000)
    rng = np.random.default_rng(13)
    _needles(sc, rng, 600, math.log(0.05), math.log(0.8), thin=(1 / 20, 1 / 5))
    cam = scenes.Camera(np.eye(3, dtype=np.float32), np.zeros(3, np.float32), 1000.0, 1000.0, 960.0, 540.0,
                        1920, 1080, 0.2)
    g = gpu_stages(sc, cam)
    rows, cols = _rect_sizes(g)
    vis = g["n_tiles"] > 0
    big = vis & ((rows > 8) | (cols > 255))
    culled = big & (g["n_tiles"] < rows * cols)
    say(f"tall ellipses: P={g['P']}, {int(big.sum())} rectangles over 8 tile rows, {int(culled.sum())} culled")
    assert big.sum() >= 200 and culled.sum() >= 0.9 * big.sum()
    check_projection(sc, cam, g, "tall ellipses")
    check_binning(cam, g, "tall ellipses")
    r = check_render_chained(cam, g, label="tall ellipses")
    say(f"tall ellipses: render {r}")


def test_large_image_two_tile_digit_passes():
    """4200x4150 pixels = 263x260 tiles: tile ids take 17 bits, so the pair sort makes two
    digit passes above the low byte and the binning counts both digits.  Three Gaussians
    cover the whole image; 300 thin needles have rectangles of many tile rows, up to more
    than 255 tile columns, which the ellipse test culls like any other."""
    sc, _ = scenes.tiny_scene(11, 2000)
    rng = np.random.default_rng(11)
    _needles(sc, rng, 300, math.log(0.05), math.log(1.2))
    # three Gaussians wider than the image: tile rows of 263 tiles, more than a turn of the
    # low byte's 256 values in one row
    sc.means[:3] = np.array([[0.0, 0.0, 3.0], [0.3, -0.2, 3.5], [-0.4, 0.1, 2.5]], np.float32)
    sc.scales[:3] = 1.5
    sc.opacities[:3] = 0.9
    cam = scenes.Camera(np.eye(3, dtype=np.float32), np.zeros(3, np.float32), 4400.0, 4400.0, 2100.0, 2075.0,
                        4200, 4150, 0.2)
    assert cam.num_tiles > 65536
    g = gpu_stages(sc, cam)
    assert np.all(g["n_tiles"][:3] == cam.num_tiles)  # every tile of the image
    rows, cols = _rect_sizes(g)
    wide = (g["n_tiles"] > 0) & (cols > 255)
    say(f"large image: P={g['P']}, pass-1 digits {int((g['digit_counts'][1] > 0).sum())}, "
        f"{int(wide[3:].sum())} needles over 255 tile columns")
    assert wide[3:].sum() >= 5 and np.all(g["n_tiles"][3:][wide[3:]] < (rows * cols)[3:][wide[3:]])
    assert g["digit_counts"][1][1] > 0  # pairs with tile ids >= 65536 exist
    check_projection(sc, cam, g, "large image")
    check_binning(cam, g, "large image")
