"""GPU parity at the 10M-Gaussian scale: the anisotropic SH3 scene of 10,000,000 Gaussians
at 1920x1080, one orbit camera, forward only, through the C ABI in the launch
configuration the benchmark uses.

At this size the oracle checks every Gaussian's projection, and the rest on properties that
hold at any size plus exact samples: the sorted keys are non-decreasing with equal keys in
id order, the tile ranges bound each tile's run, the pair count is the sum of the tile
counts, every list of 24 sampled tiles equals the depth-ordered set of Gaussians whose
(oracle-checked) rectangles cover the tile and whose records pass the oracle's ellipse
test for it, and every pixel of those tiles matches the
oracle's compositing of the GPU's own lists.  The test prints the pair count and the peak
device memory.
"""
import numpy as np
import pytest
import torch

from tile_differentiable_rasterizer_amd import scenes

pytestmark = pytest.mark.gpu

import oracle
from gpu_util import check_projection, check_render_chained, gpu_ellipses, gpu_pxrect, gpu_stages, say


@pytest.fixture(scope="module")
def big():
    sc, cams, _ = scenes.workload("aniso_10m_sh3_1080p")
    return sc, cams[0]


def test_aniso_10m_1080p_forward(big):
    sc, cam = big
    say(f"aniso10m: {sc.n} Gaussians generated; gpu stages")
    torch.cuda.synchronize()
    torch.cuda.reset_peak_memory_stats()
    g = gpu_stages(sc, cam, keep_unsorted=False)
    peak = torch.cuda.max_memory_allocated()
    P = g["P"]
    say(f"aniso10m: P={P} pairs, peak device memory {peak / 2**30:.2f} GiB")
    info = check_projection(sc, cam, g, "aniso10m")
    say(f"aniso10m: projection {info}")

    keys, vals, rg = g["keys"], g["vals"], g["ranges"]
    assert P == int(g["n_tiles"].astype(np.uint64).sum())
    assert np.all(keys[1:] >= keys[:-1]), "keys not sorted"
    eq = keys[1:] == keys[:-1]
    assert np.all(vals[1:][eq] > vals[:-1][eq]), "equal keys not in id order"
    tile_of = (keys >> np.uint64(32)).astype(np.int64)
    counts = np.bincount(tile_of, minlength=cam.num_tiles)
    starts = np.concatenate([[0], np.cumsum(counts)[:-1]])
    nz = counts > 0
    assert np.array_equal(rg[nz, 0], starts[nz]) and np.array_equal(rg[nz, 1], starts[nz] + counts[nz])
    assert np.all(rg[~nz] == 0)

    rng = np.random.default_rng(4)
    lens = rg[:, 1] - rg[:, 0]
    tiles = np.unique(np.concatenate([rng.choice(cam.num_tiles, 20, replace=False), np.argsort(lens)[-4:]]))
    rect = g["rect"]  # (x0, x1, y0, y1) in tiles
    vis = np.nonzero(g["n_tiles"] > 0)[0]
    rv, dv = rect[vis], g["depth_bits"][vis]
    ell, pxr = gpu_ellipses(g), gpu_pxrect(g)
    pix = []
    for t in tiles:
        tx, ty = int(t % cam.tiles_x), int(t // cam.tiles_x)
        cover = (rv[:, 0] <= tx) & (rv[:, 1] >= tx) & (rv[:, 2] <= ty) & (rv[:, 3] >= ty)
        ids = vis[cover]
        keep, _ = oracle.tile_keeps(ell[ids], pxr[ids], tx, ty)
        ids, dsel = ids[keep], dv[cover][keep]
        want = ids[np.lexsort((ids, dsel))]
        got = vals[rg[t, 0]:rg[t, 1]]
        assert np.array_equal(got, want.astype(np.uint32)), f"aniso10m: tile {t} list differs"
        for j in range(ty * 16, min(ty * 16 + 16, cam.height)):
            for i in range(tx * 16, min(tx * 16 + 16, cam.width)):
                pix.append(j * cam.width + i)
    r = check_render_chained(cam, g, pix=np.array(pix), label="aniso10m")
    say(f"aniso10m: {len(tiles)} tiles exact (longest list {lens.max()}), render {r}")
