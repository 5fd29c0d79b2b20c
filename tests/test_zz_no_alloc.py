"""gs_sort_keys_noalloc (the sort with the library's fixed per-GPU scratch, for callers that
cannot allocate) against gs_sort_keys with a caller workspace, through the C ABI: the same
sorted keys and ids, ranges, result buffer and a valid longest-first order, on two calls in
a row with the second smaller (the scratch keeps the first call's contents), for both the
binning's pairs (one digit pass, counts given) and arbitrary keys (a full six-pass sort
that counts its own digits); and a sort too large for the scratch is refused before any
work is queued."""
import numpy as np
import pytest
import torch

from tile_differentiable_rasterizer_amd import raster, scenes

pytestmark = pytest.mark.gpu


def _binned(name, n=None):
    sc, cams, _ = scenes.workload(name, n)
    cam = cams[0]
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
    return P, tiles, keys, vals, dc, 40


def _random(P, tiles, seed):
    rng = np.random.default_rng(seed)
    tile = rng.integers(0, tiles, P).astype(np.uint64)
    depth = np.float32(rng.uniform(0.5, 50.0, P)).view(np.uint32).astype(np.uint64)
    depth[rng.integers(0, P, P // 10)] = depth[0]  # equal keys: ids must stay in order
    k = (tile << np.uint64(32)) | depth
    dev = torch.device("cuda")
    keys = torch.from_numpy(k.view(np.int64)).to(dev)
    vals = torch.from_numpy(np.arange(P, dtype=np.int32)).to(dev)
    return P, tiles, keys, vals, None, 0


def _sort_both(P, tiles, keys, vals, dc, low):
    dev = keys.device
    out = []
    for noalloc in (False, True):
        k, v = keys.clone(), vals.clone()
        kt, vt = torch.empty_like(k), torch.empty_like(v)
        ranges = torch.full((tiles, 2), -7, dtype=torch.int64, device=dev)
        order = torch.full((tiles,), -1, dtype=torch.int32, device=dev)
        if noalloc:
            st, in_tmp = raster.sort_keys_noalloc(P, tiles, k, v, kt, vt, ranges, order, sorted_low_bits=low,
                                                  leave_in_tmp=True, digit_counts=dc)
            assert st == raster.GS_OK, raster.lib().gs_status_string(st)
        else:
            ws = torch.empty(raster.workspace_bytes(0, P, tiles), dtype=torch.uint8, device=dev)
            in_tmp = raster.sort_keys(P, tiles, k, v, kt, vt, ranges, ws, order, sorted_low_bits=low,
                                      leave_in_tmp=True, digit_counts=dc)
        torch.cuda.synchronize()
        rk, rv = (kt, vt) if in_tmp else (k, v)
        out.append((in_tmp, rk[:P].cpu().numpy(), rv[:P].cpu().numpy(), ranges.cpu().numpy(), order.cpu().numpy()))
    (t0, k0, v0, r0, o0), (t1, k1, v1, r1, o1) = out
    assert t0 == t1
    assert np.array_equal(k0, k1) and np.array_equal(v0, v1) and np.array_equal(r0, r1)
    assert np.array_equal(np.sort(o1), np.arange(tiles))
    lens = (r1[:, 1] - r1[:, 0])[o1]
    assert np.all(np.diff(np.floor(np.log2(np.maximum(lens, 1)))) <= 0)
    return P


def test_binned_pairs_twice_second_smaller():
    big = _sort_both(*_binned("spheres_100k_sh3_800"))
    small = _sort_both(*_binned("spheres_100k_sh3_800", 20000))
    assert small < big


def test_full_sort_twice_second_smaller():
    _sort_both(*_random(300_000, 5000, 1))
    _sort_both(*_random(40_000, 700, 2))


def test_too_large_for_the_scratch_is_refused():
    dev = torch.device("cuda")
    k = torch.zeros(1, dtype=torch.int64, device=dev)
    v = torch.zeros(1, dtype=torch.int32, device=dev)
    ranges = torch.zeros((8160, 2), dtype=torch.int64, device=dev)
    # a full sort of 2^26 pairs needs 6 passes x 2 KiB x 16384 partitions: more than the scratch;
    # the call checks that before touching the (too short) buffers
    st = raster.sort_keys_noalloc(1 << 26, 8160, k, v, k, v, ranges, sorted_low_bits=0)
    assert st == raster.GS_ERR_WORKSPACE
