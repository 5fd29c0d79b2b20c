"""The measurement hooks of gs_measure.h, through the C ABI: the memory-ceiling kernels move
what they say (exact checks on what they write) and the kernel timer counts the pair
sort's digit passes."""
import numpy as np
import pytest
import torch

from tile_differentiable_rasterizer_amd import raster, scenes

pytestmark = pytest.mark.gpu


def test_scatter_io_writes_every_valid_destination():
    n = 100_003
    rng = np.random.default_rng(71)
    keys = rng.integers(0, 2**63, n, dtype=np.int64)
    vals = rng.integers(0, 2**31, n, dtype=np.int64).astype(np.int32)
    dest = rng.permutation(n).astype(np.int64)
    dest[::97] = n + 5  # outside [0, n): skipped
    d = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    out = torch.full((n,), -1, dtype=torch.int32, device="cuda")
    raster.measure_scatter_io(d(keys), d(vals), d(dest.astype(np.uint32).view(np.int32)), out)
    torch.cuda.synchronize()
    got = out.cpu().numpy().view(np.uint32)
    ok = dest < n
    want = (vals.view(np.uint32).astype(np.uint64) + (keys.view(np.uint64) & 0xFFFFFFFF)) & 0xFFFFFFFF
    assert np.array_equal(got[dest[ok]], want[ok].astype(np.uint32))
    untouched = np.ones(n, bool)
    untouched[dest[ok]] = False
    assert np.all(got[untouched] == 0xFFFFFFFF)


def test_project_io_reads_the_projection_inputs():
    sc, cams, _ = scenes.workload("tiny_1k_sh0_64")
    sc3 = scenes.sphere_scene(5, 3001, anisotropic=True)
    for scene in (sc, sc3):
        means, scales, quats, opac, sh = raster.scene_to_device(scene, "cuda")
        out = raster.alloc_projected(scene.n, torch.device("cuda"))
        raster.measure_project_io(means, scales, quats, opac, sh, scene.sh_degree, out)
        torch.cuda.synchronize()
        # the depth slot receives each Gaussian's z; the record's second word its opacity
        assert torch.equal(out["depth"], means[:, 2])
        assert torch.equal(out["rec"][:, 5], opac)


def test_timer_counts_the_pair_sort_passes():
    sc, cams, _ = scenes.workload("spheres_100k_sh3_800")
    means, scales, quats, opac, sh = raster.scene_to_device(sc, "cuda")
    rz = raster.Rasterizer(means, scales, quats, opac, sh, sc.sh_degree)
    rz.forward(cams[0], with_keys=False)
    assert raster.kernel_timer_start("k_onesweep_u64") == raster.GS_OK
    for _ in range(3):
        rz.forward(cams[0], with_keys=False)
    st, launches, ms = raster.kernel_timer_stop()
    assert st == raster.GS_OK and launches == 3 and ms > 0.0  # 800x800: one digit pass per sort
