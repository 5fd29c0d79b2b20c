"""GPU parity of the quantised-SH path (gs_quantize_sh, gs_project_qsh) through the C ABI.

Codes and bounds must be bit-exact against the oracle's quantiser (oracle/qsh.py).  The
projection of the codes must be bit-equal to the float32 projection of the oracle's decoded
coefficients (the decode is one fixed float32 expression on both sides), and pass the usual
projection parity against the float64 oracle on the decoded scene.
"""
import numpy as np
import pytest
import torch

import oracle.qsh as Q
from tile_differentiable_rasterizer_amd import raster, scenes

from gpu_util import check_projection, say

pytestmark = pytest.mark.gpu


def host(proj) -> dict:
    rec = proj["rec"].cpu().numpy()
    return dict(rec=rec, bbox=rec[:, 9:11].view(np.uint32), depth_bits=proj["depth"].cpu().numpy().view(np.uint32),
                rect=proj["rect"].cpu().numpy().view(np.uint16).astype(np.int32),
                n_tiles=proj["n_tiles"].cpu().numpy().view(np.uint32), clamp=proj["clamp"].cpu().numpy(),
                runs=proj["runs"].cpu().numpy())


@pytest.mark.parametrize("bits", [8, 16])
@pytest.mark.parametrize("L,n", [(0, 1001), (1, 777), (2, 2049), (3, 5000)])
def test_codes_bit_exact(bits, L, n):
    rng = np.random.default_rng(100 + L)
    K = (L + 1) ** 2
    sh = (rng.normal(size=(n, K, 3)) * np.exp(rng.uniform(-3, 1, (n, 1, 1)))).astype(np.float32)
    sh[: n // 10] = 0.25  # constant blocks (equal bounds)
    dev = torch.device("cuda")
    codes, bounds = raster.quantize_sh(torch.from_numpy(sh).to(dev), L, bits)
    torch.cuda.synchronize()
    oc, ob = Q.quantize(sh, bits)
    gc = codes.cpu().numpy().view(np.uint16 if bits == 16 else np.uint8)
    assert np.array_equal(bounds.cpu().numpy(), ob), (bits, L)
    assert np.array_equal(gc, oc), (bits, L, int((gc != oc).sum()))


@pytest.mark.parametrize("bits", [8, 16])
@pytest.mark.parametrize("name,n,L", [("spheres_100k_sh3_800", 30000, 0), ("spheres_100k_sh3_800", 30000, 1),
                                      ("spheres_100k_sh3_800", 30000, 2), ("spheres_100k_sh3_800", 30000, 3),
                                      ("aniso_1m_sh3_1080p_8cam", None, 3)])
def test_projection_of_codes(bits, name, n, L):
    """The projection of codes (compiled per SH degree and code width) equals the float32
    projection of the decoded coefficients, and the oracle's; degrees below 3 cut the
    scene's SH."""
    sc, cams, _ = scenes.workload(name, n)
    if L < sc.sh_degree:
        sc = scenes.Scene(sc.means, sc.scales, sc.quats, sc.opacities,
                          np.ascontiguousarray(sc.sh[:, :(L + 1) ** 2, :]), L)
    cam = cams[0]
    dev = torch.device("cuda")
    means, scales, quats, opac, sh = raster.scene_to_device(sc, dev)
    codes, bounds = raster.quantize_sh(sh, sc.sh_degree, bits)
    pq = raster.project_qsh(means, scales, quats, opac, codes, bounds, bits, sc.sh_degree, cam)
    oc, ob = Q.quantize(sc.sh, bits)
    deq = Q.dequantize(oc, ob, bits)
    pf = raster.project(means, scales, quats, opac, torch.from_numpy(deq).to(dev), sc.sh_degree, cam)
    torch.cuda.synchronize()
    hq, hf = host(pq), host(pf)
    for k in hq:
        assert np.array_equal(hq[k], hf[k]), f"{name} q{bits}: {k} differs from the float32 path on decoded SH"
    sq = scenes.Scene(sc.means, sc.scales, sc.quats, sc.opacities, deq, sc.sh_degree)
    stats = check_projection(sq, cam, hq, f"{name} q{bits}")
    say(f"{name} q{bits}: {stats}")


def test_errors():
    import ctypes as C

    L = raster.lib()
    assert L.gs_quantize_sh(10, None, 3, 12, None, None, None) == raster.GS_ERR_INVALID_ARG
    assert L.gs_quantize_sh(10, None, 3, 8, None, None, None) == raster.GS_ERR_INVALID_ARG
    assert L.gs_quantize_sh(0, None, 3, 8, None, None, None) == raster.GS_OK
    cam = raster.camera_struct(scenes.workload("tiny_1k_sh0_64")[1][0])
    assert L.gs_project_qsh(5, None, None, None, None, None, None, 4, 3, C.byref(cam), raster.GsProjected(),
                            None) == raster.GS_ERR_INVALID_ARG
