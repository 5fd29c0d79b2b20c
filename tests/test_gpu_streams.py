"""Several cameras in flight on several HIP streams at once, through the C ABI.

The library keeps no state between calls beyond the caller's buffers (and, per host thread
and GPU, the event of the pair-count read-back), so independent cameras on different
streams, each with its own projection, pair, workspace and gradient buffers, must give
what they give one after another on one stream: images, final transmittance and
contributor counts bit for bit; gradients and statistics up to the order of their float32
atomic additions (relative to each array's largest magnitude, 1e-4, well above the ~1e-6
that two single-stream runs differ by and far below any wrong term); visit counts exactly.
This is how the benchmark overlaps the cameras of a step.
"""
import pytest
import torch

from tile_differentiable_rasterizer_amd import raster, scenes

from gpu_util import say

pytestmark = pytest.mark.gpu

GRAD_KEYS = ("grad_screen", "dmeans", "dscales", "dquats", "dsh")


def _frame(rz, cam, dL, accum, denom):
    fwd = rz.forward(cam, with_keys=False)
    if dL is None:
        return fwd, None
    return fwd, rz.backward(fwd, dL, accum, denom)


@pytest.mark.parametrize("n_streams", [2, 3])
def test_cameras_on_several_streams_match_one_stream(n_streams):
    sc = scenes.sphere_scene(41, 60000, anisotropic=True)
    cams = [scenes.orbit_camera(0.4 + 0.7 * k, 640, 480, f=600.0) for k in range(6)]
    dev = torch.device("cuda")
    means, scales, quats, opac, sh = raster.scene_to_device(sc, dev)
    n = sc.n
    # one stream, one set of buffers: the reference (and the upstream gradients)
    rz0 = raster.Rasterizer(means, scales, quats, opac, sh, sc.sh_degree)
    acc0 = torch.zeros((n, 2), dtype=torch.float32, device=dev)
    den0 = torch.zeros(n, dtype=torch.int32, device=dev)
    ref, dLs = [], []
    for k, cam in enumerate(cams):
        fwd, _ = _frame(rz0, cam, None, None, None)
        target = torch.from_numpy(scenes.target_image(60 + k, cam.width, cam.height)).to(dev)
        dL = torch.sign(fwd["image"] - target).contiguous()
        dLs.append(dL)
        g = rz0.backward(fwd, dL, acc0, den0)
        ref.append((fwd["image"].clone(), fwd["final_T"].clone(), fwd["n_contrib"].clone(),
                    {key: g[key].clone() for key in GRAD_KEYS}))
    torch.cuda.synchronize()
    say(f"streams={n_streams}: reference done")

    # the same cameras round-robin over n_streams streams, each with its own buffers
    rzs = [raster.Rasterizer(means, scales, quats, opac, sh, sc.sh_degree) for _ in range(n_streams)]
    for r in rzs:  # size every set's pair buffers before the concurrent run
        for cam in cams:
            r.forward(cam, with_keys=False)
    accs = [torch.zeros((n, 2), dtype=torch.float32, device=dev) for _ in range(n_streams)]
    dens = [torch.zeros(n, dtype=torch.int32, device=dev) for _ in range(n_streams)]
    streams = [torch.cuda.Stream(device=dev) for _ in range(n_streams)]  # default priority
    torch.cuda.synchronize()
    out = []
    for k, cam in enumerate(cams):
        j = k % n_streams
        with torch.cuda.stream(streams[j]):
            out.append(_frame(rzs[j], cam, dLs[k], accs[j], dens[j]))
    torch.cuda.synchronize()

    for k, ((fwd, g), (img, T, nc, gref)) in enumerate(zip(out, ref)):
        assert torch.equal(fwd["image"], img), f"camera {k}: image"
        assert torch.equal(fwd["final_T"], T), f"camera {k}: final_T"
        assert torch.equal(fwd["n_contrib"], nc), f"camera {k}: n_contrib"
        for key in GRAD_KEYS:
            a, b = g[key].double(), gref[key].double()
            scale = b.abs().max().clamp_min(1e-30)
            rel = ((a - b).abs().max() / scale).item()
            assert rel <= 1e-4, f"camera {k}: {key} differs by {rel:.3g} of its largest magnitude"
    acc = sum(a.double() for a in accs)
    assert torch.equal(sum(dens), den0)
    rel = ((acc - acc0.double()).abs().max() / acc0.double().abs().max()).item()
    assert rel <= 1e-4, f"statistics differ by {rel:.3g}"
    say(f"streams={n_streams}: {len(cams)} cameras equal the one-stream run (statistics {rel:.2g})")


def test_bench_workload_on_four_streams():
    """The benchmark's own arrangement: cameras of the 1M-Gaussian 1080p workload on the
    current stream and three new ones, each with its own buffers, against the same cameras
    on one stream."""
    sc, cams, _ = scenes.workload("aniso_1m_sh3_1080p_8cam")
    cams = cams[:4]
    dev = torch.device("cuda")
    means, scales, quats, opac, sh = raster.scene_to_device(sc, dev)
    rz0 = raster.Rasterizer(means, scales, quats, opac, sh, sc.sh_degree)
    ref, dLs = [], []
    for k, cam in enumerate(cams):
        fwd, _ = _frame(rz0, cam, None, None, None)
        target = torch.from_numpy(scenes.target_image(5, cam.width, cam.height)).to(dev)
        dL = torch.sign(fwd["image"] - target).contiguous()
        dLs.append(dL)
        g = rz0.backward(fwd, dL)
        ref.append((fwd["image"].clone(), fwd["final_T"].clone(), fwd["n_contrib"].clone(),
                    {key: g[key].clone() for key in GRAD_KEYS}))
    torch.cuda.synchronize()
    del rz0
    rzs = [raster.Rasterizer(means, scales, quats, opac, sh, sc.sh_degree) for _ in cams]
    for r, cam in zip(rzs, cams):
        r.forward(cam, with_keys=False)  # sizes the pair buffers
    streams = [torch.cuda.current_stream()] + [torch.cuda.Stream(device=dev) for _ in range(len(cams) - 1)]
    torch.cuda.synchronize()
    out = []
    for k, cam in enumerate(cams):
        with torch.cuda.stream(streams[k]):
            out.append(_frame(rzs[k], cam, dLs[k], None, None))
    torch.cuda.synchronize()
    for k, ((fwd, g), (img, T, nc, gref)) in enumerate(zip(out, ref)):
        assert torch.equal(fwd["image"], img) and torch.equal(fwd["final_T"], T), f"camera {k}"
        assert torch.equal(fwd["n_contrib"], nc), f"camera {k}: n_contrib"
        for key in GRAD_KEYS:
            a, b = g[key].double(), gref[key].double()
            rel = ((a - b).abs().max() / b.abs().max().clamp_min(1e-30)).item()
            assert rel <= 1e-4, f"camera {k}: {key} differs by {rel:.3g} of its largest magnitude"
    say(f"bench workload: {len(cams)} cameras on {len(streams)} streams equal the one-stream run")
