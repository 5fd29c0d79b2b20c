"""Benchmark: frames/s and Mpixels/s of the tile rasteriser at 1M SH3 Gaussians, 1920x1080.

One step = the whole hot path for the 8 orbit cameras of the 1M-Gaussian anisotropic SH3
workload: per camera project -> bin (incl. the pair-count read-back) -> sort -> composite
-> backward (compositing and projection, with densification statistics).  The upstream
gradient is sign(render - target) for a uniform [0, 1] target, computed once before
timing.  Inputs are resident in HBM before the timed region.

The cameras of a step are independent, so they go round-robin over --streams HIP streams
(default priority), each with its own projection, pair, workspace and gradient buffers:
the latency-bound binning and sort of one camera run beside the compositing of another.
The same loop on one stream is reported as well ("single_stream"); the per-kernel times
and the roofline come from that loop, so they are the kernels' own, without another
stream's work beside them.  Also reported: the forward-only rate, per-stage times (HIP
events on the launch stream), and the float64 oracle timed on a bounded sample on the
host cores.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--streams S] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

WORKLOAD = "aniso_1m_sh3_1080p_8cam"
HBM_PEAK_GBS = 8000.0
VALU_PEAK_TOPS = 78.6   # fp32 lane-ops/s: the published 157.3 TFLOP/s with an FMA as one op (157.3 / 2)
TMIN = float(np.float32(1e-4))

# Algorithmic VALU lane-operations of the plain per-pixel loops, one issue slot per operation.
# Forward, per (pixel, list entry) evaluation: offset (2), quadratic form (5), exp (counted
# as 4 issue slots: the transcendental rate is a quarter), opacity product and clamp (2),
# threshold test (1), weight (1), colour accumulate (3), transmittance update (2), stop
# test (1).
OPS_PER_EVAL_FWD = 21
# Backward, per (pixel, contributor) of the reverse walk with one scalar for the colour
# behind: the alpha re-evaluation (offset 2, quadratic form 5, exponent scale 1 + exp 4,
# opacity product and clamp 2 = 14), the skip and walk tests (2), transmittance recovery
# (1 - alpha, reciprocal as 4 slots, product = 6), weight (1), dL.rgb (3), colour gradients
# (3), d alpha (2) and its background term (2), colour-behind update (1), the alpha-clamp
# compare and select (2), opacity gradient (1), dq (3), dq.dx and dq.dy (2), conic terms (3),
# mean terms (4), norm of the mean gradient (product, fma, sqrt as 4 slots = 6).
OPS_PER_EVAL_BWD = 55


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--streams", type=int, default=4, help="HIP streams the cameras of a step go round-robin over")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=20.0, help="seconds of oracle work to aim for")
    ap.add_argument("--no-configs", action="store_true", help="skip the per-configuration report")
    ap.add_argument("--frames", type=int, default=20, help="timed frames per camera in the per-configuration report")
    ap.add_argument("--oracle-10m", action="store_true",
                    help="also time the oracle single-threaded on the 10M-Gaussian configuration (minutes)")
    ap.add_argument("--profile", action="store_true",
                    help="profiler run: single-stream loops only (kernels timed alone), no CPU baseline, plus a "
                         "1 GiB device copy that calibrates HBM counters")
    return ap.parse_args()


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on exactly one GPU (asked for {args.gpus}); this path is built and "
              "measured for one GPU only; it does not run across GPUs.", file=sys.stderr)
        sys.exit(2)
    import torch

    from tile_differentiable_rasterizer_amd import raster, scenes

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    log("generating the 1M-Gaussian scene")
    sc, cams, _ = scenes.workload(WORKLOAD)
    N = sc.n
    means, scales, quats, opac, sh = raster.scene_to_device(sc, dev)
    NS = max(1, args.streams)
    # one set of per-camera buffers per stream: projection, pairs, workspace (Rasterizer),
    # gradients and densification statistics
    rzs = [raster.Rasterizer(means, scales, quats, opac, sh, sc.sh_degree) for _ in range(NS)]
    rz = rzs[0]
    stream = torch.cuda.current_stream()
    streams = [stream] + [torch.cuda.Stream(device=dev) for _ in range(NS - 1)]  # default priority

    # warm-up pass per camera sizes the pair buffers and builds the upstream gradients
    log("sizing buffers")
    dLs = []
    for k, cam in enumerate(cams):
        for r in rzs:
            out = r.forward(cam)
        target = torch.from_numpy(scenes.target_image(5, cam.width, cam.height)).to(dev)
        dLs.append(torch.sign(out["image"] - target).contiguous())
    tiles = cams[0].num_tiles
    H, W = cams[0].height, cams[0].width
    ranges = [torch.empty((tiles, 2), dtype=torch.int64, device=dev) for _ in cams]
    orders = [torch.empty(tiles, dtype=torch.int32, device=dev) for _ in cams]
    images = [torch.empty((3, H, W), dtype=torch.float32, device=dev) for _ in cams]
    finalT = [torch.empty((H, W), dtype=torch.float32, device=dev) for _ in cams]
    ncon = [torch.empty((H, W), dtype=torch.int32, device=dev) for _ in cams]
    grads = [raster.alloc_grads(N, sc.sh_degree, dev) for _ in range(NS)]
    accums = [torch.zeros((N, 2), dtype=torch.float32, device=dev) for _ in range(NS)]
    denoms = [torch.zeros(N, dtype=torch.int32, device=dev) for _ in range(NS)]
    torch.cuda.synchronize()
    stages = ["project", "bin", "sort", "render_fwd", "render_bwd"]

    def ev():
        return torch.cuda.Event(enable_timing=True)

    def frame(k, cam, j, with_bwd, rec, staged):
        # camera k on stream j with stream j's buffers (the caller makes streams[j] current);
        # staged: an event between the stages for the per-stage breakdown (each costs the
        # stream a few microseconds, so the throughput runs go without them)
        rz = rzs[j]
        e = [ev() for _ in range(6)] if staged else None

        def mark(i):
            if staged:
                e[i].record(streams[j])

        mark(0)
        raster.project(means, scales, quats, opac, sh, sc.sh_degree, cam, rz.proj)
        mark(1)
        st, P = raster.bin_tiles(rz.proj, cam, rz.keys, rz.vals, rz.workspace, digit_counts=rz.digit_counts)
        assert st == raster.GS_OK
        mark(2)
        in_tmp = raster.sort_ids(P, tiles, rz.keys, rz.vals, rz.keys_tmp, rz.vals_tmp, ranges[k], rz.workspace,
                                 orders[k], digit_counts=rz.digit_counts)
        sv = rz.vals_tmp if in_tmp else rz.vals
        mark(3)
        raster.render_fwd(rz.proj, sv, ranges[k], cam, (0.0, 0.0, 0.0), images[k], finalT[k], ncon[k], orders[k])
        mark(4)
        if with_bwd:
            raster.render_bwd(means, scales, quats, opac, sh, sc.sh_degree, cam, rz.proj, sv, ranges[k],
                              (0.0, 0.0, 0.0), finalT[k], ncon[k], dLs[k], grads[j], accums[j], denoms[j],
                              orders[k])
            mark(5)
        rec.append((e, with_bwd, P))

    def run(steps, with_bwd, ns=1, staged=False, kern=None):
        """Times `steps` steps, camera k of a step on stream k mod ns.  With kern (single
        stream only) the library brackets every launch of that kernel with HIP events on
        its stream."""
        recs = []
        assert kern is None or ns == 1
        if kern:
            assert raster.kernel_timer_start(kern) == raster.GS_OK
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            for k, cam in enumerate(cams):
                j = k % ns
                with torch.cuda.stream(streams[j]):
                    frame(k, cam, j, with_bwd, recs, staged)
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        launches, kms = 0, 0.0
        if kern:
            st, launches, kms = raster.kernel_timer_stop()
            assert st == raster.GS_OK and launches == len(recs), (st, launches)
        times = {s: [] for s in stages}
        for e, wb, _ in recs:
            if e is None:
                continue
            for i, s in enumerate(stages[:4]):
                times[s].append(e[i].elapsed_time(e[i + 1]))
            if wb:
                times["render_bwd"].append(e[4].elapsed_time(e[5]))
        if kern:
            times[kern] = [kms / launches] if launches else []
        return t1 - t0, times, [p for _, _, p in recs]

    if args.profile:
        # a plain copy of known size: 1 GiB read + 1 GiB written, for counter calibration
        a = torch.empty(1 << 28, dtype=torch.float32, device=dev).fill_(1.0)
        b = torch.empty_like(a)
        b.copy_(a)
        torch.cuda.synchronize()
        del a, b
        args.no_cpu_baseline = True
    frames = args.steps * len(cams)
    overlap = NS > 1 and not args.profile
    log("warm-up")
    run(args.warmup, True)
    if overlap:
        run(args.warmup, True, NS)
        log(f"timed: {args.steps} steps x {len(cams)} cameras, forward + backward, {NS} streams")
        secs_o, _, _ = run(args.steps, True, NS)
        log(f"timed: forward only, {NS} streams")
        secs_fo, _, _ = run(args.steps, False, NS)
    log(f"timed: {args.steps} steps x {len(cams)} cameras, forward + backward, one stream")
    secs, times_t, pairs = run(args.steps, True, kern="k_render_bwd")
    log("timed: forward only, one stream")
    secs_f, times_f, _ = run(args.steps, False, kern="k_render_fwd")
    single = {"frames_per_s": round(frames / secs, 2), "forward_only_frames_per_s": round(frames / secs_f, 2),
              "ms_per_step": round(1e3 * secs / args.steps, 3)}
    if overlap:
        secs, secs_f = secs_o, secs_fo
    value = frames / secs
    fwd_fps = frames / secs_f
    log("timed: forward only, projection kernel")
    _, times_p, _ = run(max(1, args.steps // 2), False, kern="k_project")
    kernel_ms = {"k_render_bwd": times_t["k_render_bwd"][0], "k_render_fwd": times_f["k_render_fwd"][0],
                 "k_project": times_p["k_project"][0]}
    # per-stage breakdown: a separate pass with events between the stages
    log("stage breakdown")
    _, times, _ = run(max(1, args.steps // 2), True, staged=True)

    # algorithmic work per launch (camera-averaged) for the roofline
    P_mean = float(np.mean(pairs))
    K = (sc.sh_degree + 1) ** 2
    counts = [work_counts(cam, ranges[k], ncon[k], finalT[k]) for k, cam in enumerate(cams)]
    evals = float(np.mean([c[0] for c in counts]))
    walk = float(np.mean([c[1] for c in counts]))
    work = stage_work(N, K, P_mean, tiles, evals, walk, W * H, with_bwd=True)
    algo = {
        "project": ("hbm", work["project"][0]),
        "bin": ("hbm", work["bin"][0]),
        "sort": ("hbm", work["sort"][0]),
        "render_fwd": ("alu", work["render_fwd"][1]),
        "render_bwd": ("alu", work["render_bwd"][1]),
    }
    avg = {s: float(np.mean(times[s])) for s in stages if times[s]}

    def roof(work_kind, ms):
        bound, work = work_kind
        if bound == "hbm":
            ach = work / (ms * 1e-3) / 1e9
            return {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                    "frac": round(ach / HBM_PEAK_GBS, 4)}
        ach = work / (ms * 1e-3) / 1e12
        return {"bound": "alu", "achieved": round(ach, 2), "peak": round(VALU_PEAK_TOPS, 1),
                "unit": "Tlane-op/s", "frac": round(ach / VALU_PEAK_TOPS, 4)}

    # stages are whole entry points (several kernels for bin, sort and render_bwd); the
    # roofline object is for the single kernel that takes the most time, k_render_bwd
    stage_report = {s: dict(ms=round(avg[s], 4), **roof(algo[s], avg[s])) for s in algo}
    kernel_stage = {"k_render_bwd": "render_bwd", "k_render_fwd": "render_fwd", "k_project": "project"}
    kernel_report = {k: dict(ms=round(v, 4), **roof(algo[kernel_stage[k]], v)) for k, v in kernel_ms.items()}
    roof_dom = dict(kernel_report["k_render_bwd"], kernel="k_render_bwd", launches_timed=frames,
                    traffic=traffic_bytes("k_render_bwd"))

    log("memory ceilings")
    ceil = ceilings(raster, rzs[0], means, scales, quats, opac, sh, sc.sh_degree, cams[0], tiles, dev)

    log("densify")
    accum, denom = sum(accums), sum(denoms)  # every stream's cameras
    dens = densify_measure(raster, means, scales, quats, opac, sh, sc.sh_degree, accum, denom, stream,
                           with_oracle=not args.no_cpu_baseline)

    log("adam")
    adam = adam_measure(raster, dev, with_oracle=not args.no_cpu_baseline)
    log("quantised SH projection")
    qsh = qsh_measure(raster, means, scales, quats, opac, sh, sc.sh_degree, cams, rz.proj)

    cpu = None
    if not args.no_cpu_baseline:
        log("float64 oracle on the host cores")
        cpu = cpu_baseline(sc, cams, [d.cpu().numpy() for d in dLs], args.cpu_budget)

    configs = None
    if not args.profile and not args.no_configs:
        del rz, rzs, grads, accums, denoms, accum, denom, images, finalT, ncon, ranges, orders, dLs
        del means, scales, quats, opac, sh
        torch.cuda.empty_cache()
        configs = config_report(args, raster, scenes, dev, sc, cams)

    line = {
        "metric": "frames/s + Mpixels/s fwd(+bwd) at 1M SH3 Gaussians 1080p; % HBM/VALU peak",
        "value": round(value, 2),
        "unit": "frames/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(1e3 * secs / args.steps, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": WORKLOAD, "gaussians": N, "sh_degree": 3, "width": W, "height": H,
                   "cameras_per_step": len(cams), "step": "forward+backward per camera",
                   "streams": NS if overlap else 1, "mean_pairs_per_frame": int(P_mean)},
        "mpixels_per_s": round(value * W * H / 1e6, 1),
        "forward_only": {"frames_per_s": round(fwd_fps, 2), "mpixels_per_s": round(fwd_fps * W * H / 1e6, 1)},
        "single_stream": single,
        "stages": stage_report,
        "stages_timing": "separate single-stream forward+backward pass with an event between stages",
        "kernels_timing": "library kernel timer over the single-stream timed loops",
        "kernels": kernel_report,
        "evaluations_per_frame": int(evals),
        "contributor_walk_per_frame": int(walk),
        "roofline": roof_dom,
        "ceilings": ceil,
        "cpu_baseline": cpu,
        "densify": dens,
        "adam": adam,
        "project_qsh": qsh,
        "configs": configs,
    }
    print(json.dumps(line), flush=True)


def work_counts(cam, ranges, n_contrib, final_T):
    """(evaluations, contributor walk) of one frame: a pixel evaluates its tile's list up to
    its stop (the whole list when it never stops); the reverse walk visits n_contrib entries."""
    H, W = cam.height, cam.width
    lens = (ranges[:, 1] - ranges[:, 0]).cpu().numpy()
    tl = lens.reshape(cam.tiles_y, cam.tiles_x).repeat(16, 0).repeat(16, 1)[:H, :W]
    nc = n_contrib.cpu().numpy().astype(np.int64)
    stopped = final_T.cpu().numpy() < TMIN
    return float(np.where(stopped, nc, tl).sum()), float(nc.sum())


def stage_work(N, K, P, tiles, evals, walk, pixels, with_bwd):
    """Algorithmic work per stage of one frame: {stage: (HBM bytes, VALU lane-op slots)}.
    N Gaussians with K SH coefficients per channel, P pairs, `tiles` tiles, `pixels` pixels;
    `evals` and `walk` as in work_counts.  Every Gaussian is counted as visible where that
    bounds the binning work."""
    V = float(N)
    # digit passes left to gs_sort_keys after the emission's own pass over the tile's low byte
    tile_bits = max(1, math.ceil(math.log2(max(tiles, 2))))
    passes = max(0, math.ceil((32 + tile_bits - 40) / 8))
    w = {
        # inputs; record, depth, rect, count, clamp byte and the 32-byte tile record
        "project": (N * (12 + 12 + 16 + 4 + 12 * K) + N * (48 + 4 + 8 + 4 + 1 + 32), 0.0),
        # count (4 B/G), compaction (8 read + 8 written per visible), depth sort (4 passes of
        # 16 B per visible + 4 B histogram), the depth-ordered gather (20 B per visible),
        # pairs written (12 B each)
        "bin": (4 * N + 16 * V + (4 * 16 + 4) * V + 20 * V + 12 * P, 0.0),
        # gs_sort_ids: 24 B/pair per pass (keys and ids read and written) except the last,
        # which writes the ids only (16 B/pair), and the ranges written (16 B/tile); the
        # digit counts come from the binning and the last pass records the ranges, so there
        # is no counting read and no read of the sorted keys
        "sort": ((24 * passes - 8 if passes else 0) * P + 16 * tiles, 0.0),
        # list entries read once per tile; colour, transmittance and count written per pixel
        "render_fwd": (4 * P + 20 * pixels, OPS_PER_EVAL_FWD * evals),
    }
    if with_bwd:
        # upstream gradient, transmittance and count read per pixel; list entries once per
        # tile; the screen-space gradient block cleared (40 B/G)
        w["render_bwd"] = (20 * pixels + 4 * P + 40 * N, OPS_PER_EVAL_BWD * walk)
        # inputs, count, clamp byte and screen-space gradient read; parameter gradients
        # written; densification statistics read and written
        w["project_bwd"] = (N * (12 + 12 + 16 + 12 * K + 4 + 1 + 40) + N * (12 + 12 + 16 + 12 * K) + 2 * 12 * N, 0.0)
    return w


def frame_bound_ms(work, hbm_gbs):
    """Lower bound of a frame: each stage takes at least the longer of its bytes at `hbm_gbs`
    and its lane-op slots at the VALU peak; the stages run one after another."""
    return 1e3 * sum(max(b / (hbm_gbs * 1e9), a / (VALU_PEAK_TOPS * 1e12)) for b, a in work.values())


def copy_bandwidth(dev, reps=5):
    """GB/s of a 1 GiB device-to-device copy (1 GiB read + 1 GiB written), median of `reps`."""
    import torch

    a = torch.empty(1 << 28, dtype=torch.float32, device=dev).fill_(1.0)
    b = torch.empty_like(a)
    b.copy_(a)
    ts = []
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        b.copy_(a)
        e1.record()
        torch.cuda.synchronize()
        ts.append(e0.elapsed_time(e1))
    del a, b
    torch.cuda.empty_cache()
    return 2 * (1 << 30) / (float(np.median(ts)) * 1e-3) / 1e9


def config_frames(raster, scenes, dev, sc, cams, dLs, nframes, warm=3):
    """Per camera: the median wall time of `nframes` frames, each project -> bin (with the
    pair-count read-back) -> sort -> composite (-> backward when `dLs` is given), bracketed
    by device synchronisations; plus the frame's pairs and work counts."""
    import torch

    base = torch.cuda.memory_allocated(dev)
    torch.cuda.reset_peak_memory_stats(dev)
    means, scales, quats, opac, sh = raster.scene_to_device(sc, dev)
    rz = raster.Rasterizer(means, scales, quats, opac, sh, sc.sh_degree)
    N, L = sc.n, sc.sh_degree
    with_bwd = dLs is not None
    grads = raster.alloc_grads(N, L, dev) if with_bwd else None
    accum = torch.zeros((N, 2), dtype=torch.float32, device=dev) if with_bwd else None
    denom = torch.zeros(N, dtype=torch.int32, device=dev) if with_bwd else None
    out = []
    for k, cam in enumerate(cams):
        rz.forward(cam)  # sizes the pair buffers
        H, W, tiles = cam.height, cam.width, cam.num_tiles
        rg = torch.empty((tiles, 2), dtype=torch.int64, device=dev)
        order = torch.empty(tiles, dtype=torch.int32, device=dev)
        img = torch.empty((3, H, W), dtype=torch.float32, device=dev)
        fT = torch.empty((H, W), dtype=torch.float32, device=dev)
        nc = torch.empty((H, W), dtype=torch.int32, device=dev)
        dL = torch.from_numpy(dLs[k]).to(dev) if with_bwd else None
        ts, Ps = [], []
        for f in range(warm + nframes):
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            raster.project(means, scales, quats, opac, sh, L, cam, rz.proj)
            st, P = raster.bin_tiles(rz.proj, cam, rz.keys, rz.vals, rz.workspace, digit_counts=rz.digit_counts)
            assert st == raster.GS_OK
            in_tmp = raster.sort_ids(P, tiles, rz.keys, rz.vals, rz.keys_tmp, rz.vals_tmp, rg, rz.workspace, order,
                                     digit_counts=rz.digit_counts)
            sv = rz.vals_tmp if in_tmp else rz.vals
            raster.render_fwd(rz.proj, sv, rg, cam, (0.0, 0.0, 0.0), img, fT, nc, order)
            if with_bwd:
                raster.render_bwd(means, scales, quats, opac, sh, L, cam, rz.proj, sv, rg, (0.0, 0.0, 0.0), fT, nc,
                                  dL, grads, accum, denom, order)
            torch.cuda.synchronize()
            if f >= warm:
                ts.append(time.perf_counter() - t0)
                Ps.append(P)
        evals, walk = work_counts(cam, rg, nc, fT)
        out.append(dict(ms=1e3 * float(np.median(ts)), P=int(Ps[-1]), evals=evals, walk=walk, cam=cam))
    peak = torch.cuda.max_memory_allocated(dev) - base
    del rz, means, scales, quats, opac, sh, grads, accum, denom
    torch.cuda.empty_cache()
    return out, peak


def oracle_frame(sc, cam, dL, budget, round_tiles=100):
    """Seconds of one frame of the float64 oracle: projection, binning, sort and ranges on all
    Gaussians (and the projection backward when `dL` is given), then compositing (forward, and
    backward with `dL`) on rounds of `round_tiles` random tiles until `budget` seconds have
    gone into the frame or every tile is done; the compositing time is scaled to the frame."""
    import oracle

    W, H = cam.width, cam.height
    t0 = time.perf_counter()
    proj = oracle.project(sc, cam)
    keys, vals = oracle.emit_projected(proj, cam.tiles_x)
    skeys, svals = oracle.sort_pairs(keys, vals)
    ranges = oracle.tile_ranges(skeys, cam.num_tiles)
    rec = oracle.records(proj)
    if dL is not None:
        oracle.project_bwd(sc, cam, np.zeros((sc.n, 10)))  # its cost does not depend on the values
        dL = dL.astype(np.float64)
    t_fixed = time.perf_counter() - t0
    tiles = np.random.default_rng(0).permutation(cam.num_tiles)
    done, npix, t_sample = 0, 0, 0.0
    while done < tiles.size and (done == 0 or time.perf_counter() - t0 < budget):
        pix = []
        for t in tiles[done:done + round_tiles]:
            tx, ty = t % cam.tiles_x, t // cam.tiles_x
            ys = np.arange(ty * 16, min(ty * 16 + 16, H))
            xs = np.arange(tx * 16, min(tx * 16 + 16, W))
            pix.append((ys[:, None] * W + xs[None, :]).reshape(-1))
        pix = np.concatenate(pix)
        t1 = time.perf_counter()
        oracle.render_pixels(W, H, (0, 0, 0), rec, svals, ranges, pix)
        if dL is not None:
            oracle.render_bwd(W, H, (0, 0, 0), rec, svals, ranges, sc.n, dL, pix=pix)
        t_sample += time.perf_counter() - t1
        done = min(done + round_tiles, tiles.size)
        npix += pix.shape[0]
    return t_fixed + t_sample * (W * H / npix), f"{done}/{tiles.size} tiles"


def host_cpu():
    """(logical CPUs usable by this process, CPU model name)."""
    try:
        usable = len(os.sched_getaffinity(0))
    except AttributeError:
        usable = os.cpu_count()
    model = None
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return usable, model


def config_report(args, raster, scenes, dev, sc3, cams3):
    """frames/s and Mpixels/s of every configuration (median of `--frames` frames per camera,
    each project -> bin with the P read-back -> sort -> composite; configuration 5 adds the
    backward), with the whole-frame roofline fraction against the spec peaks and against the
    copy bandwidth measured here, and the float64 oracle's seconds per frame with every host
    thread and with one."""
    import torch

    import oracle

    copy_gbs = copy_bandwidth(dev)
    threads = oracle.num_threads()
    usable, model = host_cpu()
    specs = [("tiny_1k_sh0_64", False), ("spheres_100k_sh3_800", False), ("aniso_1m_sh3_1080p_8cam", False),
             ("aniso_10m_sh3_1080p", False), ("aniso_1m_sh3_720p_bwd", True)]
    rep = {"copy_gbs": round(copy_gbs, 1), "frames_per_camera": args.frames,
           "timing": "median wall time per frame between device synchronisations, pair-count read-back included",
           "roofline": "sum over stages of max(HBM bytes / rate, VALU lane-op slots / 78.6 T/s) / measured time",
           "oracle_threads": threads, "host_cpus": usable, "host_cpu_model": model, "per_config": {}}
    for name, with_bwd in specs:
        log(f"configuration {name}")
        if name == "aniso_1m_sh3_1080p_8cam":
            sc, cams, extra = sc3, cams3, {}
        else:
            sc, cams, extra = scenes.workload(name)
        dLs = None
        if with_bwd:
            # upstream gradient sign(render - target), from a forward pass of the GPU path
            means, scales, quats, opac, sh = raster.scene_to_device(sc, dev)
            rz = raster.Rasterizer(means, scales, quats, opac, sh, sc.sh_degree)
            img = rz.forward(cams[0])["image"]
            dLs = [torch.sign(img - torch.from_numpy(extra["target"]).to(dev)).contiguous().cpu().numpy()]
            del rz, means, scales, quats, opac, sh, img
            torch.cuda.empty_cache()
        per_cam, peak = config_frames(raster, scenes, dev, sc, cams, dLs, args.frames)
        K = (sc.sh_degree + 1) ** 2
        cams_out = []
        for c in per_cam:
            cam = c["cam"]
            work = stage_work(sc.n, K, c["P"], cam.num_tiles, c["evals"], c["walk"], cam.width * cam.height, with_bwd)
            fps = 1e3 / c["ms"]
            cams_out.append({"ms": round(c["ms"], 4), "frames_per_s": round(fps, 1),
                             "mpixels_per_s": round(fps * cam.width * cam.height / 1e6, 1), "pairs": c["P"],
                             "frac_spec": round(frame_bound_ms(work, HBM_PEAK_GBS) / c["ms"], 4),
                             "frac_copy": round(frame_bound_ms(work, copy_gbs) / c["ms"], 4)})
        cam = cams[0]
        mean_ms = float(np.mean([c["ms"] for c in cams_out]))
        entry = {"gaussians": sc.n, "sh_degree": sc.sh_degree, "width": cam.width, "height": cam.height,
                 "step": "forward+backward" if with_bwd else "forward", "frames_per_s": round(1e3 / mean_ms, 1),
                 "mpixels_per_s": round(1e3 / mean_ms * cam.width * cam.height / 1e6, 1),
                 "frac_spec": round(float(np.mean([c["frac_spec"] for c in cams_out])), 4),
                 "frac_copy": round(float(np.mean([c["frac_copy"] for c in cams_out])), 4),
                 "pairs": int(np.mean([c["pairs"] for c in cams_out])), "peak_alloc_bytes": int(peak)}
        if len(cams_out) > 1:
            entry["cameras"] = cams_out
        # the oracle on the first camera: every tile for the small scenes, sampled tiles beyond;
        # at 10M with every host thread by default (about half a minute), single-threaded too
        # with --oracle-10m
        big = name == "aniso_10m_sh3_1080p"
        if not args.no_cpu_baseline:
            orc = {}
            for th in ((threads, 1) if not big or args.oracle_10m else (threads,)):
                oracle.set_threads(th)
                secs, desc = oracle_frame(sc, cam, dLs[0] if with_bwd else None, budget=8.0)
                orc[f"{th}_threads"] = {"s_per_frame": round(secs, 3), "tiles": desc,
                                        "gpu_speedup": round(secs * 1e3 / mean_ms, 1)}
            oracle.set_threads(threads)
            entry["oracle"] = orc
        rep["per_config"][name] = entry
        del sc
    return rep


# HBM bytes per launch of k_render_bwd on this workload (camera average), from two rocprofv3
# counter runs of `bench.py --profile` (FETCH_SIZE, then WRITE_SIZE), each scaled by the
# ratio of the known bytes of a 1 GiB device copy to what the same counter read for that
# copy.  Valid only for the kernel source it was taken on: the digest covers the
# compositing kernels' source and the headers they include.
TRAFFIC = {"k_render_bwd": {"bytes": 545432989, "source_digest": "145902fd7d560dc5"}}


def kernel_source_digest():
    import hashlib

    h = hashlib.sha256()
    for f in ("gs_render.hip", "gs_device.h", "gs_wave.h"):
        with open(os.path.join(ROOT, "tile_differentiable_rasterizer_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def traffic_bytes(kernel):
    t = TRAFFIC.get(kernel)
    if not t or t["source_digest"] != kernel_source_digest():
        return None
    return t["bytes"]


def ceilings(raster, rz, means, scales, quats, opac, sh, L, cam, tiles, dev, reps=20):
    """The projection kernel and the pair sort's digit pass beside kernels that perform only
    their loads and stores in their layouts (gs_measure.h), on the first camera."""
    import torch

    def per_launch_ms(f):
        f()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(reps):
            f()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / reps

    N = means.shape[0]
    K = (L + 1) ** 2
    proj_io = raster.alloc_projected(N, dev)
    t_k1 = per_launch_ms(lambda: raster.project(means, scales, quats, opac, sh, L, cam, rz.proj))
    t_k1io = per_launch_ms(lambda: raster.measure_project_io(means, scales, quats, opac, sh, L, proj_io))
    k1_bytes = N * (44 + 12 * K + 97)  # the loads and stores both kernels make (as in stage_work)
    del proj_io

    # the pairs of the camera as the binning leaves them, and every pair's sorted position
    raster.project(means, scales, quats, opac, sh, L, cam, rz.proj)
    st, P = raster.bin_tiles(rz.proj, cam, rz.keys, rz.vals, rz.workspace, digit_counts=rz.digit_counts)
    assert st == raster.GS_OK
    keys0, vals0, dc = rz.keys[:P].clone(), rz.vals[:P].clone(), rz.digit_counts.clone()
    ranges = torch.empty((tiles, 2), dtype=torch.int64, device=dev)
    k, v = keys0.clone(), torch.arange(P, dtype=torch.int32, device=dev)
    kt, vt = torch.empty_like(k), torch.empty_like(v)
    in_tmp = raster.sort_keys(P, tiles, k, v, kt, vt, ranges, rz.workspace, leave_in_tmp=True, digit_counts=dc)
    perm = (vt if in_tmp else v).long()
    dest = torch.empty(P, dtype=torch.int32, device=dev)
    dest[perm] = torch.arange(P, dtype=torch.int32, device=dev)
    # the order in which a digit pass writes: its partitions of 4096 pairs, each grouped by
    # the pass's digit (the tile bits above the low byte), stably
    order = torch.argsort((torch.arange(P, device=dev) // 4096) * 256 + ((keys0 >> 40) & 255), stable=True)
    kr, vr, dr = keys0[order].contiguous(), vals0[order].contiguous(), dest[order].contiguous()
    del k, v, kt, vt, perm, order, dest
    out = torch.empty(P, dtype=torch.int32, device=dev)
    t_sio = per_launch_ms(lambda: raster.measure_scatter_io(kr, vr, dr, out))
    # the pass itself, as the frames run it (gs_sort_ids with the binning's digit counts)
    assert raster.kernel_timer_start("k_onesweep_u64") == raster.GS_OK
    for _ in range(reps):
        rz.keys[:P].copy_(keys0)
        rz.vals[:P].copy_(vals0)
        raster.sort_ids(P, tiles, rz.keys, rz.vals, rz.keys_tmp, rz.vals_tmp, ranges, rz.workspace, None,
                        digit_counts=dc)
    st, launches, ms = raster.kernel_timer_stop()
    assert st == raster.GS_OK and launches > 0
    passes = launches / reps
    t_pass = ms / launches
    del kr, vr, dr, out, keys0, vals0

    def entry(kernel_ms, io_ms, kernel_bytes, io_bytes):
        return {"kernel_ms": round(kernel_ms, 4), "io_ms": round(io_ms, 4),
                "kernel_gbs": round(kernel_bytes / (kernel_ms * 1e-3) / 1e9, 1),
                "io_gbs": round(io_bytes / (io_ms * 1e-3) / 1e9, 1),
                "kernel_frac_of_hbm_peak": round(kernel_bytes / (kernel_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                "io_frac_of_hbm_peak": round(io_bytes / (io_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                "kernel_time_over_io_time": round(kernel_ms / io_ms, 3)}

    return {
        "what": "each kernel beside a kernel with only its loads and stores in the same layout "
                "(gs_measure_project_io / gs_measure_scatter_io), first camera, back-to-back launches",
        "k_project": dict(entry(t_k1, t_k1io, k1_bytes, k1_bytes), bytes=k1_bytes),
        "k_onesweep_u64": dict(entry(t_pass, t_sio, 16 * P, 20 * P), pairs=P, passes_per_sort=passes,
                               note="the ids-only pass reads key and id and writes the id (16 B per pair); "
                                    "the ceiling kernel also reads the destination (20 B per pair)"),
    }


def densify_measure(raster, means, scales, quats, opac, sh, L, accum, denom, stream, with_oracle, reps=5):
    """gs_densify on the statistics the timed steps accumulated (every camera's backward).
    Thresholds from those statistics: the 90th percentile of the seen Gaussians' average
    gradient, the median largest scale; split into 2 children at 1/1.6 scale; prune below
    opacity 0.005.  Times the whole call (count, scan, count read-back, emission) with HIP
    events and the emission kernel with the library's kernel timer; the emission's rate is
    its algorithmic bytes over its time."""
    import torch

    a = accum.cpu().numpy()
    d = denom.cpu().numpy()
    seen = d > 0
    avg = a[seen, 0] / d[seen]
    thr = float(np.quantile(avg, 0.9)) if avg.size else 1.0
    smax = scales.max(dim=1).values
    sthr = float(smax.median())
    params = raster.densify_params(thr, sthr, use_abs=False, split_n=2, split_shrink=1.6, min_opacity=0.005)
    gen = torch.Generator(device=means.device).manual_seed(17)
    normals = torch.randn((means.shape[0], 2, 3), generator=gen, device=means.device)
    out = raster.densify(means, scales, quats, opac, sh, L, accum, denom, normals, params)  # sizes the outputs
    n, m = int(means.shape[0]), int(out["n_out"])
    full = {k: v for k, v in out.items() if torch.is_tensor(v)}
    full = {k: v.new_empty((m,) + tuple(v.shape[1:])) for k, v in full.items()}
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    assert raster.kernel_timer_start("k_densify_emit") == raster.GS_OK
    e0.record(stream)
    for _ in range(reps):
        r = raster.densify(means, scales, quats, opac, sh, L, accum, denom, normals, params, out=full)
    e1.record(stream)
    torch.cuda.synchronize()
    st, launches, kms = raster.kernel_timer_stop()
    assert st == raster.GS_OK and launches == reps and r["n_out"] == m
    call_ms = e0.elapsed_time(e1) / reps
    emit_ms = kms / launches
    K = (L + 1) ** 2
    # children are the rows whose scales differ from their source's (scale / 1.6)
    child_rows = int((r["scales"] != scales[r["src"].long()]).any(dim=1).sum().item()) if m else 0
    n_split = child_rows // 2
    # emission: decisions (28 B per input), the kept inputs' rows, normals of split inputs,
    # every output row (centre, scales, quaternion, opacity, SH, source index)
    emit_bytes = n * (28 + 12 + 16 + 12 * K) + n_split * 2 * 12 + m * (12 + 12 + 16 + 4 + 12 * K + 4)
    ach = emit_bytes / (emit_ms * 1e-3) / 1e9
    res = {"n_in": n, "n_out": m, "grad_threshold": thr, "scale_threshold": sthr, "call_ms": round(call_ms, 4),
           "emit_ms": round(emit_ms, 4),
           "emit_roofline": {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                             "frac": round(ach / HBM_PEAK_GBS, 4), "bytes": int(emit_bytes)}}
    if with_oracle:
        import time as _t

        import oracle

        args = [x.cpu().numpy() for x in (means, scales, quats, opac, sh, accum, denom, normals)]
        t0 = _t.perf_counter()
        o = oracle.densify(*args, grad_threshold=thr, use_abs=False, scale_threshold=sthr, split_n=2,
                           split_shrink=1.6, min_opacity=0.005, max_scale=0.0)
        res["cpu_oracle_ms"] = round(1e3 * (_t.perf_counter() - t0), 1)
        res["matches_oracle_count"] = bool(o["n_out"] == m)
    return res


def qsh_measure(raster, means, scales, quats, opac, sh, L, cams, proj, reps=3):
    """gs_project against gs_project_qsh (q16, q8) on the bench scene and cameras, each timed
    with the library's kernel timer over `reps` passes of the 8 cameras; the rate is the
    algorithmic bytes (inputs with the SH at their stored width, plus the bounds, and the
    97 B of outputs) over the kernel time."""
    import torch

    N = int(means.shape[0])
    K = (L + 1) ** 2
    res = {}
    for bits in (0, 16, 8):
        if bits:
            codes, bounds = raster.quantize_sh(sh, L, bits)
        torch.cuda.synchronize()
        assert raster.kernel_timer_start("k_project") == raster.GS_OK
        for _ in range(reps):
            for cam in cams:
                if bits:
                    raster.project_qsh(means, scales, quats, opac, codes, bounds, bits, L, cam, proj)
                else:
                    raster.project(means, scales, quats, opac, sh, L, cam, proj)
        torch.cuda.synchronize()
        st, launches, kms = raster.kernel_timer_stop()
        assert st == raster.GS_OK and launches == reps * len(cams)
        ms = kms / launches
        sh_bytes = 12 * K if not bits else 3 * K * bits // 8 + 8 * (3 * K) / 256
        nbytes = N * (12 + 12 + 16 + 4 + sh_bytes + 48 + 4 + 8 + 4 + 1 + 32)
        ach = nbytes / (ms * 1e-3) / 1e9
        res["fp32" if not bits else f"q{bits}"] = {
            "ms": round(ms, 4), "sh_bytes_per_gaussian": round(sh_bytes, 2),
            "roofline": {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": round(ach / HBM_PEAK_GBS, 4)}}
    return res


def adam_measure(raster, dev, with_oracle, gaussians=5_000_000, reps=5):
    """gs_adam_q16 at the size of the pages' fused-optimiser figure: 5M SH3 Gaussians, 59
    float32 parameters each (centre 3, scales 3, quaternion 4, opacity 1, SH 48), one flat
    array of units.  Synthetic parameters N(0, 1) and gradients N(0, 1e-3) from a seeded
    generator.  Times `reps` steps with the library's kernel timer; the rate is the
    algorithmic bytes (per unit: parameter, gradient and state read, parameter and state
    written; 32 B of bounds per 256 units) over the kernel time."""
    import torch

    U = gaussians * 59
    gen = torch.Generator(device=dev).manual_seed(21)
    params = torch.randn(U, generator=gen, device=dev)
    grads = torch.randn(U, generator=gen, device=dev) * 1e-3
    state, bounds = raster.adam_state(U, dev)
    raster.adam_q16(params, grads, state, bounds, lr=1e-3, step=1)
    torch.cuda.synchronize()
    assert raster.kernel_timer_start("k_adam_q16") == raster.GS_OK
    for t in range(2, reps + 2):
        raster.adam_q16(params, grads, state, bounds, lr=1e-3, step=t)
    torch.cuda.synchronize()
    st, launches, kms = raster.kernel_timer_stop()
    assert st == raster.GS_OK and launches == reps
    ms = kms / launches
    nbytes = U * (4 + 4 + 4 + 4 + 4) + ((U + 255) // 256) * 32
    ach = nbytes / (ms * 1e-3) / 1e9
    res = {"gaussians": gaussians, "units": U, "ms": round(ms, 4),
           "roofline": {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                        "frac": round(ach / HBM_PEAK_GBS, 4), "bytes": int(nbytes)},
           "pages_context_ms": {"before": 13.8, "after": 8.5, "note": "5M points, hardware unspecified"}}
    del state, bounds
    torch.cuda.empty_cache()
    # the same step with the parameters packed too (gs_adam_fpbo): per unit the three codes
    # read and written (6 B each way), the gradient read and the decoded float32 parameter
    # written for the renderer; 24 B of bounds per 256 units read and written
    pstate, pbounds = raster.fpbo_pack(params)
    raster.adam_fpbo(U, pstate, pbounds, grads, params, lr=1e-3, step=1)
    torch.cuda.synchronize()
    assert raster.kernel_timer_start("k_adam_fpbo") == raster.GS_OK
    for t in range(2, reps + 2):
        raster.adam_fpbo(U, pstate, pbounds, grads, params, lr=1e-3, step=t)
    torch.cuda.synchronize()
    st, launches, kms = raster.kernel_timer_stop()
    assert st == raster.GS_OK and launches == reps
    ms = kms / launches
    nbytes = U * (6 + 4 + 6 + 4) + ((U + 255) // 256) * 48
    ach = nbytes / (ms * 1e-3) / 1e9
    res["packed_params"] = {
        "call": "gs_adam_fpbo (parameters and both moments as 16-bit codes, decoded parameters written)",
        "ms": round(ms, 4), "state_bytes_per_unit": 6,
        "roofline": {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(ach / HBM_PEAK_GBS, 4), "bytes": int(nbytes)}}
    del params, grads, pstate, pbounds
    torch.cuda.empty_cache()
    if with_oracle:
        import time as _t

        import oracle.adam as A

        n = 2_000_000
        rng = np.random.default_rng(21)
        p = rng.normal(size=n).astype(np.float32)
        g = (rng.normal(size=n) * 1e-3).astype(np.float32)
        t0 = _t.perf_counter()
        A.adam_q16(p, g, np.zeros(n, np.uint32), np.zeros(((n + 255) // 256, 4), np.float32), lr=1e-3, beta1=0.9,
                   beta2=0.999, eps=1e-8, step=1)
        res["cpu_oracle_ms"] = round(1e3 * (_t.perf_counter() - t0) * U / n, 1)
        res["cpu_oracle_sample"] = f"one step on {n} units, scaled to {U}"
        st0, bd0 = A.fpbo_pack(p)
        t0 = _t.perf_counter()
        A.adam_fpbo(st0, bd0, g, lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, step=1)
        res["packed_params"]["cpu_oracle_ms"] = round(1e3 * (_t.perf_counter() - t0) * U / n, 1)
    return res


def cpu_baseline(sc, cams, dLs, budget):
    """The float64 oracle on the host, camera after camera until about `budget` seconds have
    been spent: per camera, projection, binning, sort and projection backward on all
    Gaussians, and compositing forward + backward on rounds of 400 random tiles (the whole
    frame when the budget allows; otherwise the rounds done, scaled to the frame).
    Returns frames/s over the cameras measured."""
    import oracle

    t_start = time.perf_counter()
    per_frame, desc = [], []
    for cam, dL in zip(cams, dLs):
        left = budget - (time.perf_counter() - t_start)
        if per_frame and left <= 0:
            break
        secs, d = oracle_frame(sc, cam, dL, budget=left, round_tiles=400)
        per_frame.append(secs)
        desc.append(d)
    cam = cams[0]
    return {"value": round(len(per_frame) / sum(per_frame), 5), "unit": "frames/s", "cores": oracle.num_threads(),
            "kind": "oracle",
            "sample": f"{len(per_frame)} orbit camera(s): projection, binning, sort and projection backward on all "
                      f"{sc.n} Gaussians; compositing forward+backward on random 16x16 tiles ({', '.join(desc)}), "
                      f"scaled to {cam.width}x{cam.height} where a frame was not covered",
            "seconds_measured": round(time.perf_counter() - t_start, 2)}


if __name__ == "__main__":
    main()
