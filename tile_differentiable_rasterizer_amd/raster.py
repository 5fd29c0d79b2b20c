"""ctypes binding of libgsraster (the C ABI in include/gs_raster.h).

Argument marshalling only: torch provides device memory and the current stream; every
step of the computation runs in the HIP kernels behind the C ABI.  Importing this module
fails loudly when the library has not been built (there is no fallback).
"""
from __future__ import annotations

import ctypes as C
import os
import threading

import numpy as np
import torch

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libgsraster.so")

GS_OK, GS_ERR_INVALID_ARG, GS_ERR_CAPACITY, GS_ERR_OVERFLOW, GS_ERR_HIP, GS_ERR_WORKSPACE = range(6)
TILE = 16
REC_FLOATS = 12
GRAD_SCREEN = 10
TILE_DIGIT_COUNTS = 512  # GS_TILE_DIGIT_COUNTS
ROW_BLOCK = 256  # GS_ROW_BLOCK
ROWS_PER_BLOCK = 128  # GS_ROWS_PER_BLOCK

EXPORTS = ("gs_project", "gs_workspace_bytes", "gs_bin_tiles", "gs_sort_keys", "gs_sort_ids", "gs_render_fwd",
           "gs_render_bwd", "gs_densify", "gs_densify_workspace_bytes", "gs_adam_q16", "gs_fpbo_pack",
           "gs_adam_fpbo", "gs_quantize_sh",
           "gs_project_qsh", "gs_status_string")


class GsError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {lib().gs_status_string(status).decode()} (status {status})")


class GsCamera(C.Structure):
    _fields_ = [("R", C.c_float * 9), ("t", C.c_float * 3), ("fx", C.c_float), ("fy", C.c_float),
                ("cx", C.c_float), ("cy", C.c_float), ("width", C.c_int32), ("height", C.c_int32),
                ("near_z", C.c_float)]


class GsProjected(C.Structure):
    _fields_ = [("rec", C.c_void_p), ("depth", C.c_void_p), ("rect", C.c_void_p),
                ("n_tiles", C.c_void_p), ("clamp", C.c_void_p), ("runs", C.c_void_p), ("rows", C.c_void_p)]


class GsDensifyParams(C.Structure):
    _fields_ = [("grad_threshold", C.c_float), ("use_abs", C.c_int32), ("scale_threshold", C.c_float),
                ("split_n", C.c_int32), ("split_shrink", C.c_float), ("min_opacity", C.c_float),
                ("max_scale", C.c_float)]


class GsAdamParams(C.Structure):
    _fields_ = [("lr", C.c_float), ("beta1", C.c_float), ("beta2", C.c_float), ("eps", C.c_float),
                ("step", C.c_int64)]


class GsGrads(C.Structure):
    _fields_ = [("grad_screen", C.c_void_p), ("dmeans", C.c_void_p), ("dscales", C.c_void_p),
                ("dquats", C.c_void_p), ("dsh", C.c_void_p)]


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise ImportError(f"{_LIB_PATH} is not built; run __graft_entry__.build() "
                              "or python -m tile_differentiable_rasterizer_amd._build")
        L = C.CDLL(_LIB_PATH)
        vp, i64, i32, sz = C.c_void_p, C.c_int64, C.c_int32, C.c_size_t
        L.gs_project.argtypes = [i64, vp, vp, vp, vp, vp, i32, C.POINTER(GsCamera), GsProjected, vp]
        L.gs_workspace_bytes.argtypes = [i64, i64, i32]
        L.gs_workspace_bytes.restype = sz
        L.gs_bin_tiles.argtypes = [i64, GsProjected, C.POINTER(GsCamera), vp, vp, i64, C.POINTER(i64), vp, vp, sz, vp]
        L.gs_sort_keys.argtypes = [i64, i32, i32, vp, vp, vp, vp, vp, vp, vp, C.POINTER(i32), vp, sz, vp]
        L.gs_sort_keys_noalloc.argtypes = [i64, i32, i32, vp, vp, vp, vp, vp, vp, vp, C.POINTER(i32), vp]
        L.gs_sort_ids.argtypes = [i64, i32, i32, vp, vp, vp, vp, vp, vp, vp, C.POINTER(i32), vp, sz, vp]
        L.gs_render_fwd.argtypes = [i64, GsProjected, vp, vp, vp, C.POINTER(GsCamera), C.POINTER(C.c_float), vp,
                                    vp, vp, vp]
        L.gs_render_bwd.argtypes = [i64, vp, vp, vp, vp, vp, i32, C.POINTER(GsCamera), GsProjected, vp, vp, vp,
                                    C.POINTER(C.c_float), vp, vp, vp, GsGrads, vp, vp, vp]
        L.gs_densify_workspace_bytes.argtypes = [i64]
        L.gs_densify_workspace_bytes.restype = sz
        L.gs_densify.argtypes = [i64, vp, vp, vp, vp, vp, i32, vp, vp, vp, C.POINTER(GsDensifyParams), vp, vp, vp,
                                 vp, vp, vp, i64, C.POINTER(i64), vp, sz, vp]
        L.gs_adam_q16.argtypes = [i64, vp, vp, vp, vp, C.POINTER(GsAdamParams), vp]
        L.gs_fpbo_pack.argtypes = [i64, vp, vp, vp, vp]
        L.gs_adam_fpbo.argtypes = [i64, vp, vp, vp, vp, C.POINTER(GsAdamParams), vp]
        L.gs_quantize_sh.argtypes = [i64, vp, i32, i32, vp, vp, vp]
        L.gs_project_qsh.argtypes = [i64, vp, vp, vp, vp, vp, vp, i32, i32, C.POINTER(GsCamera), GsProjected, vp]
        for name in ("gs_project", "gs_bin_tiles", "gs_sort_keys", "gs_sort_ids", "gs_sort_keys_noalloc", "gs_render_fwd",
                     "gs_render_bwd", "gs_densify",
                     "gs_adam_q16", "gs_fpbo_pack", "gs_adam_fpbo", "gs_quantize_sh", "gs_project_qsh"):
            getattr(L, name).restype = i32
        L.gs_status_string.argtypes = [i32]
        L.gs_status_string.restype = C.c_char_p
        L.gs_kernel_timer_start.argtypes = [C.c_char_p]
        L.gs_kernel_timer_start.restype = i32
        L.gs_kernel_timer_stop.argtypes = [C.POINTER(i64), C.POINTER(C.c_double)]
        L.gs_kernel_timer_stop.restype = i32
        L.gs_measure_project_io.argtypes = [i64, vp, vp, vp, vp, vp, i32, GsProjected, vp]
        L.gs_measure_project_io.restype = i32
        L.gs_measure_scatter_io.argtypes = [i64, vp, vp, vp, vp, vp]
        L.gs_measure_scatter_io.restype = i32
        _lib = L
    return _lib


def kernel_timer_start(kernel):
    """Arm the library's event timer for one kernel ("k_project", "k_render_fwd",
    "k_render_bwd", "k_project_bwd", "k_densify_emit", "k_adam_q16", "k_adam_fpbo", "k_onesweep_u64");
    returns the status code."""
    return lib().gs_kernel_timer_start(kernel.encode())


def kernel_timer_stop():
    """Disarm the timer: (status, launches timed, summed device milliseconds)."""
    n, ms = C.c_int64(0), C.c_double(0.0)
    st = lib().gs_kernel_timer_stop(C.byref(n), C.byref(ms))
    return st, n.value, ms.value


def measure_project_io(means, scales, quats, opacities, sh, sh_degree: int, out: dict, stream=None):
    """gs_measure_project_io: the projection's loads and stores only (a memory ceiling);
    overwrites `out` with unspecified values."""
    _check(lib().gs_measure_project_io(means.shape[0], _ptr(means), _ptr(scales), _ptr(quats), _ptr(opacities),
                                       _ptr(sh), int(sh_degree), projected_struct(out), _stream(stream)),
           "gs_measure_project_io")


def measure_scatter_io(keys, vals, dest, out, stream=None):
    """gs_measure_scatter_io: out[dest[i]] = vals[i] + low word of keys[i] (a memory ceiling)."""
    _check(lib().gs_measure_scatter_io(keys.shape[0], _ptr(keys), _ptr(vals), _ptr(dest), _ptr(out),
                                       _stream(stream)), "gs_measure_scatter_io")


def _ptr(t):
    if t is None:
        return None
    return C.c_void_p(t.data_ptr())


def _stream(stream=None):
    s = stream if stream is not None else torch.cuda.current_stream()
    return C.c_void_p(s.cuda_stream)


def _check(status: int, where: str):
    if status != GS_OK:
        raise GsError(status, where)


def camera_struct(cam) -> GsCamera:
    """gs_camera from an object with R (3x3), t (3), fx, fy, cx, cy, width, height, near."""
    c = GsCamera()
    R = np.asarray(cam.R, dtype=np.float32).reshape(9)
    t = np.asarray(cam.t, dtype=np.float32).reshape(3)
    for i in range(9):
        c.R[i] = float(R[i])
    for i in range(3):
        c.t[i] = float(t[i])
    c.fx, c.fy, c.cx, c.cy = float(cam.fx), float(cam.fy), float(cam.cx), float(cam.cy)
    c.width, c.height = int(cam.width), int(cam.height)
    c.near_z = float(cam.near)
    return c


def _bg(bg):
    arr = (C.c_float * 3)(*[float(x) for x in bg])
    return arr


def alloc_projected(n: int, device="cuda") -> dict:
    return dict(rec=torch.empty((n, REC_FLOATS), dtype=torch.float32, device=device),
                depth=torch.empty(n, dtype=torch.float32, device=device),
                rect=torch.empty((n, 4), dtype=torch.int16, device=device),
                n_tiles=torch.empty(n, dtype=torch.int32, device=device),
                clamp=torch.empty(n, dtype=torch.uint8, device=device),
                runs=torch.empty((n, 8), dtype=torch.int32, device=device),
                rows=torch.empty((max(1, -(-n // ROW_BLOCK)) * ROWS_PER_BLOCK, 2), dtype=torch.int32, device=device))


def projected_struct(p: dict) -> GsProjected:
    return GsProjected(_ptr(p["rec"]), _ptr(p["depth"]), _ptr(p["rect"]), _ptr(p["n_tiles"]), _ptr(p["clamp"]),
                       _ptr(p["runs"]), _ptr(p["rows"]))


def project(means, scales, quats, opacities, sh, sh_degree: int, cam, out: dict | None = None, stream=None) -> dict:
    """gs_project.  Tensors: float32 CUDA, contiguous.  Returns the gs_projected buffers."""
    n = means.shape[0]
    if out is None:
        out = alloc_projected(n, means.device)
    camc = camera_struct(cam)
    _check(lib().gs_project(n, _ptr(means), _ptr(scales), _ptr(quats), _ptr(opacities), _ptr(sh), int(sh_degree),
                            C.byref(camc), projected_struct(out), _stream(stream)), "gs_project")
    return out


def workspace_bytes(n: int, pair_capacity: int, num_tiles: int) -> int:
    return int(lib().gs_workspace_bytes(n, pair_capacity, num_tiles))


_tls = threading.local()


def _pinned_count():
    """One page-locked int64 per thread for gs_bin_tiles' pair count."""
    t = getattr(_tls, "count", None)
    if t is None:
        t = _tls.count = torch.zeros(1, dtype=torch.int64, pin_memory=True)
    return t


def bin_tiles(proj: dict, cam, keys, vals, workspace, stream=None, digit_counts=None) -> tuple[int, int]:
    """gs_bin_tiles.  Returns (status, P); status is GS_OK or GS_ERR_CAPACITY.
    ``digit_counts`` (int64 [GS_TILE_DIGIT_COUNTS], optional) receives the tile-digit
    counts that sort_keys(digit_counts=...) takes in place of its own counting read."""
    n = proj["rec"].shape[0]
    camc = camera_struct(cam)
    P = _pinned_count()  # page-locked, so the call waits for the count copy alone
    cap = keys.shape[0] if keys is not None else 0
    if digit_counts is not None:
        assert digit_counts.numel() >= TILE_DIGIT_COUNTS and digit_counts.dtype == torch.int64
    st = lib().gs_bin_tiles(n, projected_struct(proj), C.byref(camc), _ptr(keys), _ptr(vals), cap,
                            C.cast(P.data_ptr(), C.POINTER(C.c_int64)), _ptr(digit_counts), _ptr(workspace),
                            workspace.numel() if workspace is not None else 0, _stream(stream))
    if st not in (GS_OK, GS_ERR_CAPACITY):
        _check(st, "gs_bin_tiles")
    return st, int(P[0])


def sort_keys(n_pairs: int, num_tiles: int, keys, vals, keys_tmp, vals_tmp, ranges, workspace, order=None,
              sorted_low_bits: int = 40, stream=None, leave_in_tmp: bool = False, digit_counts=None):
    """gs_sort_keys; ``order`` (int32 [num_tiles], optional) receives the longest-first tile order.

    ``sorted_low_bits`` = 40 for pairs from gs_bin_tiles (already ordered by tile low byte,
    then depth), 0 for arbitrary keys.  With ``leave_in_tmp`` the result stays where the
    last pass wrote it and the call returns True when that is keys_tmp/vals_tmp; otherwise
    the result is in keys/vals and the call returns False.  ``digit_counts``: per-pass digit
    counts of the keys (bin_tiles' for its pairs), or None to count them."""
    where = C.c_int32(-1)
    _check(lib().gs_sort_keys(n_pairs, num_tiles, int(sorted_low_bits), _ptr(keys), _ptr(vals), _ptr(keys_tmp),
                              _ptr(vals_tmp), _ptr(ranges), _ptr(order), _ptr(digit_counts),
                              C.byref(where) if leave_in_tmp else None,
                              _ptr(workspace), workspace.numel(), _stream(stream)), "gs_sort_keys")
    return bool(where.value == 1) if leave_in_tmp else False


def sort_ids(n_pairs: int, num_tiles: int, keys, vals, keys_tmp, vals_tmp, ranges, workspace, order=None,
             sorted_low_bits: int = 40, stream=None, digit_counts=None) -> bool:
    """gs_sort_ids: sort_keys that leaves the sorted ids and the ranges but not the sorted keys
    (the compositing calls read only those).  Returns True when the result is in
    keys_tmp/vals_tmp."""
    where = C.c_int32(-1)
    _check(lib().gs_sort_ids(n_pairs, num_tiles, int(sorted_low_bits), _ptr(keys), _ptr(vals), _ptr(keys_tmp),
                             _ptr(vals_tmp), _ptr(ranges), _ptr(order), _ptr(digit_counts), C.byref(where),
                             _ptr(workspace), workspace.numel(), _stream(stream)), "gs_sort_ids")
    return bool(where.value == 1)


def sort_keys_noalloc(n_pairs: int, num_tiles: int, keys, vals, keys_tmp, vals_tmp, ranges, order=None,
                      sorted_low_bits: int = 40, stream=None, leave_in_tmp: bool = False, digit_counts=None):
    """gs_sort_keys_noalloc: sort_keys without a workspace (the library's fixed per-GPU
    scratch; no allocation).  Returns the gs_status instead of raising, so that callers can
    tell a sort too large for the scratch (GS_ERR_WORKSPACE) from other errors; with
    ``leave_in_tmp``, also whether the result is in keys_tmp/vals_tmp."""
    where = C.c_int32(-1)
    st = lib().gs_sort_keys_noalloc(n_pairs, num_tiles, int(sorted_low_bits), _ptr(keys), _ptr(vals), _ptr(keys_tmp),
                                    _ptr(vals_tmp), _ptr(ranges), _ptr(order), _ptr(digit_counts),
                                    C.byref(where) if leave_in_tmp else None, _stream(stream))
    return (st, bool(where.value == 1)) if leave_in_tmp else st


def render_fwd(proj: dict, sorted_vals, ranges, cam, bg, image, final_T, n_contrib, order=None, stream=None):
    camc = camera_struct(cam)
    _check(lib().gs_render_fwd(proj["rec"].shape[0], projected_struct(proj), _ptr(sorted_vals), _ptr(ranges),
                               _ptr(order), C.byref(camc), _bg(bg), _ptr(image), _ptr(final_T), _ptr(n_contrib),
                               _stream(stream)), "gs_render_fwd")


def alloc_grads(n: int, sh_degree: int, device="cuda") -> dict:
    K = (sh_degree + 1) ** 2
    return dict(grad_screen=torch.empty((n, GRAD_SCREEN), dtype=torch.float32, device=device),
                dmeans=torch.empty((n, 3), dtype=torch.float32, device=device),
                dscales=torch.empty((n, 3), dtype=torch.float32, device=device),
                dquats=torch.empty((n, 4), dtype=torch.float32, device=device),
                dsh=torch.empty((n, K, 3), dtype=torch.float32, device=device))


def render_bwd(means, scales, quats, opacities, sh, sh_degree, cam, proj, sorted_vals, ranges, bg, final_T,
               n_contrib, dL_dimage, grads: dict | None = None, accum=None, denom=None, order=None,
               stream=None) -> dict:
    n = means.shape[0]
    if grads is None:
        grads = alloc_grads(n, sh_degree, means.device)
    camc = camera_struct(cam)
    g = GsGrads(_ptr(grads["grad_screen"]), _ptr(grads["dmeans"]), _ptr(grads["dscales"]), _ptr(grads["dquats"]),
                _ptr(grads["dsh"]))
    _check(lib().gs_render_bwd(n, _ptr(means), _ptr(scales), _ptr(quats), _ptr(opacities), _ptr(sh),
                               int(sh_degree), C.byref(camc), projected_struct(proj), _ptr(sorted_vals),
                               _ptr(ranges), _ptr(order), _bg(bg), _ptr(final_T), _ptr(n_contrib), _ptr(dL_dimage), g,
                               _ptr(accum), _ptr(denom), _stream(stream)), "gs_render_bwd")
    return grads


class Rasterizer:
    """Holds one scene's buffers and runs the five calls in order.

    Buffers are allocated by torch and reused across frames; the pair buffers grow when
    gs_bin_tiles reports that they are too small.
    """

    def __init__(self, means, scales, quats, opacities, sh, sh_degree: int, pair_capacity: int = 0):
        self.means, self.scales, self.quats, self.opac, self.sh = means, scales, quats, opacities, sh
        self.sh_degree = int(sh_degree)
        self.n = int(means.shape[0])
        self.device = means.device
        self.proj = alloc_projected(self.n, self.device)
        self.digit_counts = torch.empty(TILE_DIGIT_COUNTS, dtype=torch.int64, device=self.device)
        self.capacity = 0
        self.keys = self.vals = self.keys_tmp = self.vals_tmp = None
        self.workspace = None
        self._ensure_pairs(max(pair_capacity, 1), 1)

    def _ensure_pairs(self, cap: int, num_tiles: int):
        if cap > self.capacity:
            self.capacity = int(cap)
            d = self.device
            self.keys = torch.empty(self.capacity, dtype=torch.int64, device=d)
            self.vals = torch.empty(self.capacity, dtype=torch.int32, device=d)
            self.keys_tmp = torch.empty(self.capacity, dtype=torch.int64, device=d)
            self.vals_tmp = torch.empty(self.capacity, dtype=torch.int32, device=d)
        need = workspace_bytes(self.n, self.capacity, num_tiles)
        if self.workspace is None or self.workspace.numel() < need:
            self.workspace = torch.empty(need, dtype=torch.uint8, device=self.device)

    def forward(self, cam, bg=(0.0, 0.0, 0.0), stream=None, with_keys: bool = True) -> dict:
        """One frame.  with_keys=False sorts with gs_sort_ids: the output's "keys" are then
        unspecified (the compositing needs the sorted ids only)."""
        W, H = int(cam.width), int(cam.height)
        tiles = ((W + TILE - 1) // TILE) * ((H + TILE - 1) // TILE)
        self._ensure_pairs(self.capacity, tiles)
        project(self.means, self.scales, self.quats, self.opac, self.sh, self.sh_degree, cam, self.proj, stream)
        st, P = bin_tiles(self.proj, cam, self.keys, self.vals, self.workspace, stream, self.digit_counts)
        if st == GS_ERR_CAPACITY:
            self._ensure_pairs(P + P // 4 + 1, tiles)
            st, P = bin_tiles(self.proj, cam, self.keys, self.vals, self.workspace, stream, self.digit_counts)
            _check(st, "gs_bin_tiles")
        ranges = torch.empty((tiles, 2), dtype=torch.int64, device=self.device)
        order = torch.empty(tiles, dtype=torch.int32, device=self.device)
        if with_keys:
            in_tmp = sort_keys(P, tiles, self.keys, self.vals, self.keys_tmp, self.vals_tmp, ranges, self.workspace,
                               order, stream=stream, leave_in_tmp=True, digit_counts=self.digit_counts)
        else:
            in_tmp = sort_ids(P, tiles, self.keys, self.vals, self.keys_tmp, self.vals_tmp, ranges, self.workspace,
                              order, stream=stream, digit_counts=self.digit_counts)
        sk, sv = (self.keys_tmp, self.vals_tmp) if in_tmp else (self.keys, self.vals)
        image = torch.empty((3, H, W), dtype=torch.float32, device=self.device)
        final_T = torch.empty((H, W), dtype=torch.float32, device=self.device)
        n_contrib = torch.empty((H, W), dtype=torch.int32, device=self.device)
        render_fwd(self.proj, sv, ranges, cam, bg, image, final_T, n_contrib, order, stream=stream)
        return dict(image=image, final_T=final_T, n_contrib=n_contrib, ranges=ranges, order=order, n_pairs=P,
                    keys=sk[:P], vals=sv[:P], sorted_vals=sv, proj=self.proj, cam=cam, bg=tuple(bg))

    def backward(self, fwd: dict, dL_dimage, accum=None, denom=None, stream=None) -> dict:
        return render_bwd(self.means, self.scales, self.quats, self.opac, self.sh, self.sh_degree, fwd["cam"],
                          fwd["proj"], fwd["sorted_vals"], fwd["ranges"], fwd["bg"], fwd["final_T"], fwd["n_contrib"],
                          dL_dimage, None, accum, denom, fwd.get("order"), stream=stream)


def scene_to_device(scene, device="cuda"):
    """Upload a scenes.Scene's arrays once (float32, contiguous)."""
    f = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(device)
    return f(scene.means), f(scene.scales), f(scene.quats), f(scene.opacities), f(scene.sh)


def densify_params(grad_threshold: float, scale_threshold: float, use_abs: bool = False, split_n: int = 2,
                   split_shrink: float = 1.6, min_opacity: float = 0.005, max_scale: float = 0.0) -> GsDensifyParams:
    return GsDensifyParams(grad_threshold, 1 if use_abs else 0, scale_threshold, split_n, split_shrink, min_opacity,
                           max_scale)


def densify(means, scales, quats, opacities, sh, sh_degree: int, accum, denom, normals, params: GsDensifyParams,
            out: dict | None = None, stream=None) -> dict:
    """gs_densify.  Sizes the outputs with a count-only call unless ``out`` (dict of output
    tensors, capacity = out["src"].shape[0]) is given; returns the outputs trimmed to the
    new count, plus ``n_out``."""
    L = lib()
    n = means.shape[0]
    dev = means.device
    ws = torch.empty(max(int(L.gs_densify_workspace_bytes(n)), 8), dtype=torch.uint8, device=dev)
    cnt = C.c_int64(0)
    args = (n, _ptr(means), _ptr(scales), _ptr(quats), _ptr(opacities), _ptr(sh), int(sh_degree), _ptr(accum),
            _ptr(denom), _ptr(normals), C.byref(params))
    if out is None:
        _check(L.gs_densify(*args, None, None, None, None, None, None, 0, C.byref(cnt), _ptr(ws), ws.numel(),
                            _stream(stream)), "gs_densify")
        m = max(int(cnt.value), 1)
        K = (sh_degree + 1) ** 2
        out = dict(means=torch.empty((m, 3), dtype=torch.float32, device=dev),
                   scales=torch.empty((m, 3), dtype=torch.float32, device=dev),
                   quats=torch.empty((m, 4), dtype=torch.float32, device=dev),
                   opacities=torch.empty(m, dtype=torch.float32, device=dev),
                   sh=torch.empty((m, K, 3), dtype=torch.float32, device=dev),
                   src=torch.empty(m, dtype=torch.int32, device=dev))
    st = L.gs_densify(*args, _ptr(out["means"]), _ptr(out["scales"]), _ptr(out["quats"]), _ptr(out["opacities"]),
                      _ptr(out["sh"]), _ptr(out["src"]), out["src"].shape[0], C.byref(cnt), _ptr(ws), ws.numel(),
                      _stream(stream))
    if st == GS_ERR_CAPACITY:
        return dict(status=st, n_out=int(cnt.value))
    _check(st, "gs_densify")
    k = int(cnt.value)
    res = {key: v[:k] for key, v in out.items()}
    res["n_out"] = k
    res["status"] = st
    return res


def adam_state(n_units: int, device="cuda") -> tuple:
    """Zero Adam state for gs_adam_q16: (state uint32 as int32 [n], bounds float32 [ceil(n/256)][4])."""
    return (torch.zeros(n_units, dtype=torch.int32, device=device),
            torch.zeros(((n_units + 255) // 256, 4), dtype=torch.float32, device=device))


def adam_q16(params, grads, state, bounds, lr: float, step: int, beta1: float = 0.9, beta2: float = 0.999,
             eps: float = 1e-8, stream=None):
    """gs_adam_q16 on flat float32 tensors (params and state updated in place)."""
    h = GsAdamParams(lr, beta1, beta2, eps, int(step))
    _check(lib().gs_adam_q16(params.numel(), _ptr(params), _ptr(grads), _ptr(state), _ptr(bounds), C.byref(h),
                             _stream(stream)), "gs_adam_q16")


def fpbo_pack(params, stream=None) -> tuple:
    """gs_fpbo_pack: packed start state of flat float32 params, (state uint16 as int16
    [ceil(n/256)][3][256], bounds float32 [ceil(n/256)][6])."""
    n = params.numel()
    nb = (n + 255) // 256
    state = torch.empty((nb, 3, 256), dtype=torch.int16, device=params.device)
    bounds = torch.empty((nb, 6), dtype=torch.float32, device=params.device)
    _check(lib().gs_fpbo_pack(n, _ptr(params), _ptr(state), _ptr(bounds), _stream(stream)), "gs_fpbo_pack")
    return state, bounds


def adam_fpbo(n: int, state, bounds, grads, params_out, lr: float, step: int, beta1: float = 0.9,
              beta2: float = 0.999, eps: float = 1e-8, stream=None):
    """gs_adam_fpbo on a packed state (updated in place); params_out (flat float32, or None)
    receives the decoded new parameters."""
    h = GsAdamParams(lr, beta1, beta2, eps, int(step))
    _check(lib().gs_adam_fpbo(int(n), _ptr(state), _ptr(bounds), _ptr(grads), _ptr(params_out), C.byref(h),
                              _stream(stream)), "gs_adam_fpbo")


def quantize_sh(sh, sh_degree: int, bits: int, stream=None) -> tuple:
    """gs_quantize_sh: (codes uint8 / int16-typed uint16 [n][K][3], bounds float32 [nb][2])."""
    n = sh.shape[0]
    K = (sh_degree + 1) ** 2
    units = n * K * 3
    codes = torch.empty((n, K, 3), dtype=torch.uint8 if bits == 8 else torch.int16, device=sh.device)
    bounds = torch.empty(((units + 255) // 256, 2), dtype=torch.float32, device=sh.device)
    _check(lib().gs_quantize_sh(n, _ptr(sh), int(sh_degree), int(bits), _ptr(codes), _ptr(bounds), _stream(stream)),
           "gs_quantize_sh")
    return codes, bounds


def project_qsh(means, scales, quats, opacities, codes, bounds, bits: int, sh_degree: int, cam,
                out: dict | None = None, stream=None) -> dict:
    """gs_project_qsh into ``out`` (allocated if None)."""
    n = means.shape[0]
    if out is None:
        out = alloc_projected(n, means.device)
    camc = camera_struct(cam)
    _check(lib().gs_project_qsh(n, _ptr(means), _ptr(scales), _ptr(quats), _ptr(opacities), _ptr(codes),
                                _ptr(bounds), int(bits), int(sh_degree), C.byref(camc), projected_struct(out),
                                _stream(stream)), "gs_project_qsh")
    return out
