"""CPU-side checks of the C-ABI library: it loads (no GPU needed), exports every entry
point that include/gs_raster.h declares, and its host-only calls behave."""
import ctypes as C
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = [os.path.join(ROOT, "include", h) for h in ("gs_raster.h", "gs_measure.h")]
LIB = os.path.join(ROOT, "tile_differentiable_rasterizer_amd", "libgsraster.so")


def declared():
    text = "".join(open(h).read() for h in HEADERS)
    return sorted(set(re.findall(r"^\s*(?:gs_status|size_t|const char\*)\s+(gs_\w+)\s*\(", text, re.M)))


def test_header_declares_the_five_calls():
    names = declared()
    for f in ("gs_project", "gs_bin_tiles", "gs_sort_keys", "gs_render_fwd", "gs_render_bwd"):
        assert f in names


@pytest.mark.skipif(not os.path.exists(LIB), reason="libgsraster.so not built")
def test_library_exports_every_declared_symbol():
    lib = C.CDLL(LIB)
    for name in declared():
        assert hasattr(lib, name), name


@pytest.mark.skipif(not os.path.exists(LIB), reason="libgsraster.so not built")
def test_host_only_calls():
    lib = C.CDLL(LIB)
    lib.gs_status_string.restype = C.c_char_p
    lib.gs_status_string.argtypes = [C.c_int32]
    assert lib.gs_status_string(0) == b"ok"
    assert lib.gs_status_string(2) == b"pair buffer too small"
    lib.gs_workspace_bytes.restype = C.c_size_t
    lib.gs_workspace_bytes.argtypes = [C.c_int64, C.c_int64, C.c_int32]
    assert lib.gs_workspace_bytes(-1, 0, 1) == 0
    assert lib.gs_workspace_bytes(10, 10, 0) == 0
    small = lib.gs_workspace_bytes(1000, 1000, 16)
    big = lib.gs_workspace_bytes(1000, 10_000_000, 8160)
    assert 0 < small < big
    # the sort's per-pass look-back words dominate: at least 6 passes x 8 B x 256 digits per 4096 keys
    assert big >= 6 * 8 * 256 * (10_000_000 // 4096)


@pytest.mark.skipif(not os.path.exists(LIB), reason="libgsraster.so not built")
def test_packed_adam_argument_checks():
    # every case is refused before any HIP call: null or misaligned pointers, bad hyper-parameters
    from tile_differentiable_rasterizer_amd import raster

    L = raster.lib()
    ok = raster.GsAdamParams(1e-3, 0.9, 0.999, 1e-8, 1)
    a16, a8 = 1 << 20, 1 << 20  # aligned stand-ins, never dereferenced
    bad = raster.GS_ERR_INVALID_ARG
    assert L.gs_fpbo_pack(-1, a16, a8, a8, None) == bad
    assert L.gs_fpbo_pack(10, None, a8, a8, None) == bad
    assert L.gs_fpbo_pack(10, a16 + 4, a8, a8, None) == bad
    assert L.gs_fpbo_pack(10, a16, a8 + 2, a8, None) == bad
    assert L.gs_adam_fpbo(10, a8, a8, None, None, C.byref(ok), None) == bad
    assert L.gs_adam_fpbo(10, a8, a8, a16 + 8, None, C.byref(ok), None) == bad
    assert L.gs_adam_fpbo(10, a8, a8, a16, a16 + 4, C.byref(ok), None) == bad
    assert L.gs_adam_fpbo(10, a8, a8 + 4, a16, None, C.byref(ok), None) == bad
    for h in (raster.GsAdamParams(1e-3, 0.9, 0.999, 1e-8, 0), raster.GsAdamParams(1e-3, 1.0, 0.999, 1e-8, 1)):
        assert L.gs_adam_fpbo(10, a8, a8, a16, None, C.byref(h), None) == bad
    assert L.gs_adam_fpbo(1 << 40, a8, a8, a16, None, C.byref(ok), None) == raster.GS_ERR_OVERFLOW
    # nothing to do: no launch
    assert L.gs_fpbo_pack(0, None, None, None, None) == raster.GS_OK
    assert L.gs_adam_fpbo(0, None, None, None, None, C.byref(ok), None) == raster.GS_OK


@pytest.mark.skipif(not os.path.exists(LIB), reason="libgsraster.so not built")
def test_kernel_timer_host_logic():
    # no launch happens between start and stop, so no HIP call is made
    from tile_differentiable_rasterizer_amd import raster

    assert raster.kernel_timer_stop()[0] == 1          # not armed
    assert raster.kernel_timer_start("k_nothing") == 1  # unknown kernel
    assert raster.kernel_timer_start("k_render_bwd") == 0
    assert raster.kernel_timer_start("k_render_fwd") == 1  # already armed
    assert raster.kernel_timer_stop() == (0, 0, 0.0)
    assert raster.kernel_timer_start("k_project") == 0
    assert raster.kernel_timer_stop() == (0, 0, 0.0)


def test_binding_module_fails_loudly_without_library(tmp_path, monkeypatch):
    from tile_differentiable_rasterizer_amd import raster

    monkeypatch.setattr(raster, "_LIB_PATH", str(tmp_path / "missing.so"))
    monkeypatch.setattr(raster, "_lib", None)
    with pytest.raises(ImportError):
        raster.lib()
