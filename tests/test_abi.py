"""The C-ABI library loads, exports what include/lfattn.h declares, and rejects
invalid arguments before any HIP call (so these run without a GPU)."""

import ctypes
import os
import re
import subprocess

import numpy as np
import pytest

from long_context_sparse_band_amd import lfattn as L

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "lfattn.h")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(lfattn_[a-z_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(L.LIB_PATH):
        from long_context_sparse_band_amd import build
        build.build()
    return L.load()


def test_header_declares_the_binding_names():
    assert _declared() == sorted(L.EXPORTS)


def test_library_exports_every_declared_symbol(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", L.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\bT (lfattn_\w+)", out))
    for name in _declared():
        assert name in exported, name
        assert hasattr(lib, name)


def test_library_holds_gfx950_code():
    """The fat binary built here carries a gfx950 code object (its bundle id)."""
    data = open(L.LIB_PATH, "rb").read()
    assert b"amdgcn-amd-amdhsa--gfx950" in data


def test_status_strings(lib):
    assert L.lfattn_status_string(L.LFATTN_OK) == "ok"
    assert L.lfattn_status_string(L.LFATTN_EINVAL) == "invalid argument"
    assert L.lfattn_status_string(L.LFATTN_EUNSUPPORTED) == "unsupported configuration"
    assert L.lfattn_status_string(99) == "unknown status"


def _create(lib, B=1, H=2, N=100, D=64, dtype=1, window=16, dil=None, glob=None, scale=0.0,
            out=True):
    h = ctypes.c_void_p(12345)
    dil_arr = (ctypes.c_int * len(dil))(*dil) if dil is not None else None
    g_arr = (ctypes.c_int * len(glob))(*glob) if glob else None
    st = lib.lfattn_create(ctypes.byref(h) if out else None, B, H, N, D, dtype, window,
                           dil_arr, g_arr, len(glob) if glob else 0, scale)
    return st, h.value


@pytest.mark.parametrize("kw", [
    dict(B=0), dict(H=0), dict(N=0), dict(D=0), dict(D=-64), dict(window=-1),
    dict(dtype=7), dict(dil=[1, 0]), dict(dil=[-2, 1]), dict(glob=[100]), dict(glob=[-1]),
    dict(glob=[3, 5, 200]), dict(scale=float("nan")), dict(scale=float("inf")),
    dict(out=False)])
def test_create_rejects_invalid(lib, kw):
    st, h = _create(lib, **kw)
    assert st == L.LFATTN_EINVAL
    if kw.get("out", True):
        assert h is None  # *out cleared


def test_create_rejects_null_global_list_with_count(lib):
    h = ctypes.c_void_p()
    assert lib.lfattn_create(ctypes.byref(h), 1, 1, 10, 64, 1, 4, None, None, 3, 0.0) == \
        L.LFATTN_EINVAL


@pytest.mark.parametrize("D", [32, 96, 256, 1])
def test_create_unsupported_head_dim(lib, D):
    st, _ = _create(lib, D=D)
    assert st == L.LFATTN_EUNSUPPORTED


def test_null_handle_calls(lib):
    n = ctypes.c_longlong()
    assert lib.lfattn_scored_pairs(None, ctypes.byref(n)) == L.LFATTN_EINVAL
    assert lib.lfattn_band_launch_pairs(None, ctypes.byref(n)) == L.LFATTN_EINVAL
    rows = ctypes.c_int()
    assert lib.lfattn_band_rows(None, ctypes.byref(rows)) == L.LFATTN_EINVAL
    assert lib.lfattn_forward(None, 16, 16, 16, 16, None) == L.LFATTN_EINVAL
    assert lib.lfattn_destroy(None) == L.LFATTN_OK
    assert lib.lfattn_set_timing(None, 1) == L.LFATTN_EINVAL
    cnt = ctypes.c_int()
    assert lib.lfattn_global_list(None, None, 0, ctypes.byref(cnt)) == L.LFATTN_EINVAL


@pytest.mark.parametrize("kw", [
    dict(B=0), dict(N=0), dict(window=-1), dict(dtype=7), dict(dil=[0]),
    dict(scale=float("nan")), dict(out=False)])
def test_create_masked_rejects_invalid(lib, kw):
    B, H, N = kw.get("B", 2), 1, kw.get("N", 16)
    mask = (ctypes.c_ubyte * max(1, B * N))()
    h = ctypes.c_void_p(1234)
    dil = (ctypes.c_int * 1)(*kw["dil"]) if "dil" in kw else None
    st = lib.lfattn_create_masked(ctypes.byref(h) if kw.get("out", True) else None, B, H, N, 64,
                                  kw.get("dtype", 1), kw.get("window", 4), dil, mask,
                                  kw.get("scale", 0.0))
    assert st == L.LFATTN_EINVAL
    if kw.get("out", True):
        assert h.value is None


def test_create_masked_unsupported_head_dim(lib):
    h = ctypes.c_void_p()
    assert lib.lfattn_create_masked(ctypes.byref(h), 1, 1, 16, 96, 1, 4, None, None, 0.0) == \
        L.LFATTN_EUNSUPPORTED


def test_create_causal_rejects_invalid(lib):
    h = ctypes.c_void_p(1234)
    assert lib.lfattn_create_causal(None, 1, 1, 16, 64, 1, 4, None, 0.0) == L.LFATTN_EINVAL
    assert lib.lfattn_create_causal(ctypes.byref(h), 1, 1, 16, 64, 1, -2, None, 0.0) == \
        L.LFATTN_EINVAL
    assert h.value is None
    assert lib.lfattn_create_causal(ctypes.byref(h), 1, 1, 16, 96, 1, 4, None, 0.0) == \
        L.LFATTN_EUNSUPPORTED


def test_create_chunked_rejects_invalid(lib):
    h = ctypes.c_void_p(1234)
    assert lib.lfattn_create_chunked(None, 1, 1, 16, 64, 1, 4, 2, 0.0) == L.LFATTN_EINVAL
    for chunk, mem in [(0, 2), (-1, 2), (4, -1), (4, 17)]:
        assert lib.lfattn_create_chunked(ctypes.byref(h), 1, 1, 16, 64, 1, chunk, mem, 0.0) == \
            L.LFATTN_EINVAL
        assert h.value is None
    assert lib.lfattn_create_chunked(ctypes.byref(h), 1, 1, 16, 96, 1, 4, 2, 0.0) == \
        L.LFATTN_EUNSUPPORTED


def test_backward_rejects_null_handle(lib):
    assert lib.lfattn_backward(None, 16, 16, 16, 16, 16, 16, 16, 16, 16, None) == \
        L.LFATTN_EINVAL


def test_new_entry_points_reject_null_handle(lib):
    assert lib.lfattn_forward_global_proj(None, 16, 16, 16, None, None, None, 16, None) == \
        L.LFATTN_EINVAL
    cnt = ctypes.c_int()
    assert lib.lfattn_global_list_batch(None, 0, None, 0, ctypes.byref(cnt)) == L.LFATTN_EINVAL


def test_binding_raises_on_missing_library(tmp_path, monkeypatch):
    monkeypatch.setattr(L, "LIB_PATH", str(tmp_path / "nope.so"))
    monkeypatch.setattr(L, "_lib", None)
    with pytest.raises(FileNotFoundError):
        L.load()


def test_bf16_global_limit_checked_before_any_hip_call():
    """bf16 handles take at most 512 distinct global positions; one more is
    refused with LFATTN_EUNSUPPORTED before the library touches the GPU."""
    with pytest.raises(L.LfattnError) as e:
        L.lfattn_create(1, 1, 1000, 64, L.LFATTN_BF16, 16, None, list(range(513)))
    assert e.value.status == L.LFATTN_EUNSUPPORTED
    mask = np.zeros((2, 1000), dtype=np.uint8)
    mask[1, :513] = 1
    with pytest.raises(L.LfattnError) as e:
        L.lfattn_create_masked(2, 1, 1000, 64, L.LFATTN_BF16, 16, None, mask)
    assert e.value.status == L.LFATTN_EUNSUPPORTED
