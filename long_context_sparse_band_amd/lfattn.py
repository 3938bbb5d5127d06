"""Thin ctypes binding of liblfattn (include/lfattn.h), same names as the C ABI.

Argument marshalling only: every step of the forward pass runs in the HIP
kernels of liblfattn.so.  PyTorch appears only to hand over device pointers
and the current HIP stream.  If the library is missing, loading it raises;
there is no fallback.
"""

from __future__ import annotations

import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "liblfattn.so")

LFATTN_OK = 0
LFATTN_EINVAL = 1
LFATTN_EUNSUPPORTED = 2
LFATTN_ENOMEM = 3
LFATTN_EHIP = 4
LFATTN_ESCRATCH = 5

LFATTN_F32 = 0
LFATTN_BF16 = 1

# Every entry point include/lfattn.h declares.
EXPORTS = ("lfattn_create", "lfattn_create_masked", "lfattn_create_causal",
           "lfattn_create_chunked", "lfattn_forward", "lfattn_forward_noalloc", "lfattn_forward_lse",
           "lfattn_forward_global_proj_lse", "lfattn_backward_global_proj", "lfattn_backward",
           "lfattn_forward_global_proj", "lfattn_destroy", "lfattn_status_string",
           "lfattn_scored_pairs", "lfattn_band_launch_pairs", "lfattn_band_rows",
           "lfattn_global_list", "lfattn_global_list_batch",
           "lfattn_set_timing", "lfattn_read_timing", "lfattn_read_backward_timing")

_lib = None


class LfattnError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {lfattn_status_string(status)} (status {status})")


def load():
    """Open liblfattn.so and declare the C signatures.  Raises if it is missing."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise FileNotFoundError(
            f"{LIB_PATH} is not built; run __graft_entry__.build() (hipcc, gfx950)")
    lib = ctypes.CDLL(LIB_PATH)
    vp = ctypes.c_void_p
    i32p = ctypes.POINTER(ctypes.c_int)
    lib.lfattn_create.restype = ctypes.c_int
    lib.lfattn_create.argtypes = [ctypes.POINTER(vp), ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                  ctypes.c_int, ctypes.c_int, ctypes.c_int, i32p, i32p,
                                  ctypes.c_int, ctypes.c_float]
    lib.lfattn_create_masked.restype = ctypes.c_int
    lib.lfattn_create_masked.argtypes = [ctypes.POINTER(vp), ctypes.c_int, ctypes.c_int,
                                         ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                         i32p, ctypes.POINTER(ctypes.c_ubyte), ctypes.c_float]
    lib.lfattn_create_causal.restype = ctypes.c_int
    lib.lfattn_create_causal.argtypes = [ctypes.POINTER(vp), ctypes.c_int, ctypes.c_int,
                                         ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                         i32p, ctypes.c_float]
    lib.lfattn_create_chunked.restype = ctypes.c_int
    lib.lfattn_create_chunked.argtypes = [ctypes.POINTER(vp), ctypes.c_int, ctypes.c_int,
                                          ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                          ctypes.c_int, ctypes.c_int, ctypes.c_float]
    lib.lfattn_forward.restype = ctypes.c_int
    lib.lfattn_forward.argtypes = [vp, vp, vp, vp, vp, vp]
    lib.lfattn_forward_global_proj_lse.restype = ctypes.c_int
    lib.lfattn_forward_global_proj_lse.argtypes = [vp] * 10
    lib.lfattn_backward_global_proj.restype = ctypes.c_int
    lib.lfattn_backward_global_proj.argtypes = [vp] * 17
    lib.lfattn_forward_noalloc.restype = ctypes.c_int
    lib.lfattn_forward_noalloc.argtypes = [vp, vp, vp, vp, vp, vp]
    lib.lfattn_backward.restype = ctypes.c_int
    lib.lfattn_backward.argtypes = [vp] * 10 + [vp]
    lib.lfattn_forward_lse.restype = ctypes.c_int
    lib.lfattn_forward_lse.argtypes = [vp, vp, vp, vp, vp, vp, vp]
    lib.lfattn_forward_global_proj.restype = ctypes.c_int
    lib.lfattn_forward_global_proj.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp]
    lib.lfattn_destroy.restype = ctypes.c_int
    lib.lfattn_destroy.argtypes = [vp]
    lib.lfattn_status_string.restype = ctypes.c_char_p
    lib.lfattn_status_string.argtypes = [ctypes.c_int]
    lib.lfattn_scored_pairs.restype = ctypes.c_int
    lib.lfattn_scored_pairs.argtypes = [vp, ctypes.POINTER(ctypes.c_longlong)]
    lib.lfattn_band_launch_pairs.restype = ctypes.c_int
    lib.lfattn_band_launch_pairs.argtypes = [vp, ctypes.POINTER(ctypes.c_longlong)]
    lib.lfattn_band_rows.restype = ctypes.c_int
    lib.lfattn_band_rows.argtypes = [vp, i32p]
    lib.lfattn_global_list.restype = ctypes.c_int
    lib.lfattn_global_list.argtypes = [vp, i32p, ctypes.c_int, i32p]
    lib.lfattn_global_list_batch.restype = ctypes.c_int
    lib.lfattn_global_list_batch.argtypes = [vp, ctypes.c_int, i32p, ctypes.c_int, i32p]
    lib.lfattn_set_timing.restype = ctypes.c_int
    lib.lfattn_set_timing.argtypes = [vp, ctypes.c_int]
    lib.lfattn_read_timing.restype = ctypes.c_int
    lib.lfattn_read_timing.argtypes = [vp, ctypes.POINTER(ctypes.c_double),
                                       ctypes.POINTER(ctypes.c_double), i32p]
    lib.lfattn_read_backward_timing.restype = ctypes.c_int
    lib.lfattn_read_backward_timing.argtypes = [vp] + [ctypes.POINTER(ctypes.c_double)] * 3 + [i32p]
    _lib = lib
    return lib


def lfattn_status_string(status: int) -> str:
    return load().lfattn_status_string(int(status)).decode()


def _check(status: int, what: str):
    if status != LFATTN_OK:
        raise LfattnError(status, what)


def _int_array(values):
    if values is None:
        return None
    vals = [int(x) for x in values]
    return (ctypes.c_int * max(1, len(vals)))(*vals)


def lfattn_create(B: int, H: int, N: int, D: int, dtype: int, window: int,
                  dilation=None, global_idx=(), scale: float = 0.0) -> int:
    """Returns the handle (an integer address).  dtype: LFATTN_F32 or LFATTN_BF16."""
    lib = load()
    handle = ctypes.c_void_p()
    g = list(global_idx) if global_idx is not None else []
    st = lib.lfattn_create(ctypes.byref(handle), B, H, N, D, dtype, window,
                           _int_array(dilation), _int_array(g) if g else None, len(g),
                           float(scale))
    _check(st, "lfattn_create")
    return handle.value


def lfattn_create_masked(B: int, H: int, N: int, D: int, dtype: int, window: int,
                         dilation=None, global_mask=None, scale: float = 0.0) -> int:
    """As lfattn_create, with one global set per batch element: global_mask is
    a [B, N] array-like of booleans/bytes (nonzero: global), or None."""
    lib = load()
    handle = ctypes.c_void_p()
    mp = None
    if global_mask is not None:
        import numpy as np
        m = np.ascontiguousarray(np.asarray(global_mask).astype(np.uint8).reshape(B * N))
        mp = (ctypes.c_ubyte * (B * N)).from_buffer_copy(m.tobytes())
    st = lib.lfattn_create_masked(ctypes.byref(handle), B, H, N, D, dtype, window,
                                  _int_array(dilation), mp, float(scale))
    _check(st, "lfattn_create_masked")
    return handle.value


def lfattn_create_causal(B: int, H: int, N: int, D: int, dtype: int, window: int,
                         dilation=None, scale: float = 0.0) -> int:
    """As lfattn_create for the causal band (no global tokens)."""
    lib = load()
    handle = ctypes.c_void_p()
    st = lib.lfattn_create_causal(ctypes.byref(handle), B, H, N, D, dtype, window,
                                  _int_array(dilation), float(scale))
    _check(st, "lfattn_create_causal")
    return handle.value


def lfattn_create_chunked(B: int, H: int, N: int, D: int, dtype: int, chunk: int,
                          n_memory: int, scale: float = 0.0) -> int:
    """GMAT chunked attention: chunks of `chunk` keys after n_memory memory
    positions (the global rows)."""
    lib = load()
    handle = ctypes.c_void_p()
    st = lib.lfattn_create_chunked(ctypes.byref(handle), B, H, N, D, dtype, chunk, n_memory,
                                   float(scale))
    _check(st, "lfattn_create_chunked")
    return handle.value


def _ptr(x) -> int:
    if x is None:
        return None
    return x if isinstance(x, int) else x.data_ptr()


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    return stream if isinstance(stream, int) else stream.cuda_stream


def lfattn_forward(handle: int, Q, K, V, O, stream=None) -> None:
    """Enqueue one forward.  Q, K, V, O: device tensors (or raw addresses);
    stream: a HIP stream handle (int), a torch stream, or None for torch's
    current stream on the current device."""
    lib = load()
    _check(lib.lfattn_forward(handle, _ptr(Q), _ptr(K), _ptr(V), _ptr(O), _stream(stream)),
           "lfattn_forward")


def lfattn_forward_global_proj_lse(handle: int, Q, K, V, Qg, Kg, Vg, O, LSE,
                                   stream=None) -> None:
    """lfattn_forward_global_proj that also writes each row's log-sum-exp
    (the global rows' from their own projections); bf16 handles."""
    lib = load()
    _check(lib.lfattn_forward_global_proj_lse(handle, _ptr(Q), _ptr(K), _ptr(V), _ptr(Qg),
                                              _ptr(Kg), _ptr(Vg), _ptr(O), _ptr(LSE),
                                              _stream(stream)),
           "lfattn_forward_global_proj_lse")


def lfattn_backward_global_proj(handle: int, Q, K, V, Qg, Kg, Vg, O, dO, LSE, dQ, dK, dV,
                                dQg, dKg, dVg, stream=None) -> None:
    """Gradients of the forward with the global rows' own projections: the
    global rows' terms in dQg, dKg, dVg, the other rows' in dQ, dK, dV (fp32
    device tensors [B, H, N, D]); Qg, Kg, Vg may be None for Q, K, V."""
    lib = load()
    _check(lib.lfattn_backward_global_proj(
        handle, *(_ptr(x) for x in (Q, K, V, Qg, Kg, Vg, O, dO, LSE, dQ, dK, dV, dQg, dKg, dVg)),
        _stream(stream)), "lfattn_backward_global_proj")


def lfattn_forward_noalloc(handle: int, Q, K, V, O, stream=None) -> None:
    """lfattn_forward with the global rows' partial records in the library's
    static device scratch (allocates nothing; calls that may overlap on one
    GPU race)."""
    lib = load()
    _check(lib.lfattn_forward_noalloc(handle, _ptr(Q), _ptr(K), _ptr(V), _ptr(O),
                                      _stream(stream)), "lfattn_forward_noalloc")


def lfattn_forward_lse(handle: int, Q, K, V, O, LSE, stream=None) -> None:
    """Forward that also writes the natural log-sum-exp of each row's scaled
    scores into LSE (a float32 device tensor [B, H, N]); bf16 handles."""
    lib = load()
    _check(lib.lfattn_forward_lse(handle, _ptr(Q), _ptr(K), _ptr(V), _ptr(O), _ptr(LSE),
                                  _stream(stream)), "lfattn_forward_lse")


def lfattn_backward(handle: int, Q, K, V, O, dO, LSE, dQ, dK, dV, stream=None) -> None:
    """Gradients dQ, dK, dV (float32 device tensors [B, H, N, D]) of the forward
    for the upstream gradient dO; LSE from lfattn_forward_lse.  bf16 handles."""
    lib = load()
    _check(lib.lfattn_backward(handle, _ptr(Q), _ptr(K), _ptr(V), _ptr(O), _ptr(dO), _ptr(LSE),
                               _ptr(dQ), _ptr(dK), _ptr(dV), _stream(stream)),
           "lfattn_backward")


def lfattn_forward_global_proj(handle: int, Q, K, V, Qg, Kg, Vg, O, stream=None) -> None:
    """Enqueue one forward in which the global rows take Qg, Kg, Vg (each may be
    None for Q, K, V)."""
    lib = load()
    _check(lib.lfattn_forward_global_proj(handle, _ptr(Q), _ptr(K), _ptr(V), _ptr(Qg),
                                          _ptr(Kg), _ptr(Vg), _ptr(O), _stream(stream)),
           "lfattn_forward_global_proj")


def lfattn_destroy(handle: int) -> None:
    _check(load().lfattn_destroy(handle), "lfattn_destroy")


def lfattn_scored_pairs(handle: int) -> int:
    n = ctypes.c_longlong()
    _check(load().lfattn_scored_pairs(handle, ctypes.byref(n)), "lfattn_scored_pairs")
    return int(n.value)


def lfattn_band_launch_pairs(handle: int) -> int:
    n = ctypes.c_longlong()
    _check(load().lfattn_band_launch_pairs(handle, ctypes.byref(n)), "lfattn_band_launch_pairs")
    return int(n.value)


def lfattn_band_rows(handle: int) -> int:
    n = ctypes.c_int()
    _check(load().lfattn_band_rows(handle, ctypes.byref(n)), "lfattn_band_rows")
    return int(n.value)


def lfattn_global_list(handle: int) -> list:
    lib = load()
    n = ctypes.c_int()
    _check(lib.lfattn_global_list(handle, None, 0, ctypes.byref(n)), "lfattn_global_list")
    buf = (ctypes.c_int * max(1, n.value))()
    _check(lib.lfattn_global_list(handle, buf, n.value, ctypes.byref(n)), "lfattn_global_list")
    return list(buf[: n.value])


def lfattn_global_list_batch(handle: int, b: int) -> list:
    lib = load()
    n = ctypes.c_int()
    _check(lib.lfattn_global_list_batch(handle, b, None, 0, ctypes.byref(n)),
           "lfattn_global_list_batch")
    buf = (ctypes.c_int * max(1, n.value))()
    _check(lib.lfattn_global_list_batch(handle, b, buf, n.value, ctypes.byref(n)),
           "lfattn_global_list_batch")
    return list(buf[: n.value])


def lfattn_set_timing(handle: int, enable: bool) -> None:
    _check(load().lfattn_set_timing(handle, 1 if enable else 0), "lfattn_set_timing")


def lfattn_read_timing(handle: int):
    """(band_ms_total, global_ms_total, n_forwards) since timing was enabled/read."""
    b, g, n = ctypes.c_double(), ctypes.c_double(), ctypes.c_int()
    _check(load().lfattn_read_timing(handle, ctypes.byref(b), ctypes.byref(g), ctypes.byref(n)),
           "lfattn_read_timing")
    return b.value, g.value, n.value


def lfattn_read_backward_timing(handle: int):
    """(rows_ms_total, keys_ms_total, merge_ms_total, n_backwards) of the
    backward calls since timing was enabled/read."""
    t = [ctypes.c_double() for _ in range(3)]
    n = ctypes.c_int()
    _check(load().lfattn_read_backward_timing(handle, *(ctypes.byref(x) for x in t),
                                              ctypes.byref(n)), "lfattn_read_backward_timing")
    return t[0].value, t[1].value, t[2].value, n.value


class LFAttention:
    """Owns one handle: create on construction, destroy on close()."""

    def __init__(self, B, H, N, D, dtype, window, dilation=None, global_idx=(), scale=0.0):
        self.shape = (B, H, N, D)
        self.dtype = dtype
        self.handle = lfattn_create(B, H, N, D, dtype, window, dilation, global_idx, scale)

    def forward(self, Q, K, V, O, stream=None, Qg=None, Kg=None, Vg=None):
        """Qg, Kg, Vg: the global rows' own projections (None: Q, K, V)."""
        if Qg is None and Kg is None and Vg is None:
            lfattn_forward(self.handle, Q, K, V, O, stream)
        else:
            lfattn_forward_global_proj(self.handle, Q, K, V, Qg, Kg, Vg, O, stream)
        return O

    def forward_lse(self, Q, K, V, O, LSE, stream=None):
        """Forward that also writes each row's log-sum-exp (bf16 handles)."""
        lfattn_forward_lse(self.handle, Q, K, V, O, LSE, stream)
        return O, LSE

    def backward(self, Q, K, V, O, dO, LSE, dQ, dK, dV, stream=None):
        """Gradients into the caller's fp32 dQ, dK, dV (bf16 handles)."""
        lfattn_backward(self.handle, Q, K, V, O, dO, LSE, dQ, dK, dV, stream)
        return dQ, dK, dV

    @property
    def scored_pairs(self) -> int:
        return lfattn_scored_pairs(self.handle)

    def close(self):
        if self.handle:
            lfattn_destroy(self.handle)
            self.handle = 0

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
