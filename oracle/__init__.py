"""The oracle: TEST INFRASTRUCTURE, NOT PART OF THE PRODUCT.

A plain, slow, double-precision CPU implementation of band + global sparse
attention (``lfattn_oracle.c``, loaded here through ctypes) and a numpy
brute-force mask form of it (``brute.py``).  Only the test suite, the smoke
check and the benchmark's CPU baseline leg may import this package; the GPU
library never does, and the two share no code.

The definition it implements, and the passages it follows, are stated in the
header of ``lfattn_oracle.c``.
"""

from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "lfattn_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

_lib = None


def build(force: bool = True) -> str:
    """Compile the C oracle with gcc into oracle/liboracle.so."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-std=c11", "-Wall", "-Wextra", "-shared", "-fPIC",
               "-pthread", _SRC, "-o", tmp, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        # LFATTN_ORACLE_LIB names another build of the same source (the
        # sanitizer build of the CPU tests); otherwise build when missing or
        # older than its source.
        path = os.environ.get("LFATTN_ORACLE_LIB")
        if not path:
            path = _LIB
            if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
                build(force=True)
        lib = ctypes.CDLL(path)
        i32p = ctypes.POINTER(ctypes.c_int)
        i64p = ctypes.POINTER(ctypes.c_int64)
        f32p = ctypes.POINTER(ctypes.c_float)
        f64p = ctypes.POINTER(ctypes.c_double)
        lib.lfo_allowed_set.restype = ctypes.c_int64
        lib.lfo_allowed_set.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, i32p,
                                        ctypes.c_int, ctypes.c_int, i32p]
        lib.lfo_count_pairs.restype = ctypes.c_int64
        lib.lfo_count_pairs.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                        i32p, i32p, ctypes.c_int]
        lib.lfo_attention.restype = ctypes.c_int
        lib.lfo_attention.argtypes = [f32p, f32p, f32p, f64p, ctypes.c_int, ctypes.c_int,
                                      ctypes.c_int, ctypes.c_int, ctypes.c_int, i32p, i32p,
                                      ctypes.c_int, ctypes.c_double, i64p, ctypes.c_int64,
                                      ctypes.c_int]
        lib.lfo_attention_ex.restype = ctypes.c_int
        lib.lfo_attention_ex.argtypes = [f32p, f32p, f32p, f32p, f32p, f32p, f64p,
                                         ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                         ctypes.c_int, i32p, ctypes.c_int, i32p, i32p,
                                         ctypes.c_int, ctypes.c_double, i64p, ctypes.c_int64,
                                         ctypes.c_int]
        lib.lfo_allowed_set_ex.restype = ctypes.c_int64
        lib.lfo_allowed_set_ex.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                           ctypes.c_int, i32p, ctypes.c_int, ctypes.c_int, i32p]
        lib.lfo_allowed_set_chunked.restype = ctypes.c_int64
        lib.lfo_allowed_set_chunked.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                                ctypes.c_int, i32p]
        lib.lfo_attention_chunked.restype = ctypes.c_int
        lib.lfo_attention_chunked.argtypes = [f32p, f32p, f32p, f32p, f32p, f32p, f64p,
                                              ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                              ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                              ctypes.c_double, i64p, ctypes.c_int64,
                                              ctypes.c_int]
        lib.lfo_attention_grad.restype = ctypes.c_int
        lib.lfo_attention_grad.argtypes = [f32p, f32p, f32p, f32p, f64p, f64p, f64p,
                                           ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                           ctypes.c_int, ctypes.c_int, i32p, ctypes.c_int,
                                           i32p, i32p, ctypes.c_int, ctypes.c_int,
                                           ctypes.c_int, ctypes.c_double, ctypes.c_int]
        lib.lfo_attention_grad_ex.restype = ctypes.c_int
        lib.lfo_attention_grad_ex.argtypes = [f32p, f32p, f32p, f32p, f32p, f32p, f32p,
                                              f64p, f64p, f64p, f64p, f64p, f64p,
                                              ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                              ctypes.c_int, ctypes.c_int, i32p, ctypes.c_int,
                                              i32p, i32p, ctypes.c_int, ctypes.c_int,
                                              ctypes.c_int, ctypes.c_double, ctypes.c_int]
        lib.lfo_row_lse.restype = ctypes.c_int
        lib.lfo_row_lse.argtypes = [f32p, f32p, f64p, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                    ctypes.c_int, ctypes.c_int, i32p, ctypes.c_int, i32p, i32p,
                                    ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_double]
        lib.lfo_count_pairs_ex.restype = ctypes.c_int64
        lib.lfo_count_pairs_ex.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                           ctypes.c_int, i32p, ctypes.c_int, i32p, ctypes.c_int]
        _lib = lib
    return _lib


def _i32(a):
    if a is None:
        return None, None
    arr = np.ascontiguousarray(np.asarray(a, dtype=np.int32))
    return arr, arr.ctypes.data_as(ctypes.POINTER(ctypes.c_int))


def allowed_set(n: int, window: int, dilation: int, glob, i: int,
                causal: bool = False) -> np.ndarray:
    """Sorted key positions row i scores (one head).  causal: the band's left
    half and the row itself (no global tokens)."""
    lib = _load()
    g, gp = _i32(list(glob))
    keys = np.empty(n + len(g) + 1, dtype=np.int32)
    cnt = lib.lfo_allowed_set_ex(n, window, dilation, int(causal), gp, len(g), i,
                                 keys.ctypes.data_as(ctypes.POINTER(ctypes.c_int)))
    if cnt < 0:
        raise ValueError("oracle: invalid arguments (code %d)" % cnt)
    return keys[:cnt].copy()


def count_pairs(B: int, H: int, n: int, window: int, dilation=None, glob=(),
                batch_glob=None, causal: bool = False) -> int:
    """Total scored pairs over B x H x n rows, by explicit set construction.
    batch_glob: B lists, one global set per batch element (glob ignored)."""
    if batch_glob is not None:
        assert len(batch_glob) == B
        return sum(count_pairs(1, H, n, window, dilation, list(g), causal=causal)
                   for g in batch_glob)
    lib = _load()
    g, gp = _i32(list(glob))
    d, dp = _i32(dilation)
    cnt = lib.lfo_count_pairs_ex(B, H, n, window, dp, int(causal), gp, len(g))
    if cnt < 0:
        raise ValueError("oracle: invalid arguments (code %d)" % cnt)
    return int(cnt)


def attention(q, k, v, window: int, dilation=None, glob=(), scale: float = 0.0,
              rows=None, nthreads: int | None = None, qg=None, kg=None, vg=None,
              batch_glob=None, causal: bool = False) -> np.ndarray:
    """Oracle attention output in float64.

    q, k, v: float32 arrays [B, H, N, D] (bf16 data already widened).
    rows: None for every row (returns [B, H, N, D]) or flat indices
    (b*H + h)*N + i (returns [len(rows), D]).
    qg, kg, vg: the global rows' own projections (same shape), or None for q,
    k, v.  batch_glob: B lists, one global set per batch element (then glob is
    ignored), or None for glob shared by all.  causal: the band's left half
    and the row itself (no global tokens).
    """
    lib = _load()
    q = np.ascontiguousarray(q, dtype=np.float32)
    k = np.ascontiguousarray(k, dtype=np.float32)
    v = np.ascontiguousarray(v, dtype=np.float32)
    B, H, N, D = q.shape
    assert k.shape == q.shape and v.shape == q.shape
    proj = []
    for x in (qg, kg, vg):
        if x is None:
            proj.append(None)
        else:
            x = np.ascontiguousarray(x, dtype=np.float32)
            assert x.shape == q.shape
            proj.append(x)
    if batch_glob is not None:
        assert len(batch_glob) == B
        flat = [int(x) for lst in batch_glob for x in lst]
        offs = np.cumsum([0] + [len(lst) for lst in batch_glob]).astype(np.int32)
        g, gp = _i32(flat)
        go, gop = _i32(offs)
    else:
        g, gp = _i32(list(glob))
        go, gop = None, None
    d, dp = _i32(dilation)
    if d is not None:
        assert len(d) == H
    if nthreads is None:
        nthreads = os.cpu_count() or 1
    if rows is None:
        n_rows = B * H * N
        rp = None
        out = np.empty((B, H, N, D), dtype=np.float64)
    else:
        r = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
        n_rows = len(r)
        rp = r.ctypes.data_as(ctypes.POINTER(ctypes.c_int64))
        out = np.empty((n_rows, D), dtype=np.float64)
    f32p = ctypes.POINTER(ctypes.c_float)
    pp = [None if x is None else x.ctypes.data_as(f32p) for x in proj]
    st = lib.lfo_attention_ex(q.ctypes.data_as(f32p), k.ctypes.data_as(f32p),
                              v.ctypes.data_as(f32p), pp[0], pp[1], pp[2],
                              out.ctypes.data_as(ctypes.POINTER(ctypes.c_double)),
                              B, H, N, D, window, dp, int(causal), gp, gop, len(g),
                              float(scale), rp, n_rows, int(nthreads))
    if st != 0:
        raise ValueError("oracle: attention failed (code %d)" % st)
    return out


def allowed_set_chunked(n: int, chunk: int, n_memory: int, i: int) -> np.ndarray:
    """Sorted key positions row i scores under C x k chunked attention with
    n_memory memory tokens at positions 0..n_memory-1 (chunks start after)."""
    lib = _load()
    keys = np.empty(n + 1, dtype=np.int32)
    cnt = lib.lfo_allowed_set_chunked(n, chunk, n_memory, i,
                                      keys.ctypes.data_as(ctypes.POINTER(ctypes.c_int)))
    if cnt < 0:
        raise ValueError("oracle: invalid arguments (code %d)" % cnt)
    return keys[:cnt].copy()


def count_pairs_chunked(B: int, H: int, n: int, chunk: int, n_memory: int) -> int:
    """Total scored pairs under chunked attention, by explicit set construction."""
    return B * H * sum(len(allowed_set_chunked(n, chunk, n_memory, i)) for i in range(n))


def attention_chunked(q, k, v, chunk: int, n_memory: int, scale: float = 0.0, rows=None,
                      nthreads: int | None = None, qg=None, kg=None, vg=None) -> np.ndarray:
    """Oracle output under GMAT's C x k chunked attention with n_memory memory
    tokens (the memory rows take qg, kg, vg when given).  Shapes as attention()."""
    lib = _load()
    q = np.ascontiguousarray(q, dtype=np.float32)
    k = np.ascontiguousarray(k, dtype=np.float32)
    v = np.ascontiguousarray(v, dtype=np.float32)
    B, H, N, D = q.shape
    proj = [None if x is None else np.ascontiguousarray(x, dtype=np.float32)
            for x in (qg, kg, vg)]
    if nthreads is None:
        nthreads = os.cpu_count() or 1
    if rows is None:
        n_rows, rp = B * H * N, None
        out = np.empty((B, H, N, D), dtype=np.float64)
    else:
        r = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
        n_rows = len(r)
        rp = r.ctypes.data_as(ctypes.POINTER(ctypes.c_int64))
        out = np.empty((n_rows, D), dtype=np.float64)
    f32p = ctypes.POINTER(ctypes.c_float)
    pp = [None if x is None else x.ctypes.data_as(f32p) for x in proj]
    st = lib.lfo_attention_chunked(q.ctypes.data_as(f32p), k.ctypes.data_as(f32p),
                                   v.ctypes.data_as(f32p), pp[0], pp[1], pp[2],
                                   out.ctypes.data_as(ctypes.POINTER(ctypes.c_double)),
                                   B, H, N, D, chunk, n_memory, float(scale), rp, n_rows,
                                   int(nthreads))
    if st != 0:
        raise ValueError("oracle: chunked attention failed (code %d)" % st)
    return out


def attention_grad(q, k, v, do, window: int = 0, dilation=None, glob=(), batch_glob=None,
                   causal: bool = False, chunk: int = 0, n_memory: int = 0, scale: float = 0.0,
                   nthreads: int | None = None, qg=None, kg=None, vg=None):
    """Gradients (dq, dk, dv), float64 [B, H, N, D], of the attention output
    for the upstream gradient do, under the same patterns as attention() and
    attention_chunked() (chunk > 0).  With qg, kg, vg (the global rows' own
    projections; a missing one is q, k or v) returns (dq, dk, dv, dqg, dkg,
    dvg): the global rows' terms go to the last three."""
    lib = _load()
    q, k, v, do = (np.ascontiguousarray(x, dtype=np.float32) for x in (q, k, v, do))
    B, H, N, D = q.shape
    proj = not (qg is None and kg is None and vg is None)
    if proj:
        qg, kg, vg = (np.ascontiguousarray(y if y is not None else x, dtype=np.float32)
                      for x, y in ((q, qg), (k, kg), (v, vg)))
        for x in (qg, kg, vg):
            assert x.shape == q.shape
    if batch_glob is not None:
        flat = [int(x) for lst in batch_glob for x in lst]
        offs = np.cumsum([0] + [len(lst) for lst in batch_glob]).astype(np.int32)
        g, gp = _i32(flat)
        go, gop = _i32(offs)
    else:
        g, gp = _i32(list(glob))
        go, gop = None, None
    d, dp = _i32(dilation)
    if nthreads is None:
        nthreads = os.cpu_count() or 1
    out = [np.empty((B, H, N, D), dtype=np.float64) for _ in range(6 if proj else 3)]
    f32p = ctypes.POINTER(ctypes.c_float)
    f64p = ctypes.POINTER(ctypes.c_double)
    pin = [x.ctypes.data_as(f32p) if proj else None for x in ((qg, kg, vg) if proj else (0, 0, 0))]
    pout = [out[3 + x].ctypes.data_as(f64p) if proj else None for x in range(3)]
    st = lib.lfo_attention_grad_ex(q.ctypes.data_as(f32p), k.ctypes.data_as(f32p),
                                   v.ctypes.data_as(f32p), pin[0], pin[1], pin[2],
                                   do.ctypes.data_as(f32p), out[0].ctypes.data_as(f64p),
                                   out[1].ctypes.data_as(f64p), out[2].ctypes.data_as(f64p),
                                   pout[0], pout[1], pout[2], B, H, N, D, window, dp,
                                   int(causal), gp, gop, len(g), int(chunk), int(n_memory),
                                   float(scale), int(nthreads))
    if st != 0:
        raise ValueError("oracle: gradient failed (code %d)" % st)
    return tuple(out)


def row_lse(q, k, window: int = 0, dilation=None, glob=(), batch_glob=None, causal: bool = False,
            chunk: int = 0, n_memory: int = 0, scale: float = 0.0) -> np.ndarray:
    """Natural log-sum-exp of each row's scaled scores over its key set,
    float64 [B, H, N]; patterns as attention_grad()."""
    lib = _load()
    q, k = (np.ascontiguousarray(x, dtype=np.float32) for x in (q, k))
    B, H, N, D = q.shape
    if batch_glob is not None:
        flat = [int(x) for lst in batch_glob for x in lst]
        offs = np.cumsum([0] + [len(lst) for lst in batch_glob]).astype(np.int32)
        g, gp = _i32(flat)
        go, gop = _i32(offs)
    else:
        g, gp = _i32(list(glob))
        go, gop = None, None
    d, dp = _i32(dilation)
    out = np.empty((B, H, N), dtype=np.float64)
    f32p = ctypes.POINTER(ctypes.c_float)
    st = lib.lfo_row_lse(q.ctypes.data_as(f32p), k.ctypes.data_as(f32p),
                         out.ctypes.data_as(ctypes.POINTER(ctypes.c_double)), B, H, N, D,
                         window, dp, int(causal), gp, gop, len(g), int(chunk), int(n_memory),
                         float(scale))
    if st != 0:
        raise ValueError("oracle: row_lse failed (code %d)" % st)
    return out
