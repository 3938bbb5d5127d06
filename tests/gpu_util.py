"""Helpers for the GPU tests: upload seeded inputs, run the library through its
C ABI, and compare with the oracle at the stated tolerances."""

from __future__ import annotations

import sys

import numpy as np

from long_context_sparse_band_amd import lfattn as L

# Tolerances: fp32 max-abs 1e-5; bf16 (inputs rounded to bf16, oracle on the
# rounded values) max-abs 2e-2 and mean-abs 2e-3.
TOL = {"f32": dict(max_abs=1e-5, mean_abs=1e-5), "bf16": dict(max_abs=2e-2, mean_abs=2e-3)}


def say(msg: str):
    """Name the case before each GPU step (flushed, so a crash still shows it)."""
    print(msg, flush=True)
    sys.stdout.flush()


def to_device(inp):
    import torch
    tens = []
    for a in (inp.q, inp.k, inp.v):
        t = torch.from_numpy(a).to("cuda:0")
        if inp.wl.dtype == "bf16":
            t = t.to(torch.bfloat16)  # exact: the values are bf16 already
        tens.append(t.contiguous())
    return tens


def run(inp, glob=None, scale=0.0, stream=None, handle=None, out=None):
    """One forward through the C ABI; returns (output float64 numpy, pairs)."""
    import torch
    wl = inp.wl
    q, k, v = to_device(inp)
    o = out if out is not None else torch.empty_like(q)
    dtype = L.LFATTN_BF16 if wl.dtype == "bf16" else L.LFATTN_F32
    g = list(inp.glob) if glob is None else list(glob)
    own = handle is None
    h = handle or L.lfattn_create(wl.B, wl.H, wl.N, wl.D, dtype, wl.window,
                                  list(inp.dilation), g, scale)
    try:
        L.lfattn_forward(h, q, k, v, o, stream)
        torch.cuda.synchronize()
        pairs = L.lfattn_scored_pairs(h)
    finally:
        if own:
            L.lfattn_destroy(h)
    return o.float().cpu().numpy().astype(np.float64), pairs


def compare(got, want, dtype, what=""):
    err = np.abs(got - want)
    tol = TOL[dtype]
    mx, mean = float(err.max()) if err.size else 0.0, float(err.mean()) if err.size else 0.0
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    assert mx <= tol["max_abs"], f"{what}: max-abs {mx:.3g} > {tol['max_abs']}"
    assert mean <= tol["mean_abs"], f"{what}: mean-abs {mean:.3g} > {tol['mean_abs']}"
    return mx, mean
