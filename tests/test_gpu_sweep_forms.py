"""Seeded random sweep of the general forms on the GPU, every output element
against the oracle: per-batch global sets with the global rows' own
projections, the causal band, and chunked attention with a memory prefix, for
both element types, D = 64 and 128, and (bf16) both band kernels."""

import numpy as np
import pytest

import oracle
from long_context_sparse_band_amd import lfattn as L
from long_context_sparse_band_amd import workloads as W
from gpu_util import compare, say, to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    L.load()


def _forward(h, inp, proj=None):
    import torch
    q, k, v = to_device(inp)
    o = torch.full_like(q, float("nan"))
    if proj is None:
        L.lfattn_forward(h, q, k, v, o)
    else:
        qg, kg, vg = to_device(proj)
        L.lfattn_forward_global_proj(h, q, k, v, qg, kg, vg, o)
    torch.cuda.synchronize()
    return o.float().cpu().numpy().astype(np.float64), L.lfattn_scored_pairs(h)


@pytest.mark.parametrize("form", ["masked_proj", "causal", "chunked"])
def test_random_forms(form, monkeypatch):
    rng = np.random.default_rng({"masked_proj": 101, "causal": 102, "chunked": 103}[form])
    for t in range(12):
        B, H = int(rng.integers(1, 4)), int(rng.integers(1, 4))
        N = int(rng.integers(1, 700))
        D = int(rng.choice([64, 128]))
        dt = str(rng.choice(["f32", "bf16"]))
        rows = int(rng.choice([64, 128])) if dt == "bf16" else None
        if rows:
            monkeypatch.setenv("LFATTN_BAND_ROWS", str(rows))
        else:
            monkeypatch.delenv("LFATTN_BAND_ROWS", raising=False)
        dtype = L.LFATTN_BF16 if dt == "bf16" else L.LFATTN_F32
        seed = 5000 + 100 * t + len(form)
        if form == "masked_proj":
            window = int(rng.integers(0, 2 * N + 3))
            dil = [int(x) for x in rng.integers(1, 5, size=H)]
            sets = []
            for _ in range(B):
                n_g = int(rng.integers(0, min(N, 40) + 1))
                sets.append(sorted(rng.choice(N, size=n_g, replace=False).tolist()) if n_g else [])
            mask = np.zeros((B, N), dtype=np.uint8)
            for b, s in enumerate(sets):
                mask[b, s] = 1
            inp = W.small_case(B, H, N, D, dt, window, dilation=dil, seed=seed)
            proj = W.small_case(B, H, N, D, dt, window, dilation=dil, seed=seed + 1)
            say(f"sweep {form} {t}: B{B} H{H} N{N} D{D} {dt} rows {rows} w{window} dil{dil} "
                f"|G_b| {[len(s) for s in sets]}")
            h = L.lfattn_create_masked(B, H, N, D, dtype, window, dil, mask)
            try:
                got, pairs = _forward(h, inp, proj)
            finally:
                L.lfattn_destroy(h)
            want = oracle.attention(inp.q, inp.k, inp.v, window, dil, batch_glob=sets,
                                    qg=proj.q, kg=proj.k, vg=proj.v)
            want_pairs = oracle.count_pairs(B, H, N, window, dil, batch_glob=sets)
        elif form == "causal":
            window = int(rng.integers(0, 2 * N + 3))
            dil = [int(x) for x in rng.integers(1, 5, size=H)]
            inp = W.small_case(B, H, N, D, dt, window, dilation=dil, seed=seed)
            say(f"sweep {form} {t}: B{B} H{H} N{N} D{D} {dt} rows {rows} w{window} dil{dil}")
            h = L.lfattn_create_causal(B, H, N, D, dtype, window, dil)
            try:
                got, pairs = _forward(h, inp)
            finally:
                L.lfattn_destroy(h)
            want = oracle.attention(inp.q, inp.k, inp.v, window, dil, causal=True)
            want_pairs = oracle.count_pairs(B, H, N, window, dil, causal=True)
        else:
            chunk = int(rng.integers(1, 200))
            M = int(rng.integers(0, min(N, 70) + 1))
            inp = W.small_case(B, H, N, D, dt, 0, seed=seed)
            proj = W.small_case(B, H, N, D, dt, 0, seed=seed + 1) if rng.random() < 0.5 else None
            say(f"sweep {form} {t}: B{B} H{H} N{N} D{D} {dt} rows {rows} C{chunk} M{M} "
                f"proj {proj is not None}")
            h = L.lfattn_create_chunked(B, H, N, D, dtype, chunk, M)
            try:
                got, pairs = _forward(h, inp, proj)
            finally:
                L.lfattn_destroy(h)
            kw = dict(qg=proj.q, kg=proj.k, vg=proj.v) if proj is not None else {}
            want = oracle.attention_chunked(inp.q, inp.k, inp.v, chunk, M, **kw)
            want_pairs = oracle.count_pairs_chunked(B, H, N, chunk, M)
        compare(got, want, dt, f"{form} sweep {t}")
        assert pairs == want_pairs
