"""GPU parity of GMAT's C x k chunked attention with a memory prefix
(lfattn_create_chunked) against the CPU oracle, on every output element: the
page's three (C x k, M) settings and ragged, memory-free and projected cases,
both element types and both bf16 band kernels; key sets read out
bit-exactly."""

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


# (B, H, D, dtype, C, k, M, extra main positions past the last full chunk, seed)
CASES = [
    (1, 4, 64, "bf16", 512, 4, 64, 0, 1),    # (512 x 4, 64)
    (1, 4, 64, "bf16", 8, 64, 64, 0, 2),     # (8 x 64, 64)
    (2, 2, 128, "bf16", 70, 2, 30, 0, 3),    # (70 x 2, 30)
    (1, 3, 64, "f32", 70, 2, 30, 0, 4),
    (1, 2, 128, "bf16", 50, 3, 7, 13, 5),    # ragged last chunk
    (2, 2, 64, "bf16", 40, 5, 0, 9, 6),      # no memory
    (1, 2, 64, "f32", 33, 4, 5, 1, 7),
]


def _case_ids(c):
    return "B%dH%dD%d_%s_C%dk%dM%d+%d" % c[:8]


# bf16 runs both band kernels besides the host's own choice; fp32 has one.
ROW_CASES = [pytest.param(c, r, id=_case_ids(c) + "-rows%s" % r)
             for c in CASES for r in ([None, 64, 128] if c[3] == "bf16" else [None])]


@pytest.mark.parametrize("proj", [False, True])
@pytest.mark.parametrize("case,rows_mode", ROW_CASES)
def test_chunked_every_element(case, rows_mode, proj, monkeypatch):
    import torch
    B, H, D, dt, C, k, M, extra, seed = case
    if rows_mode is not None:
        monkeypatch.setenv("LFATTN_BAND_ROWS", str(rows_mode))
    N = M + C * k + extra
    a = W.small_case(B, H, N, D, dt, 0, seed=seed)
    g = W.small_case(B, H, N, D, dt, 0, seed=seed + 1000) if proj else None
    dtype = L.LFATTN_BF16 if dt == "bf16" else L.LFATTN_F32
    h = L.lfattn_create_chunked(B, H, N, D, dtype, C, M)
    try:
        assert L.lfattn_global_list(h) == list(range(M))
        q, k_, v = to_device(a)
        o = torch.full_like(q, float("nan"))
        say(f"chunked {case} rows {rows_mode} proj {proj}")
        if proj:
            qg, kg, vg = to_device(g)
            L.lfattn_forward_global_proj(h, q, k_, v, qg, kg, vg, o)
        else:
            L.lfattn_forward(h, q, k_, v, o)
        torch.cuda.synchronize()
        pairs = L.lfattn_scored_pairs(h)
    finally:
        L.lfattn_destroy(h)
    got = o.float().cpu().numpy().astype(np.float64)
    kw = dict(qg=g.q, kg=g.k, vg=g.v) if proj else {}
    want = oracle.attention_chunked(a.q, a.k, a.v, C, M, **kw)
    compare(got, want, dt, f"{case} proj {proj}")
    assert pairs == oracle.count_pairs_chunked(B, H, N, C, M)


@pytest.mark.parametrize("rows_mode", [64, 128])
def test_chunked_mask_readout(rows_mode, monkeypatch):
    """Key sets, bit-exact (Q = K = 0, one-hot V rows), (70 x 3, 30) plus a
    ragged tail."""
    import torch
    monkeypatch.setenv("LFATTN_BAND_ROWS", str(rows_mode))
    B, H, D, C, M = 1, 2, 64, 70, 30
    N = M + C * 3 + 11
    h = L.lfattn_create_chunked(B, H, N, D, L.LFATTN_BF16, C, M)
    q = torch.zeros((B, H, N, D), dtype=torch.bfloat16, device="cuda:0")
    v = torch.zeros_like(q)
    o = torch.empty_like(q)
    codes = []
    try:
        say(f"chunked mask readout, {rows_mode}-row band workgroups")
        for c0 in range(0, N, D):
            v.zero_()
            n = min(D, N - c0)
            v[:, :, c0:c0 + n, :n] = torch.eye(n, dtype=torch.bfloat16, device=v.device)
            L.lfattn_forward(h, q, q, v, o)
            torch.cuda.synchronize()
            of = o.float()
            nz = of > 0
            rowmax = of.amax(dim=3, keepdim=True)
            assert bool(((of == rowmax) | ~nz).all()), f"unequal weights in chunk {c0}"
            idx = torch.nonzero(nz)
            bh = idx[:, 0] * H + idx[:, 1]
            codes.append(((bh * N + idx[:, 2]) * N + (c0 + idx[:, 3])).cpu().numpy())
    finally:
        L.lfattn_destroy(h)
    got = np.sort(np.concatenate(codes))
    want = np.sort(np.concatenate([
        ((hh * N + i) * N + oracle.allowed_set_chunked(N, C, M, i).astype(np.int64))
        for hh in range(H) for i in range(N)]))
    assert np.array_equal(got, want)
