"""GPU parity of the causal band (lfattn_create_causal: the band's left half
and the row itself, no global tokens) against the CPU oracle: small shapes on
every element for both element types and both bf16 band kernels, a full-size
dilated character-LM shape on every element, and the key sets read out
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


def _run(inp):
    import torch
    wl = inp.wl
    dtype = L.LFATTN_BF16 if wl.dtype == "bf16" else L.LFATTN_F32
    h = L.lfattn_create_causal(wl.B, wl.H, wl.N, wl.D, dtype, wl.window, list(inp.dilation))
    try:
        q, k, v = to_device(inp)
        o = torch.full_like(q, float("nan"))
        L.lfattn_forward(h, q, k, v, o)
        torch.cuda.synchronize()
        pairs = L.lfattn_scored_pairs(h)
    finally:
        L.lfattn_destroy(h)
    return o.float().cpu().numpy().astype(np.float64), pairs


# (B, H, N, D, dtype, window, dilation, seed)
CASES = [
    (1, 1, 1, 64, "bf16", 512, None, 1),
    (1, 2, 37, 64, "bf16", 8, None, 2),
    (2, 2, 300, 64, "bf16", 40, [1, 3], 3),
    (1, 3, 333, 128, "bf16", 100, [1, 2, 5], 4),
    (1, 2, 500, 128, "f32", 64, [2, 1], 5),
    (2, 2, 1000, 128, "bf16", 256, None, 6),
    (1, 2, 4099, 64, "bf16", 300, [3, 1], 7),
    (1, 1, 300, 64, "f32", 1000, None, 8),
]


# bf16 runs both band kernels besides the host's own choice; fp32 has one.
ROW_CASES = [pytest.param(c, r, id="B%dH%dN%dD%d_%s_w%d" % c[:6] + "-rows%s" % r)
             for c in CASES for r in ([None, 64, 128] if c[4] == "bf16" else [None])]


@pytest.mark.parametrize("case,rows_mode", ROW_CASES)
def test_causal_every_element(case, rows_mode, monkeypatch):
    B, H, N, D, dt, window, dil, seed = case
    if rows_mode is not None:
        monkeypatch.setenv("LFATTN_BAND_ROWS", str(rows_mode))
    inp = W.small_case(B, H, N, D, dt, window, dilation=dil, seed=seed)
    say(f"causal {case} rows {rows_mode}")
    got, pairs = _run(inp)
    want = oracle.attention(inp.q, inp.k, inp.v, window, list(inp.dilation), causal=True)
    compare(got, want, dt, str(case))
    assert pairs == oracle.count_pairs(B, H, N, window, list(inp.dilation), causal=True)


def test_causal_dilated_charlm_shape_every_element():
    """The dilated character-LM shape (B 2, H 8, N 8192, D 64, bf16, window
    512, heads 6-7 dilated by 2), causal, every output element."""
    wl = W.BY_NAME["dilated_charlm_n8192"]
    inp = W.generate(wl)
    say("causal dilated char-LM shape, every row")
    got, pairs = _run(inp)
    assert np.all(np.isfinite(got)), "unwritten output rows"
    want = oracle.attention(inp.q, inp.k, inp.v, wl.window, list(inp.dilation), causal=True)
    compare(got, want, "bf16", "causal char-LM")
    assert pairs == oracle.count_pairs(wl.B, wl.H, wl.N, wl.window, list(inp.dilation),
                                       causal=True)


@pytest.mark.parametrize("rows_mode", [64, 128])
def test_causal_mask_readout(rows_mode, monkeypatch):
    """Key sets, bit-exact (Q = K = 0, one-hot V rows)."""
    import torch
    monkeypatch.setenv("LFATTN_BAND_ROWS", str(rows_mode))
    B, H, N, D, window, dil = 1, 3, 1100, 64, 200, [1, 2, 5]
    h = L.lfattn_create_causal(B, H, N, D, L.LFATTN_BF16, window, dil)
    q = torch.zeros((B, H, N, D), dtype=torch.bfloat16, device="cuda:0")
    v = torch.zeros_like(q)
    o = torch.empty_like(q)
    codes = []
    try:
        say(f"causal mask readout, {rows_mode}-row band workgroups")
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
        ((hh * N + i) * N + oracle.allowed_set(N, window, dil[hh], [], i, causal=True)
         .astype(np.int64)) for hh in range(H) for i in range(N)]))
    assert np.array_equal(got, want)
