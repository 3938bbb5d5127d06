"""GPU parity of the general form: one global set per batch element (created
from a [B, N] mask) and separate projections for the global rows, through the
C ABI against the CPU oracle.  Small shapes on every element (both bf16 band
kernels), a full-size Longformer-base shape with two batch elements on every
element, the allowed key sets read out bit-exactly, and the reductions to the
plain entry points (bit-identical outputs)."""

import numpy as np
import pytest

import oracle
from long_context_sparse_band_amd import lfattn as L
from long_context_sparse_band_amd import workloads as W
from gpu_util import compare, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    L.load()


def _dev(a, dt):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a)).to("cuda:0")
    return (t.to(torch.bfloat16) if dt == "bf16" else t).contiguous()


def _mask(B, N, sets):
    m = np.zeros((B, N), dtype=np.uint8)
    for b, s in enumerate(sets):
        m[b, list(s)] = 1
    return m


def _run(B, H, N, D, dt, window, dil, sets, seed, proj=True, rows=None):
    """Inputs (q, k, v and, with proj, qg, kg, vg from a second seed), the GPU
    output through lfattn_create_masked + lfattn_forward_global_proj, and the
    oracle's (on `rows` only, if given)."""
    import torch
    a = W.small_case(B, H, N, D, dt, window, dilation=dil, seed=seed)
    g = W.small_case(B, H, N, D, dt, window, dilation=dil, seed=seed + 1000) if proj else None
    dtype = L.LFATTN_BF16 if dt == "bf16" else L.LFATTN_F32
    h = L.lfattn_create_masked(B, H, N, D, dtype, window, list(a.dilation), _mask(B, N, sets))
    try:
        for b in range(B):
            assert L.lfattn_global_list_batch(h, b) == sorted(set(sets[b]))
        q, k, v = (_dev(x, dt) for x in (a.q, a.k, a.v))
        qg, kg, vg = ((_dev(x, dt) for x in (g.q, g.k, g.v)) if proj else (None, None, None))
        o = torch.full_like(q, float("nan"))
        L.lfattn_forward_global_proj(h, q, k, v, qg, kg, vg, o)
        torch.cuda.synchronize()
        pairs = L.lfattn_scored_pairs(h)
    finally:
        L.lfattn_destroy(h)
    got = o.float().cpu().numpy().astype(np.float64)
    kw = dict(qg=g.q, kg=g.k, vg=g.v) if proj else {}
    want = oracle.attention(a.q, a.k, a.v, window, list(a.dilation), batch_glob=sets,
                            rows=rows, **kw)
    return got, want, pairs, a


# (B, H, N, D, dtype, window, dilation, per-batch global sets, seed)
CASES = [
    (2, 2, 300, 64, "bf16", 40, [1, 3], [[5, 100, 299], [0]], 1),
    (3, 1, 257, 128, "bf16", 100, None, [[], [256, 1], [7]], 2),
    (2, 2, 200, 64, "f32", 30, [2, 1], [[0, 199], [50]], 3),
    (2, 3, 1000, 128, "bf16", 256, [1, 2, 1], [list(range(0, 1000, 9)), [999]], 4),
    (2, 1, 700, 64, "bf16", 128, [3], [list(range(0, 700, 7)), list(range(3, 700, 11))], 5),
    (2, 2, 129, 128, "f32", 2, [1, 64], [[64, 128], []], 6),
]


# bf16 runs both band kernels (64- and 128-row workgroups) besides the host's
# own choice; fp32 has one band kernel.
ROW_CASES = [pytest.param(c, r, id="B%dH%dN%dD%d_%s_s%d-rows%s" % (
    c[0], c[1], c[2], c[3], c[4], c[8], r)) for c in CASES
    for r in ([None, 64, 128] if c[4] == "bf16" else [None])]


@pytest.mark.parametrize("case,rows_mode", ROW_CASES)
def test_per_batch_sets_and_projections_every_element(case, rows_mode, monkeypatch):
    B, H, N, D, dt, window, dil, sets, seed = case
    if rows_mode is not None:
        monkeypatch.setenv("LFATTN_BAND_ROWS", str(rows_mode))
    say(f"per-batch sets + projections {case} rows {rows_mode}")
    got, want, pairs, _ = _run(B, H, N, D, dt, window, dil, sets, seed)
    compare(got, want, dt, str(case))
    assert pairs == oracle.count_pairs(B, H, N, window, dil or [1] * H, batch_glob=sets)


def test_no_projections_is_the_plain_forward():
    import torch
    a = W.small_case(2, 2, 500, 64, "bf16", 64, dilation=[1, 2], glob=[0, 250], seed=7)
    h = L.lfattn_create(2, 2, 500, 64, L.LFATTN_BF16, 64, [1, 2], [0, 250])
    try:
        q, k, v = (_dev(x, "bf16") for x in (a.q, a.k, a.v))
        o1, o2 = torch.empty_like(q), torch.empty_like(q)
        say("global projections NULL vs plain forward")
        L.lfattn_forward(h, q, k, v, o1)
        L.lfattn_forward_global_proj(h, q, k, v, None, None, None, o2)
        torch.cuda.synchronize()
        assert torch.equal(o1, o2)
    finally:
        L.lfattn_destroy(h)


def test_mask_with_equal_rows_is_the_list_create():
    import torch
    B, H, N, D = 3, 2, 600, 128
    a = W.small_case(B, H, N, D, "bf16", 90, dilation=[2, 1], seed=8)
    q, k, v = (_dev(x, "bf16") for x in (a.q, a.k, a.v))
    glob = [3, 77, 599]
    h1 = L.lfattn_create(B, H, N, D, L.LFATTN_BF16, 90, [2, 1], glob)
    h2 = L.lfattn_create_masked(B, H, N, D, L.LFATTN_BF16, 90, [2, 1], _mask(B, N, [glob] * B))
    try:
        o1, o2 = torch.empty_like(q), torch.empty_like(q)
        say("masked create with equal rows vs list create")
        L.lfattn_forward(h1, q, k, v, o1)
        L.lfattn_forward(h2, q, k, v, o2)
        torch.cuda.synchronize()
        assert torch.equal(o1, o2)
        assert L.lfattn_scored_pairs(h1) == L.lfattn_scored_pairs(h2)
    finally:
        L.lfattn_destroy(h1)
        L.lfattn_destroy(h2)


def test_longformer_base_shape_two_sequences_every_element():
    """Longformer-base shape (H 12, N 4096, D 64, bf16, window 512) with two
    sequences of different global sets ([CLS] + 31 question tokens; [CLS] + 10
    seeded positions) and their own global projections, every output element."""
    B, H, N, D, window = 2, 12, 4096, 64, 512
    rng = np.random.default_rng(9)
    sets = [list(range(32)), sorted({0} | set(rng.choice(N, size=10, replace=False).tolist()))]
    say("Longformer-base shape, two sequences, every row")
    got, want, pairs, _ = _run(B, H, N, D, "bf16", window, None, sets, 20261)
    assert np.all(np.isfinite(got)), "unwritten output rows"
    compare(got, want, "bf16", "longformer-base two sequences")
    assert pairs == oracle.count_pairs(B, H, N, window, None, batch_glob=sets)


@pytest.mark.parametrize("rows_mode", [64, 128])
def test_mask_readout_per_batch_sets(rows_mode, monkeypatch):
    """Allowed key sets, bit-exact: Q = K = Qg = Kg = 0 weighs every scored key
    of a row equally, and one-hot V (= Vg) rows show which keys those are."""
    import torch
    monkeypatch.setenv("LFATTN_BAND_ROWS", str(rows_mode))
    B, H, N, D, window, dil = 2, 2, 700, 64, 128, [1, 3]
    sets = [[0, 5, 350, 699], [100]]
    h = L.lfattn_create_masked(B, H, N, D, L.LFATTN_BF16, window, dil, _mask(B, N, sets))
    q = torch.zeros((B, H, N, D), dtype=torch.bfloat16, device="cuda:0")
    v = torch.zeros_like(q)
    o = torch.empty_like(q)
    codes = []
    try:
        say(f"per-batch mask readout, {rows_mode}-row band workgroups")
        for c0 in range(0, N, D):
            v.zero_()
            n = min(D, N - c0)
            v[:, :, c0:c0 + n, :n] = torch.eye(n, dtype=torch.bfloat16, device=v.device)
            L.lfattn_forward_global_proj(h, q, q, v, q, q, v, o)
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
    want = []
    for b in range(B):
        for hh in range(H):
            for i in range(N):
                keys = oracle.allowed_set(N, window, dil[hh], sets[b], i).astype(np.int64)
                want.append(((b * H + hh) * N + i) * N + keys)
    want = np.sort(np.concatenate(want))
    assert np.array_equal(got, want)
