"""GPU parity of the backward pass (lfattn_backward, bf16, D = 64 and 128): dQ,
dK, dV against the oracle's double-precision gradients on the same
bf16-valued inputs, every pattern, both forward band kernels feeding the
log-sum-exp."""

import numpy as np
import pytest

import oracle
from long_context_sparse_band_amd import lfattn as L
from long_context_sparse_band_amd import workloads as W
from gpu_util import moving_max_case, say, to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    L.load()


def _bf16(x):
    return W.bf16_bits_to_f32(W.bf16_round_bits(x)).reshape(x.shape)


# Gradient tolerances relative to the reference's largest magnitude: the
# weights P and dS enter the MFMAs rounded to bf16 (relative error 2^-9, a
# few such roundings summed over a row's keys) and Delta is taken from the
# bf16 output O.  Measured: max about 4e-3, mean about 2.5e-4 of that scale.
REL_MAX, REL_MEAN = 1e-2, 1e-3


def check(got, want, what):
    # Floor of the scale: where the exact gradient cancels to zero (one key
    # per row: dS = P (dP - Delta) = 0) fp32 leaves residues of about 1e-7
    # of the O(1..10) terms that cancel.
    ref = max(1e-3, float(np.abs(want).max()))
    err = np.abs(got - want)
    assert np.all(np.isfinite(got)), f"{what}: non-finite"
    assert err.max() <= REL_MAX * ref, f"{what}: max-abs {err.max():.3g} (ref max {ref:.3g})"
    assert err.mean() <= REL_MEAN * ref, f"{what}: mean-abs {err.mean():.3g} (ref max {ref:.3g})"
    return err.max() / ref, err.mean() / ref


CASES = [
    ("band", dict(B=1, H=2, N=300, window=64, dil=[1, 2], glob=[0, 150])),
    ("band", dict(B=2, H=1, N=700, window=256, dil=[1], glob=list(range(0, 700, 23)))),
    ("band", dict(B=1, H=2, N=129, window=1000, dil=[1, 3], glob=[])),
    ("masked", dict(B=2, H=2, N=400, window=40, dil=[1, 2], sets=[[3, 200, 399], []])),
    ("causal", dict(B=1, H=2, N=500, window=100, dil=[1, 2])),
    ("chunked", dict(B=1, H=2, N=20 + 64 * 3 + 7, chunk=64, M=20)),
    ("band", dict(B=1, H=1, N=1, window=8, dil=[1], glob=[])),
    ("band", dict(B=1, H=1, N=65, window=16, dil=[3], glob=[64])),
    ("causal", dict(B=2, H=1, N=1, window=4, dil=[1])),
    # 512 global positions (the most a bf16 handle takes); every position global.
    ("band", dict(B=1, H=1, N=600, window=32, dil=[1], glob=[i * 599 // 511 for i in range(512)])),
    ("band", dict(B=1, H=2, N=96, window=16, dil=[1, 2], glob=list(range(96)))),
]


# D, query-side wavefronts per SIMD (D = 64: the 3- and 4-wavefront kernels).
KERNELS = [(64, 3), (64, 4), (128, 2)]


@pytest.mark.parametrize("D,wpe", KERNELS, ids=["D%d-w%d" % k for k in KERNELS])
@pytest.mark.parametrize("rows_mode", [64, 128])
@pytest.mark.parametrize("case", CASES, ids=lambda c: c[0] + "_N%d" % c[1]["N"])
def test_backward_every_element(case, rows_mode, D, wpe, monkeypatch):
    import torch
    # Both forward band kernels (the log-sum-exp), both backward item sizes
    # (64 rows with split tiles, 128 rows with one tile stream) and both
    # query-side kernels at D = 64.
    monkeypatch.setenv("LFATTN_BAND_ROWS", str(rows_mode))
    monkeypatch.setenv("LFATTN_BWD_ROWS", str(rows_mode))
    if D == 64:
        monkeypatch.setenv("LFATTN_BWD_ROWS_WPE", str(wpe))
    kind, p = case
    B, H, N = p["B"], p["H"], p["N"]
    a = W.small_case(B, H, N, D, "bf16", p.get("window", 0), dilation=p.get("dil"), seed=88)
    rng = np.random.default_rng(89)
    do = _bf16(rng.standard_normal((B, H, N, D)).astype(np.float32))
    if kind == "band":
        h = L.lfattn_create(B, H, N, D, L.LFATTN_BF16, p["window"], p["dil"], p["glob"])
        kw = dict(window=p["window"], dilation=p["dil"], glob=p["glob"])
    elif kind == "masked":
        mask = np.zeros((B, N), dtype=np.uint8)
        for b, s in enumerate(p["sets"]):
            mask[b, s] = 1
        h = L.lfattn_create_masked(B, H, N, D, L.LFATTN_BF16, p["window"], p["dil"], mask)
        kw = dict(window=p["window"], dilation=p["dil"], batch_glob=p["sets"])
    elif kind == "causal":
        h = L.lfattn_create_causal(B, H, N, D, L.LFATTN_BF16, p["window"], p["dil"])
        kw = dict(window=p["window"], dilation=p["dil"], causal=True)
    else:
        h = L.lfattn_create_chunked(B, H, N, D, L.LFATTN_BF16, p["chunk"], p["M"])
        kw = dict(chunk=p["chunk"], n_memory=p["M"])
    try:
        q, k, v = to_device(a)
        g = torch.from_numpy(do).to("cuda:0").to(torch.bfloat16)
        o = torch.empty_like(q)
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
        dq, dk, dv = (torch.full((B, H, N, D), float("nan"), dtype=torch.float32,
                                 device=q.device) for _ in range(3))
        say(f"backward {kind} {p} D {D} rows {rows_mode}")
        L.lfattn_forward_lse(h, q, k, v, o, lse)
        L.lfattn_backward(h, q, k, v, o, g, lse, dq, dk, dv)
        torch.cuda.synchronize()
    finally:
        L.lfattn_destroy(h)
    want = oracle.attention_grad(a.q, a.k, a.v, do, **kw)
    errs = [check(x.cpu().numpy().astype(np.float64), w, f"{kind} {n}")
            for x, w, n in zip((dq, dk, dv), want, ("dq", "dk", "dv"))]
    say(f"  relative max/mean errors dq dk dv: {errs}")


# Scores that rise along the keys (up to about 100) or are large at random
# (standard deviation about 16): softmax weights near one-hot, log-sum-exp
# far from zero.
BIG_SCORES = [
    ("rising", 1, 2, 600, 64, 512, [1, 2], [0, 300, 599]),
    ("rising", 1, 1, 500, 128, 200, [1], [5]),
    ("large", 1, 2, 700, 64, 256, [1, 3], [0, 1, 699]),
    ("large", 1, 2, 400, 128, 128, [1, 2], [7]),
]


@pytest.mark.parametrize("rows_mode", [64, 128])
@pytest.mark.parametrize("case", BIG_SCORES, ids=lambda c: "%s_N%dD%d" % (c[0], c[3], c[4]))
def test_backward_large_scores(case, rows_mode, monkeypatch):
    import torch
    monkeypatch.setenv("LFATTN_BAND_ROWS", str(rows_mode))
    monkeypatch.setenv("LFATTN_BWD_ROWS", str(rows_mode))
    kind, B, H, N, D, window, dil, glob = case
    a = moving_max_case(kind, B, H, N, D, "bf16", window, dil, glob, seed=500 + N)
    rng = np.random.default_rng(501 + N)
    do = _bf16(rng.standard_normal((B, H, N, D)).astype(np.float32))
    h = L.lfattn_create(B, H, N, D, L.LFATTN_BF16, window, dil, glob)
    try:
        q, k, v = to_device(a)
        g = torch.from_numpy(do).to("cuda:0").to(torch.bfloat16)
        o = torch.empty_like(q)
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
        dq, dk, dv = (torch.full((B, H, N, D), float("nan"), dtype=torch.float32,
                                 device=q.device) for _ in range(3))
        say(f"backward, large scores: {case}, rows {rows_mode}")
        L.lfattn_forward_lse(h, q, k, v, o, lse)
        L.lfattn_backward(h, q, k, v, o, g, lse, dq, dk, dv)
        torch.cuda.synchronize()
    finally:
        L.lfattn_destroy(h)
    kw = dict(window=window, dilation=dil, glob=glob)
    want = oracle.attention_grad(a.q, a.k, a.v, do, **kw)
    want_lse = oracle.row_lse(a.q, a.k, **kw)
    err = np.abs(lse.cpu().numpy().astype(np.float64) - want_lse)
    assert err.max() <= 1e-2, f"{kind}: LSE max-abs {err.max():.3g}"
    # The backward takes Delta = dO . O from the O it is given (the forward's
    # bf16 output), so it computes the gradient with dS' = P (dP - Delta -
    # dDelta) = dS - P dDelta: dQ' = dQ - scale dDelta (P K) and dK' = dK -
    # scale P^T (dDelta Q).  Both terms come from the oracle (attention with
    # K as the values; the value gradient for the upstream gradient dDelta Q).
    o_got = o.float().cpu().numpy().astype(np.float64)
    ddelta = np.sum(do.astype(np.float64) * (o_got - oracle.attention(a.q, a.k, a.v, **kw)),
                    axis=-1)
    scale = 1.0 / np.sqrt(D)
    pk = oracle.attention(a.q, a.k, a.k, **kw)
    ptq = oracle.attention_grad(a.q, a.k, a.v, ddelta[..., None] * a.q, **kw)[2]
    want = (want[0] - scale * ddelta[..., None] * pk, want[1] - scale * ptq, want[2])
    # dS enters the dS K and dS^T Q products rounded to bf16 (relative error
    # at most 2^-9), so dQ_i can be off by up to scale 2^-9 sum_j |dS_ij| |K_j|
    # (and dK_j by scale 2^-9 sum_i |dS_ij| |Q_i|): terms that the exact
    # gradient cancels (it does not change when every key moves by one
    # vector) but this rounding does not.  Here the keys share a large common
    # direction, and that bound (doubled), not the plain relative one, is
    # the measure.  |dS| from the dense masked softmax of each head.
    extra = [np.zeros_like(want[0]), np.zeros_like(want[1])]
    for b in range(B):
        for hh in range(H):
            qh, kh_, vh = (x[b, hh].astype(np.float64) for x in (a.q, a.k, a.v))
            allowed = np.zeros((N, N), dtype=bool)
            for i in range(N):
                allowed[i, oracle.allowed_set(N, window, dil[hh], glob, i)] = True
            sc = np.where(allowed, scale * (qh @ kh_.T), -np.inf)
            pm = np.exp(sc - sc.max(axis=1, keepdims=True))
            pm /= pm.sum(axis=1, keepdims=True)
            dp = do[b, hh].astype(np.float64) @ vh.T
            dsm = np.abs(pm * (dp - np.sum(do[b, hh] * o_got[b, hh], axis=1)[:, None]))
            extra[0][b, hh] = 2 * scale * 2.0 ** -9 * (dsm @ np.abs(kh_))
            extra[1][b, hh] = 2 * scale * 2.0 ** -9 * (dsm.T @ np.abs(qh))
    for i, (x, w, n) in enumerate(zip((dq, dk, dv), want, ("dq", "dk", "dv"))):
        got = x.cpu().numpy().astype(np.float64)
        assert np.all(np.isfinite(got)), f"{kind} {n}: non-finite"
        ref = max(1e-3, float(np.abs(w).max()))
        allow = REL_MAX * ref + (extra[i] if i < 2 else 0.0)
        over = np.abs(got - w) - allow
        say(f"  {n}: max-abs {np.abs(got - w).max():.3g}, worst margin {over.max():.3g}")
        assert over.max() <= 0, f"{kind} {n}: max-abs {np.abs(got - w).max():.3g} over the bound"
        assert np.abs(got - w).mean() <= REL_MEAN * ref + (extra[i].mean() if i < 2 else 0.0)


FULL = ["longformer_base_n4096", "dilated_charlm_n8192", "gmat_memory_m64_l16384",
        "long_stress_n65536_d128"]


@pytest.mark.parametrize("bwd_rows", [64, 128])
@pytest.mark.parametrize("name", FULL)
def test_backward_full_size(name, bwd_rows, monkeypatch):
    """At the full sizes: the whole launch over every head, checked element
    by element on every head up to 16448 tokens, and on the first and last
    heads of the 65536-token workload (heads are independent; its oracle
    takes seconds per head)."""
    import torch
    monkeypatch.setenv("LFATTN_BWD_ROWS", str(bwd_rows))
    wl = W.BY_NAME[name]
    a = W.generate(wl)
    B, H, N, D = wl.B, wl.H, wl.N, wl.D
    rng = np.random.default_rng(wl.seed + 7)
    do = _bf16(rng.standard_normal((B, H, N, D)).astype(np.float32))
    h = L.lfattn_create(B, H, N, D, L.LFATTN_BF16, wl.window, list(a.dilation), list(a.glob))
    try:
        q, k, v = to_device(a)
        g = torch.from_numpy(do).to("cuda:0").to(torch.bfloat16)
        o = torch.empty_like(q)
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
        dq, dk, dv = (torch.full((B, H, N, D), float("nan"), dtype=torch.float32,
                                 device=q.device) for _ in range(3))
        say(f"backward full size {name}")
        L.lfattn_forward_lse(h, q, k, v, o, lse)
        L.lfattn_backward(h, q, k, v, o, g, lse, dq, dk, dv)
        torch.cuda.synchronize()
    finally:
        L.lfattn_destroy(h)
    hs = list(range(H)) if N <= 16448 else [0, H - 1]
    want = oracle.attention_grad(a.q[:, hs], a.k[:, hs], a.v[:, hs], do[:, hs],
                                 window=wl.window, dilation=[int(a.dilation[x]) for x in hs],
                                 glob=list(a.glob))
    for x, w, n in zip((dq, dk, dv), want, ("dq", "dk", "dv")):
        assert np.all(np.isfinite(x.cpu().numpy())), f"{name} {n}: non-finite"
        say(f"  {n}: {check(x[:, hs].cpu().numpy().astype(np.float64), w, f'{name} {n}')}")


def test_backward_timing_records_each_call():
    import torch
    B, H, N, D = 1, 2, 512, 64
    a = W.small_case(B, H, N, D, "bf16", 128, seed=5)
    h = L.lfattn_create(B, H, N, D, L.LFATTN_BF16, 128, [1, 1], [0])
    try:
        q, k, v = to_device(a)
        o = torch.empty_like(q)
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
        dq, dk, dv = (torch.empty((B, H, N, D), dtype=torch.float32, device=q.device)
                      for _ in range(3))
        say("backward timing")
        L.lfattn_forward_lse(h, q, k, v, o, lse)
        L.lfattn_set_timing(h, True)
        for _ in range(3):
            L.lfattn_backward(h, q, k, v, o, q, lse, dq, dk, dv)
        rows, keys, merge, n = L.lfattn_read_backward_timing(h)
        assert n == 3 and rows > 0 and keys > 0 and merge > 0
        assert L.lfattn_read_backward_timing(h)[3] == 0
        L.lfattn_set_timing(h, False)
    finally:
        L.lfattn_destroy(h)


def test_backward_rejects_bad_arguments():
    """Error paths, all taken before any kernel launch: handles the backward
    does not support (fp32), misaligned pointers, outputs overlapping an
    input or each other."""
    import torch
    dev = "cuda:0"
    B, H, N = 1, 1, 64
    for dtype, D in ((L.LFATTN_F32, 64), (L.LFATTN_F32, 128)):
        h = L.lfattn_create(B, H, N, D, dtype, 8, None, [0])
        try:
            t = torch.zeros((B, H, N, D), dtype=torch.float32, device=dev)
            lse = torch.zeros((B, H, N), dtype=torch.float32, device=dev)
            g = [torch.zeros_like(t) for _ in range(3)]
            with pytest.raises(L.LfattnError) as e:
                L.lfattn_backward(h, t, t, t, t, t, lse, *g)
            assert e.value.status == L.LFATTN_EUNSUPPORTED
        finally:
            L.lfattn_destroy(h)
    D = 64
    h = L.lfattn_create(B, H, N, D, L.LFATTN_BF16, 8, None, [0])
    try:
        x = torch.zeros((B, H, N, D), dtype=torch.bfloat16, device=dev)
        lse = torch.zeros((B, H, N), dtype=torch.float32, device=dev)
        outs = [torch.zeros((B, H, N, D), dtype=torch.float32, device=dev) for _ in range(3)]
        buf = torch.zeros(B * H * N * D + 8, dtype=torch.bfloat16, device=dev)
        say("backward argument checks")
        cases = [
            ("misaligned input", (buf.data_ptr() + 2, x, x, x, x, lse, *outs)),
            ("dQ overlaps dK", (x, x, x, x, x, lse, outs[0], outs[0], outs[2])),
            ("dV overlaps the log-sum-exp", (x, x, x, x, x, outs[2], outs[0], outs[1], outs[2])),
            ("null dK", (x, x, x, x, x, lse, outs[0], None, outs[2])),
        ]
        for what, args in cases:
            with pytest.raises(L.LfattnError) as e:
                L.lfattn_backward(h, *args)
            assert e.value.status == L.LFATTN_EINVAL, what
    finally:
        L.lfattn_destroy(h)


@pytest.mark.parametrize("rows_mode", [64, 128])
def test_forward_and_backward_at_the_global_limit(rows_mode, monkeypatch):
    """512 distinct global positions (the bf16 maximum), seeded and spread
    over a 1200-token sequence with dilation: forward output and all three
    gradients element by element."""
    import torch
    monkeypatch.setenv("LFATTN_BAND_ROWS", str(rows_mode))
    monkeypatch.setenv("LFATTN_BWD_ROWS", str(rows_mode))
    B, H, N, D, window, dil = 1, 2, 1200, 64, 48, [1, 3]
    rng = np.random.default_rng(90)
    glob = sorted(rng.choice(N, size=512, replace=False).tolist())
    a = W.small_case(B, H, N, D, "bf16", window, dilation=dil, glob=glob, seed=91)
    do = _bf16(rng.standard_normal((B, H, N, D)).astype(np.float32))
    h = L.lfattn_create(B, H, N, D, L.LFATTN_BF16, window, dil, glob)
    try:
        q, k, v = to_device(a)
        g = torch.from_numpy(do).to("cuda:0").to(torch.bfloat16)
        o = torch.empty_like(q)
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
        dq, dk, dv = (torch.full((B, H, N, D), float("nan"), dtype=torch.float32,
                                 device=q.device) for _ in range(3))
        say(f"forward + backward with 512 global positions, rows {rows_mode}")
        L.lfattn_forward_lse(h, q, k, v, o, lse)
        L.lfattn_backward(h, q, k, v, o, g, lse, dq, dk, dv)
        torch.cuda.synchronize()
    finally:
        L.lfattn_destroy(h)
    want_o = oracle.attention(a.q, a.k, a.v, window, dil, glob)
    err = np.abs(o.float().cpu().numpy().astype(np.float64) - want_o)
    assert err.max() <= 2e-2 and err.mean() <= 2e-3, (err.max(), err.mean())
    want = oracle.attention_grad(a.q, a.k, a.v, do, window=window, dilation=dil, glob=glob)
    for x, w, n in zip((dq, dk, dv), want, ("dq", "dk", "dv")):
        check(x.cpu().numpy().astype(np.float64), w, f"512 globals {n}")


def test_handle_class_forward_lse_and_backward():
    """The LFAttention class runs the same calls as the functions."""
    import torch
    B, H, N, D = 1, 1, 300, 64
    a = W.small_case(B, H, N, D, "bf16", 64, seed=95)
    q, k, v = to_device(a)
    g = q.flip(2).contiguous()
    f32 = dict(dtype=torch.float32, device=q.device)
    outs = []
    with L.LFAttention(B, H, N, D, L.LFATTN_BF16, 64, None, [0, 7]) as att:
        for _ in range(2):
            o, lse = att.forward_lse(q, k, v, torch.empty_like(q), torch.empty((B, H, N), **f32))
            grads = att.backward(q, k, v, o, g, lse,
                                 *(torch.empty((B, H, N, D), **f32) for _ in range(3)))
            outs.append((o, lse, *grads))
    torch.cuda.synchronize()
    for x, y in zip(*outs):
        assert torch.equal(x, y)
    want = oracle.attention_grad(a.q, a.k, a.v, g.float().cpu().numpy(), window=64, glob=[0, 7])
    for x, w, n in zip(outs[0][2:], want, ("dq", "dk", "dv")):
        check(x.cpu().numpy().astype(np.float64), w, f"class {n}")


@pytest.mark.parametrize("form", ["causal_dilated_charlm_n8192", "chunked_gmat_m64_l16384"])
def test_backward_general_forms_full_size(form):
    """The causal band at the dilated character-LM shape and GMAT chunked
    attention ((512 x 32, 64)) at the 16K shape: every head runs and is
    checked element by element."""
    import torch
    if form.startswith("causal"):
        wl = W.BY_NAME["dilated_charlm_n8192"]
    else:
        wl = W.BY_NAME["gmat_memory_m64_l16384"]
    a = W.generate(wl)
    B, H, N, D = wl.B, wl.H, wl.N, wl.D
    rng = np.random.default_rng(wl.seed + 8)
    do = _bf16(rng.standard_normal((B, H, N, D)).astype(np.float32))
    hs = list(range(H))
    if form.startswith("causal"):
        h = L.lfattn_create_causal(B, H, N, D, L.LFATTN_BF16, wl.window, list(a.dilation))
        kw = dict(window=wl.window, dilation=[int(a.dilation[x]) for x in hs], causal=True)
    else:
        h = L.lfattn_create_chunked(B, H, N, D, L.LFATTN_BF16, 512, len(wl.glob))
        kw = dict(chunk=512, n_memory=len(wl.glob))
    try:
        q, k, v = to_device(a)
        g = torch.from_numpy(do).to("cuda:0").to(torch.bfloat16)
        o = torch.empty_like(q)
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
        dq, dk, dv = (torch.full((B, H, N, D), float("nan"), dtype=torch.float32,
                                 device=q.device) for _ in range(3))
        say(f"backward full size, {form}")
        L.lfattn_forward_lse(h, q, k, v, o, lse)
        L.lfattn_backward(h, q, k, v, o, g, lse, dq, dk, dv)
        torch.cuda.synchronize()
    finally:
        L.lfattn_destroy(h)
    want = oracle.attention_grad(a.q[:, hs], a.k[:, hs], a.v[:, hs], do[:, hs], **kw)
    for x, w, n in zip((dq, dk, dv), want, ("dq", "dk", "dv")):
        assert np.all(np.isfinite(x.cpu().numpy())), f"{form} {n}: non-finite"
        say(f"  {n}: {check(x[:, hs].cpu().numpy().astype(np.float64), w, f'{form} {n}')}")


# ---------------------------------------------------------------------------
# Separate projections for the global rows: lfattn_forward_global_proj_lse +
# lfattn_backward_global_proj against the oracle's six gradients.
# ---------------------------------------------------------------------------

PROJ_CASES = [
    ("band", dict(B=1, H=2, N=300, window=64, dil=[1, 2], glob=[0, 150, 299])),
    ("band", dict(B=1, H=1, N=700, window=256, dil=[1], glob=list(range(0, 700, 23)))),
    ("band", dict(B=1, H=2, N=200, window=40, dil=[1, 3], glob=[])),
    ("masked", dict(B=2, H=2, N=400, window=40, dil=[1, 2], sets=[[3, 200, 399], [7]])),
    ("chunked", dict(B=1, H=2, N=20 + 64 * 3 + 7, chunk=64, M=20)),
]


def _proj_handle(kind, p, D):
    B, H, N = p["B"], p["H"], p["N"]
    if kind == "band":
        h = L.lfattn_create(B, H, N, D, L.LFATTN_BF16, p["window"], p["dil"], p["glob"])
        kw = dict(window=p["window"], dilation=p["dil"], glob=p["glob"])
    elif kind == "masked":
        mask = np.zeros((B, N), dtype=np.uint8)
        for b, s in enumerate(p["sets"]):
            mask[b, s] = 1
        h = L.lfattn_create_masked(B, H, N, D, L.LFATTN_BF16, p["window"], p["dil"], mask)
        kw = dict(window=p["window"], dilation=p["dil"], batch_glob=p["sets"])
    else:
        h = L.lfattn_create_chunked(B, H, N, D, L.LFATTN_BF16, p["chunk"], p["M"])
        kw = dict(chunk=p["chunk"], n_memory=p["M"])
    return h, kw


def _run_proj(h, a, g, do, shape):
    import torch
    B, H, N, D = shape
    q, k, v = to_device(a)
    qg, kg, vg = to_device(g)
    dgrad = torch.from_numpy(do).to("cuda:0").to(torch.bfloat16)
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    outs = [torch.full((B, H, N, D), float("nan"), dtype=torch.float32, device=q.device)
            for _ in range(6)]
    L.lfattn_forward_global_proj_lse(h, q, k, v, qg, kg, vg, o, lse)
    L.lfattn_backward_global_proj(h, q, k, v, qg, kg, vg, o, dgrad, lse, *outs)
    torch.cuda.synchronize()
    return [x.cpu().numpy().astype(np.float64) for x in outs]


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("rows_mode", [64, 128])
@pytest.mark.parametrize("case", PROJ_CASES, ids=lambda c: c[0] + "_N%d" % c[1]["N"])
def test_backward_global_proj_every_element(case, rows_mode, D, monkeypatch):
    monkeypatch.setenv("LFATTN_BAND_ROWS", str(rows_mode))
    monkeypatch.setenv("LFATTN_BWD_ROWS", str(rows_mode))
    kind, p = case
    B, H, N = p["B"], p["H"], p["N"]
    a = W.small_case(B, H, N, D, "bf16", p.get("window", 0), dilation=p.get("dil"), seed=188)
    g = W.small_case(B, H, N, D, "bf16", p.get("window", 0), dilation=p.get("dil"), seed=189)
    rng = np.random.default_rng(190)
    do = _bf16(rng.standard_normal((B, H, N, D)).astype(np.float32))
    h, kw = _proj_handle(kind, p, D)
    try:
        say(f"backward with global projections {kind} {p} D {D} rows {rows_mode}")
        got = _run_proj(h, a, g, do, (B, H, N, D))
    finally:
        L.lfattn_destroy(h)
    want = oracle.attention_grad(a.q, a.k, a.v, do, qg=g.q, kg=g.k, vg=g.v, **kw)
    for x, w, n in zip(got, want, ("dq", "dk", "dv", "dqg", "dkg", "dvg")):
        if not np.any(w):  # (no global rows: an all-zero gradient, exactly)
            assert np.array_equal(x, w), f"{kind} {n}: not zero"
        else:
            check(x, w, f"{kind} {n}")


def test_backward_global_proj_shared_adds_up():
    """Qg = Q, Kg = K, Vg = V: the two gradient sets add up to lfattn_backward's."""
    import torch
    B, H, N, D = 1, 2, 600, 64
    a = W.small_case(B, H, N, D, "bf16", 128, dilation=[1, 2], seed=191)
    do = _bf16(np.random.default_rng(192).standard_normal((B, H, N, D)).astype(np.float32))
    glob = [0, 5, 300, 599]
    h = L.lfattn_create(B, H, N, D, L.LFATTN_BF16, 128, [1, 2], glob)
    try:
        say("backward with global projections = the shared ones")
        six = _run_proj(h, a, a, do, (B, H, N, D))
        q, k, v = to_device(a)
        dgrad = torch.from_numpy(do).to("cuda:0").to(torch.bfloat16)
        o = torch.empty_like(q)
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
        three = [torch.empty((B, H, N, D), dtype=torch.float32, device=q.device)
                 for _ in range(3)]
        L.lfattn_forward_lse(h, q, k, v, o, lse)
        L.lfattn_backward(h, q, k, v, o, dgrad, lse, *three)
        torch.cuda.synchronize()
    finally:
        L.lfattn_destroy(h)
    for x, y, w in zip(six[:3], six[3:], three):
        w = w.cpu().numpy().astype(np.float64)
        check(x + y, w, "shared projections")


def test_backward_global_proj_full_size_two_sequences():
    """The Longformer-base shape with two sequences of different global sets
    and their own projections: every head of both sequences is checked
    element by element, all six gradients."""
    import torch
    B, H, N, D, window = 2, 12, 4096, 64, 512
    rng = np.random.default_rng(9)
    sets = [list(range(32)), sorted({0} | set(rng.choice(N, size=10, replace=False).tolist()))]
    a = W.small_case(B, H, N, D, "bf16", window, seed=20261)
    g = W.small_case(B, H, N, D, "bf16", window, seed=21261)
    do = _bf16(rng.standard_normal((B, H, N, D)).astype(np.float32))
    mask = np.zeros((B, N), dtype=np.uint8)
    for b, s in enumerate(sets):
        mask[b, s] = 1
    h = L.lfattn_create_masked(B, H, N, D, L.LFATTN_BF16, window, None, mask)
    try:
        say("backward with global projections, Longformer-base shape, two sequences")
        got = _run_proj(h, a, g, do, (B, H, N, D))
    finally:
        L.lfattn_destroy(h)
    hs = list(range(H))
    want = oracle.attention_grad(a.q[:, hs], a.k[:, hs], a.v[:, hs], do[:, hs],
                                 qg=g.q[:, hs], kg=g.k[:, hs], vg=g.v[:, hs], window=window,
                                 batch_glob=sets)
    for x, w, n in zip(got, want, ("dq", "dk", "dv", "dqg", "dkg", "dvg")):
        assert np.all(np.isfinite(x)), f"{n}: non-finite"
        check(x[:, hs], w, f"two sequences {n}")
