"""Pins of the oracle's gradients (dQ, dK, dV of the attention output for an
upstream gradient dO) under every pattern: torch autograd in float64 through a
dense masked softmax (a library routine and an independent mask
construction), central finite differences, and closed-form sums (the V
gradients of a head add up to the dO rows; the K gradients of a head add up to
zero, softmax being unchanged by a shift of all scores: footnote 3 of section
2.3 of the Unlimiformer page).  CPU only."""

import numpy as np
import pytest
import torch

import oracle
from oracle import brute
from long_context_sparse_band_amd import workloads as W


def _mask(N, H, pattern):
    kind = pattern[0]
    if kind == "band":
        _, window, dil, glob = pattern
        return [brute.band_global_mask(N, window, dil[h], glob) for h in range(H)]
    if kind == "causal":
        _, window, dil = pattern
        return [brute.causal_band_mask(N, window, dil[h]) for h in range(H)]
    _, chunk, M = pattern
    return [brute.chunked_mask(N, chunk, M)] * H


def _torch_grads(q, k, v, do, masks_per_b):
    """Autograd through softmax(scale q k^T + mask) v in float64."""
    qt, kt, vt = (torch.from_numpy(x).double().requires_grad_(True) for x in (q, k, v))
    B, H, N, D = q.shape
    outs = []
    for b in range(B):
        rows = []
        for h in range(H):
            add = torch.from_numpy(np.where(masks_per_b[b][h], 0.0, -np.inf))
            z = (qt[b, h] @ kt[b, h].T) / np.sqrt(D) + add
            rows.append(torch.softmax(z, dim=1) @ vt[b, h])
        outs.append(torch.stack(rows))
    o = torch.stack(outs)
    (o * torch.from_numpy(do).double()).sum().backward()
    return qt.grad.numpy(), kt.grad.numpy(), vt.grad.numpy()


def _case(rng, t):
    B, H = int(rng.integers(1, 3)), int(rng.integers(1, 3))
    N, D = int(rng.integers(1, 40)), int(rng.choice([1, 4, 8]))
    kind = ["band", "causal", "chunked", "batch"][t % 4]
    dil = [int(x) for x in rng.integers(1, 4, size=H)]
    window = int(rng.integers(0, 2 * N + 3))
    if kind == "band":
        n_g = int(rng.integers(0, min(N, 4) + 1))
        glob = sorted(rng.choice(N, size=n_g, replace=False).tolist()) if n_g else []
        masks = [_mask(N, H, ("band", window, dil, glob))] * B
        kw = dict(window=window, dilation=dil, glob=glob)
    elif kind == "causal":
        masks = [_mask(N, H, ("causal", window, dil))] * B
        kw = dict(window=window, dilation=dil, causal=True)
    elif kind == "chunked":
        chunk, M = int(rng.integers(1, 12)), int(rng.integers(0, min(N, 4) + 1))
        masks = [_mask(N, H, ("chunked", chunk, M))] * B
        kw = dict(chunk=chunk, n_memory=M)
    else:
        sets = []
        for _ in range(B):
            n_g = int(rng.integers(0, min(N, 4) + 1))
            sets.append(sorted(rng.choice(N, size=n_g, replace=False).tolist()) if n_g else [])
        masks = [_mask(N, H, ("band", window, dil, sets[b])) for b in range(B)]
        kw = dict(window=window, dilation=dil, batch_glob=sets)
    return B, H, N, D, masks, kw


def test_gradients_match_torch_autograd():
    rng = np.random.default_rng(51)
    for t in range(32):
        B, H, N, D, masks, kw = _case(rng, t)
        a = W.small_case(B, H, N, D, "f32", 0, seed=800 + t)
        do = rng.standard_normal((B, H, N, D)).astype(np.float32)
        got = oracle.attention_grad(a.q, a.k, a.v, do, **kw)
        ref = _torch_grads(a.q, a.k, a.v, do, masks)
        for g, r, name in zip(got, ref, ("dq", "dk", "dv")):
            np.testing.assert_allclose(g, r, rtol=1e-10, atol=1e-12, err_msg=f"{t} {name} {kw}")


def test_gradients_match_finite_differences():
    rng = np.random.default_rng(52)
    B, H, N, D = 1, 2, 23, 4
    a = W.small_case(B, H, N, D, "f32", 0, seed=901)
    q, k, v = (x.astype(np.float64) for x in (a.q, a.k, a.v))
    do = rng.standard_normal((B, H, N, D))
    kw = dict(window=6, dilation=[1, 2], glob=[0, 11])

    def loss(qq, kk, vv):
        o = oracle.attention(qq.astype(np.float32), kk.astype(np.float32), vv.astype(np.float32),
                             6, [1, 2], [0, 11])
        return float((o * do).sum())

    # The oracle reads float32 inputs: a step of 1e-2 keeps their rounding small.
    got = oracle.attention_grad(q.astype(np.float32), k.astype(np.float32), v.astype(np.float32),
                                do.astype(np.float32), **kw)
    eps = 1e-2
    for which, arr in enumerate((q, k, v)):
        for _ in range(6):
            idx = tuple(int(rng.integers(0, s)) for s in arr.shape)
            # (divided by the step the float32 inputs actually take)
            up, dn = arr.copy(), arr.copy()
            up[idx] += eps
            dn[idx] -= eps
            args_up = [q, k, v]
            args_dn = [q, k, v]
            args_up[which], args_dn[which] = up, dn
            fd = (loss(*args_up) - loss(*args_dn)) / (float(np.float32(arr[idx] + eps)) -
                                                      float(np.float32(arr[idx] - eps)))
            assert abs(fd - got[which][idx]) <= 2e-3 * max(1.0, abs(fd)), (which, idx, fd,
                                                                          got[which][idx])


@pytest.mark.parametrize("kw", [dict(window=10, dilation=[1, 3], glob=[2]),
                                dict(window=10, dilation=[2, 1], causal=True),
                                dict(chunk=7, n_memory=3)])
def test_gradient_sums(kw):
    """Per head: sum_j dV_j = sum_i dO_i, sum_j dK_j = 0."""
    rng = np.random.default_rng(53)
    a = W.small_case(2, 2, 60, 8, "f32", 0, seed=902)
    do = rng.standard_normal((2, 2, 60, 8)).astype(np.float32)
    dq, dk, dv = oracle.attention_grad(a.q, a.k, a.v, do, **kw)
    np.testing.assert_allclose(dv.sum(axis=2), do.astype(np.float64).sum(axis=2), rtol=1e-10,
                               atol=1e-10)
    np.testing.assert_allclose(dk.sum(axis=2), 0.0, atol=1e-10)


def test_row_lse_matches_torch_logsumexp():
    """Library routine: torch.logsumexp (float64) of the masked scores."""
    rng = np.random.default_rng(54)
    for t in range(16):
        B, H, N, D, masks, kw = _case(rng, t)
        a = W.small_case(B, H, N, D, "f32", 0, seed=950 + t)
        got = oracle.row_lse(a.q, a.k, **kw)
        for b in range(B):
            for h in range(H):
                z = torch.from_numpy(a.q[b, h]).double() @ torch.from_numpy(a.k[b, h]).double().T
                z = z / np.sqrt(D) + torch.from_numpy(np.where(masks[b][h], 0.0, -np.inf))
                np.testing.assert_allclose(got[b, h], torch.logsumexp(z, dim=1).numpy(),
                                           rtol=1e-12, atol=1e-12)


# ---------------------------------------------------------------------------
# Separate projections for the global rows (the memory rows of chunked
# attention): a global row i attends all keys with Qg_i, Kg, Vg; every other
# row keeps Q, K, V over its set.
# ---------------------------------------------------------------------------

def _torch_grads_proj(q, k, v, qg, kg, vg, do, masks_per_b, gsets_per_b):
    """Autograd through the dense two-projection form in float64: a global
    row's output is softmax(scale Qg_i Kg^T) Vg over every key, any other
    row's the masked softmax with Q, K, V."""
    ts = [torch.from_numpy(x).double().requires_grad_(True) for x in (q, k, v, qg, kg, vg)]
    qt, kt, vt, qgt, kgt, vgt = ts
    B, H, N, D = q.shape
    outs = []
    for b in range(B):
        rows = []
        isg = torch.zeros(N, dtype=torch.bool)
        isg[list(gsets_per_b[b])] = True
        for h in range(H):
            add = torch.from_numpy(np.where(masks_per_b[b][h], 0.0, -np.inf))
            ob = torch.softmax((qt[b, h] @ kt[b, h].T) / np.sqrt(D) + add, dim=1) @ vt[b, h]
            og = torch.softmax((qgt[b, h] @ kgt[b, h].T) / np.sqrt(D), dim=1) @ vgt[b, h]
            rows.append(torch.where(isg[:, None], og, ob))
        outs.append(torch.stack(rows))
    o = torch.stack(outs)
    (o * torch.from_numpy(do).double()).sum().backward()
    return tuple(t.grad.numpy() for t in ts)


def _proj_case(rng, t):
    B, H = int(rng.integers(1, 3)), int(rng.integers(1, 3))
    N, D = int(rng.integers(2, 40)), int(rng.choice([1, 4, 8]))
    kind = ["band", "batch", "chunked"][t % 3]
    dil = [int(x) for x in rng.integers(1, 4, size=H)]
    window = int(rng.integers(0, 2 * N + 3))
    if kind == "chunked":
        chunk, M = int(rng.integers(1, 12)), int(rng.integers(1, min(N, 4) + 1))
        masks = [_mask(N, H, ("chunked", chunk, M))] * B
        return B, H, N, D, masks, [list(range(M))] * B, dict(chunk=chunk, n_memory=M)
    sets = []
    for _ in range(B if kind == "batch" else 1):
        n_g = int(rng.integers(1, min(N, 4) + 1))
        sets.append(sorted(rng.choice(N, size=n_g, replace=False).tolist()))
    if kind == "band":
        sets = sets * B
        kw = dict(window=window, dilation=dil, glob=sets[0])
    else:
        kw = dict(window=window, dilation=dil, batch_glob=sets)
    masks = [_mask(N, H, ("band", window, dil, sets[b])) for b in range(B)]
    return B, H, N, D, masks, sets, kw


def test_gradients_with_global_projections_match_torch_autograd():
    rng = np.random.default_rng(61)
    for t in range(24):
        B, H, N, D, masks, gsets, kw = _proj_case(rng, t)
        a = W.small_case(B, H, N, D, "f32", 0, seed=900 + t)
        g = W.small_case(B, H, N, D, "f32", 0, seed=1900 + t)
        do = rng.standard_normal((B, H, N, D)).astype(np.float32)
        got = oracle.attention_grad(a.q, a.k, a.v, do, qg=g.q, kg=g.k, vg=g.v, **kw)
        want = _torch_grads_proj(a.q, a.k, a.v, g.q, g.k, g.v, do, masks, gsets)
        for x, w, n in zip(got, want, ("dq", "dk", "dv", "dqg", "dkg", "dvg")):
            np.testing.assert_allclose(x, w, rtol=1e-9, atol=1e-10, err_msg=f"case {t} {n}")


def test_gradients_with_global_projections_closed_forms():
    """Each head: the V gradients of the global rows' attention add up to their
    dO rows and the others' to the rest; both K gradient sums vanish; rows
    outside G have no Qg gradient and rows in G no Q gradient."""
    rng = np.random.default_rng(62)
    for t in range(12):
        B, H, N, D, masks, gsets, kw = _proj_case(rng, t)
        a = W.small_case(B, H, N, D, "f32", 0, seed=950 + t)
        g = W.small_case(B, H, N, D, "f32", 0, seed=1950 + t)
        do = rng.standard_normal((B, H, N, D)).astype(np.float64)
        dq, dk, dv, dqg, dkg, dvg = oracle.attention_grad(a.q, a.k, a.v, do.astype(np.float32),
                                                          qg=g.q, kg=g.k, vg=g.v, **kw)
        do32 = do.astype(np.float32).astype(np.float64)
        for b in range(B):
            isg = np.zeros(N, dtype=bool)
            isg[gsets[b]] = True
            for h in range(H):
                np.testing.assert_allclose(dvg[b, h].sum(0), do32[b, h][isg].sum(0), atol=1e-9)
                np.testing.assert_allclose(dv[b, h].sum(0), do32[b, h][~isg].sum(0), atol=1e-9)
                np.testing.assert_allclose(dkg[b, h].sum(0), 0.0, atol=1e-9)
                np.testing.assert_allclose(dk[b, h].sum(0), 0.0, atol=1e-9)
                assert np.all(dq[b, h][isg] == 0.0) and np.all(dqg[b, h][~isg] == 0.0)


def test_gradients_with_shared_global_projections_add_up():
    """Qg = Q, Kg = K, Vg = V: the two gradient sets add up to the shared-
    projection gradients."""
    rng = np.random.default_rng(63)
    for t in range(9):
        B, H, N, D, masks, gsets, kw = _proj_case(rng, t)
        a = W.small_case(B, H, N, D, "f32", 0, seed=990 + t)
        do = rng.standard_normal((B, H, N, D)).astype(np.float32)
        six = oracle.attention_grad(a.q, a.k, a.v, do, qg=a.q, kg=a.k, vg=a.v, **kw)
        three = oracle.attention_grad(a.q, a.k, a.v, do, **kw)
        for x, y, w in zip(six[:3], six[3:], three):
            np.testing.assert_allclose(x + y, w, rtol=1e-12, atol=1e-12)
