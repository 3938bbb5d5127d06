"""Pins of the oracle's general form: one global set per batch element and
separate projections (Qg, Kg, Vg) for the global rows.

Sources: the Ultralytics glossary page "Longformer", section on how the
attention works, global-attention bullet (global attention uses its own query,
key and value projections), and the page's closing paragraph (the Hugging Face
implementation takes the global tokens as a per-sequence global_attention_mask).
Reading: the separate projections are the global rows' own attention (a global
query scores every key with Kg and weights Vg); the other rows score the global
keys with Q, K, V.  CPU only.
"""

import numpy as np
import pytest
import torch

import oracle
from oracle import brute


def _draw(rng, B, H, N, D):
    return [rng.standard_normal((B, H, N, D)).astype(np.float32) for _ in range(6)]


def _random_sets(rng, B, N):
    out = []
    for _ in range(B):
        n_g = int(rng.integers(0, min(N, 6) + 1))
        out.append(rng.choice(N, size=n_g, replace=False).tolist() if n_g else [])
    return out


def test_general_form_matches_bruteforce():
    rng = np.random.default_rng(11)
    for t in range(40):
        B, H = int(rng.integers(1, 4)), int(rng.integers(1, 3))
        N, D = int(rng.integers(1, 48)), int(rng.choice([1, 3, 8, 16]))
        window = int(rng.integers(0, 2 * N + 3))
        dil = [int(x) for x in rng.integers(1, 5, size=H)]
        q, k, v, qg, kg, vg = _draw(rng, B, H, N, D)
        sets = _random_sets(rng, B, N)
        got = oracle.attention(q, k, v, window, dil, qg=qg, kg=kg, vg=vg, batch_glob=sets)
        ref = brute.attention_ex(q, k, v, window, dil, sets, qg, kg, vg)
        np.testing.assert_allclose(got, ref, rtol=1e-11, atol=1e-13, err_msg=str(t))
        want_pairs = sum(int(brute.band_global_mask(N, window, dil[h], sets[b]).sum())
                         for b in range(B) for h in range(H))
        assert oracle.count_pairs(B, H, N, window, dil, batch_glob=sets) == want_pairs


def test_global_rows_are_full_attention_with_own_projections():
    """Library routine: a global row is torch's scaled_dot_product_attention
    (float64, no mask) of its Qg row over Kg, Vg."""
    rng = np.random.default_rng(12)
    B, H, N, D = 2, 2, 300, 16
    q, k, v, qg, kg, vg = _draw(rng, B, H, N, D)
    sets = [[0, 7, 299], [150]]
    got = oracle.attention(q, k, v, 40, None, qg=qg, kg=kg, vg=vg, batch_glob=sets)
    for b in range(B):
        for h in range(H):
            rows = sets[b]
            ref = torch.nn.functional.scaled_dot_product_attention(
                torch.from_numpy(qg[b, h][rows]).double()[None],
                torch.from_numpy(kg[b, h]).double()[None],
                torch.from_numpy(vg[b, h]).double()[None])[0].numpy()
            np.testing.assert_allclose(got[b, h][rows], ref, rtol=1e-12, atol=1e-14)


def test_band_rows_ignore_global_projections():
    rng = np.random.default_rng(13)
    B, H, N, D = 2, 2, 120, 8
    q, k, v, qg, kg, vg = _draw(rng, B, H, N, D)
    sets = [[3, 60], [0]]
    a = oracle.attention(q, k, v, 30, [1, 2], qg=qg, kg=kg, vg=vg, batch_glob=sets)
    b_ = oracle.attention(q, k, v, 30, [1, 2], qg=qg + 1.5, kg=kg * 2.0, vg=vg - 3.0,
                          batch_glob=sets)
    for b in range(B):
        band = np.setdiff1d(np.arange(N), sets[b])
        assert np.array_equal(a[b][:, band], b_[b][:, band])
        assert not np.allclose(a[b][:, sets[b]], b_[b][:, sets[b]])


def test_global_rows_ignore_ordinary_projections():
    rng = np.random.default_rng(14)
    B, H, N, D = 2, 1, 90, 8
    q, k, v, qg, kg, vg = _draw(rng, B, H, N, D)
    sets = [[10, 11], [89]]
    a = oracle.attention(q, k, v, 20, None, qg=qg, kg=kg, vg=vg, batch_glob=sets)
    b_ = oracle.attention(q * 3.0, k + 1.0, v - 2.0, 20, None, qg=qg, kg=kg, vg=vg,
                          batch_glob=sets)
    for b in range(B):
        assert np.array_equal(a[b][:, sets[b]], b_[b][:, sets[b]])


def test_per_batch_sets_equal_separate_runs():
    rng = np.random.default_rng(15)
    B, H, N, D = 3, 2, 70, 8
    q, k, v, qg, kg, vg = _draw(rng, B, H, N, D)
    sets = [[0, 1, 2], [], [69, 30]]
    got = oracle.attention(q, k, v, 16, [1, 3], qg=qg, kg=kg, vg=vg, batch_glob=sets)
    for b in range(B):
        one = oracle.attention(q[b:b + 1], k[b:b + 1], v[b:b + 1], 16, [1, 3], glob=sets[b],
                               qg=qg[b:b + 1], kg=kg[b:b + 1], vg=vg[b:b + 1])
        assert np.array_equal(got[b:b + 1], one)


def test_shared_sets_and_ordinary_projections_reduce_to_the_default():
    rng = np.random.default_rng(16)
    B, H, N, D = 2, 2, 80, 8
    q, k, v, _, _, _ = _draw(rng, B, H, N, D)
    glob = [5, 40]
    base = oracle.attention(q, k, v, 24, [1, 2], glob=glob)
    same = oracle.attention(q, k, v, 24, [1, 2], qg=q, kg=k, vg=v, batch_glob=[glob, glob])
    assert np.array_equal(base, same)


def test_other_reading_is_distinguishable():
    """Were the band rows to score the global keys with Kg and Vg instead (the
    other reading of the bullet), the results would differ: a path taking it
    fails parity against this oracle."""
    rng = np.random.default_rng(17)
    B, H, N, D = 1, 1, 60, 8
    q, k, v, qg, kg, vg = _draw(rng, B, H, N, D)
    sets = [[0, 30]]
    ours = oracle.attention(q, k, v, 10, None, qg=qg, kg=kg, vg=vg, batch_glob=sets)
    # Other reading: band rows' global columns from kg/vg.
    alt = np.empty_like(ours)
    scale = 1.0 / np.sqrt(D)
    mask = brute.band_global_mask(N, 10, 1, sets[0])
    for i in range(N):
        if i in sets[0]:
            alt[0, 0, i] = ours[0, 0, i]
            continue
        keys = np.nonzero(mask[i])[0]
        kk = np.where(np.isin(keys, sets[0])[:, None], kg[0, 0][keys], k[0, 0][keys])
        vv = np.where(np.isin(keys, sets[0])[:, None], vg[0, 0][keys], v[0, 0][keys])
        z = scale * (kk.astype(np.float64) @ q[0, 0, i].astype(np.float64))
        w = np.exp(z - z.max())
        alt[0, 0, i] = (w @ vv) / w.sum()
    assert np.abs(alt - ours).max() > 1e-3


def test_general_form_rejects_bad_offsets():
    q = np.zeros((2, 1, 8, 4), dtype=np.float32)
    with pytest.raises((ValueError, AssertionError)):
        oracle.attention(q, q, q, 2, batch_glob=[[0]])  # one list for two batch elements
    with pytest.raises(ValueError):
        oracle.attention(q, q, q, 2, batch_glob=[[0], [8]])  # position out of range
