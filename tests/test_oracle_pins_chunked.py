"""Pins of the oracle's chunked pattern: GMAT's C x k chunked self-attention
with M memory tokens prefixed ("GMAT: Global Memory Augmentation for
Transformers", sections "Global Memory" and "Chunked self-attention": a token
attends to its own chunk and to the memory; memory tokens attend to all M + L
positions).  CPU only."""

import numpy as np
import pytest
import torch

import oracle
from oracle import brute
from long_context_sparse_band_amd import workloads as W


@pytest.mark.parametrize("n,chunk,M", [(1, 1, 0), (1, 5, 1), (40, 8, 0), (40, 8, 5),
                                       (170, 70, 30), (576, 8, 64), (2112, 512, 64),
                                       (103, 10, 3)])
def test_sets_match_chunked_mask(n, chunk, M):
    mask = brute.chunked_mask(n, chunk, M)
    step = max(1, n // 300)
    for i in range(0, n, step):
        assert oracle.allowed_set_chunked(n, chunk, M, i).tolist() == \
            np.nonzero(mask[i])[0].tolist(), (n, chunk, M, i)
    assert oracle.count_pairs_chunked(1, 1, n, chunk, M) == int(mask.sum())


@pytest.mark.parametrize("C,k,M", [(512, 4, 64), (8, 64, 64), (70, 2, 30), (16, 5, 0)])
def test_chunked_count_closed_form(C, k, M):
    """(C x k, M): M rows of M + Ck keys, Ck rows of C + M keys."""
    n = M + C * k
    assert oracle.count_pairs_chunked(1, 1, n, C, M) == M * n + C * k * (C + M)


def test_chunked_values_match_bruteforce():
    rng = np.random.default_rng(41)
    for t in range(25):
        B, H = int(rng.integers(1, 3)), int(rng.integers(1, 3))
        n, D = int(rng.integers(1, 80)), int(rng.choice([1, 4, 8, 16]))
        chunk = int(rng.integers(1, 40))
        M = int(rng.integers(0, min(n, 8) + 1))
        a = W.small_case(B, H, n, D, "f32", 0, seed=600 + t)
        g = W.small_case(B, H, n, D, "f32", 0, seed=700 + t)
        got = oracle.attention_chunked(a.q, a.k, a.v, chunk, M, qg=g.q, kg=g.k, vg=g.v)
        ref = brute.attention_chunked(a.q, a.k, a.v, chunk, M, g.q, g.k, g.v)
        np.testing.assert_allclose(got, ref, rtol=1e-11, atol=1e-13)


def test_no_memory_is_independent_attention_per_chunk():
    """Library routine: with M = 0 every chunk is plain attention over itself
    (torch's scaled_dot_product_attention, float64, no mask)."""
    C, k, D = 70, 3, 16
    a = W.small_case(1, 2, C * k, D, "f32", 0, seed=42)
    got = oracle.attention_chunked(a.q, a.k, a.v, C, 0)
    for c in range(k):
        sl = slice(c * C, (c + 1) * C)
        ref = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(a.q[:, :, sl]).double(), torch.from_numpy(a.k[:, :, sl]).double(),
            torch.from_numpy(a.v[:, :, sl]).double()).numpy()
        np.testing.assert_allclose(got[:, :, sl], ref, rtol=1e-12, atol=1e-14)


def test_one_chunk_is_full_attention():
    """Library routine: a chunk covering the whole main sequence gives plain
    attention over all positions, memory included."""
    a = W.small_case(1, 2, 150, 16, "f32", 0, seed=43)
    got = oracle.attention_chunked(a.q, a.k, a.v, 1000, 20)
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(a.q).double(), torch.from_numpy(a.k).double(),
        torch.from_numpy(a.v).double()).numpy()
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-14)


def test_chunked_equals_band_form_when_chunk_is_one_token():
    """C = 1: each main token sees itself and the memory, which is the band
    pattern with window 0 and G = {0..M-1} (the band oracle, pinned elsewhere)."""
    a = W.small_case(1, 2, 90, 8, "f32", 0, seed=44)
    got = oracle.attention_chunked(a.q, a.k, a.v, 1, 7)
    ref = oracle.attention(a.q, a.k, a.v, 0, None, list(range(7)))
    np.testing.assert_array_equal(got, ref)


def test_chunks_do_not_see_each_other():
    a = W.small_case(1, 1, 100, 8, "f32", 0, seed=45)
    x = oracle.attention_chunked(a.q, a.k, a.v, 30, 10)
    k2, v2 = a.k.copy(), a.v.copy()
    k2[:, :, 40:70] += 2.0   # the second chunk (positions 40..69)
    v2[:, :, 40:70] -= 1.0
    y = oracle.attention_chunked(a.q, k2, v2, 30, 10)
    same = np.r_[10:40, 70:100]
    assert np.array_equal(x[:, :, same], y[:, :, same])
    assert not np.allclose(x[:, :, 40:70], y[:, :, 40:70])
