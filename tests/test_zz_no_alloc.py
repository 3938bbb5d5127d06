"""lfattn_forward_noalloc (global-row partials in the library's static device
scratch) against lfattn_forward on the same inputs: two calls in a row, the
second on a smaller problem, each bit-identical to the allocating entry point
and within the bf16 tolerance of the oracle; a handle whose records exceed
the scratch is refused."""

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


def _both(B, H, N, D, window, dil, glob, seed):
    import torch
    inp = W.small_case(B, H, N, D, "bf16", window, dilation=dil, glob=glob, seed=seed)
    q, k, v = to_device(inp)
    o_ref = torch.full_like(q, float("nan"))
    o_na = torch.full_like(q, float("nan"))
    h = L.lfattn_create(B, H, N, D, L.LFATTN_BF16, window, list(inp.dilation), list(inp.glob))
    try:
        L.lfattn_forward(h, q, k, v, o_ref)
        torch.cuda.synchronize()
        L.lfattn_forward_noalloc(h, q, k, v, o_na)
        torch.cuda.synchronize()
    finally:
        L.lfattn_destroy(h)
    return inp, o_ref, o_na


def test_noalloc_matches_forward_two_calls_second_smaller():
    import torch
    cases = [
        # Longformer-base shape: 12 heads x 32 global rows in partial records.
        (1, 12, 4096, 64, 512, None, list(range(32)), 11),
        # A smaller problem after it: fewer, other records in the same array.
        (2, 2, 1000, 128, 256, [1, 2], [0, 7, 999], 12),
    ]
    for B, H, N, D, window, dil, glob, seed in cases:
        say(f"noalloc vs forward: B{B} H{H} N{N} D{D} w{window} globals {len(glob)}")
        inp, o_ref, o_na = _both(B, H, N, D, window, dil, glob, seed)
        assert bool(torch.isfinite(o_na.float()).all())
        assert torch.equal(o_na, o_ref)
        got = o_na.float().cpu().numpy().astype(np.float64)
        want = oracle.attention(inp.q, inp.k, inp.v, window, list(inp.dilation), list(inp.glob))
        compare(got, want, "bf16", "noalloc")


def test_noalloc_without_global_rows():
    import torch
    say("noalloc without global positions")
    _, o_ref, o_na = _both(1, 2, 700, 64, 128, [1, 3], [], 13)
    assert torch.equal(o_na, o_ref)


def test_noalloc_refuses_records_beyond_the_scratch():
    import torch
    # 65536 tokens, 64 global rows per head, 16 heads: about 69 MB of records.
    B, H, N, D = 1, 16, 65536, 128
    glob = list(range(0, N, N // 64))
    h = L.lfattn_create(B, H, N, D, L.LFATTN_BF16, 1024, None, glob)
    try:
        x = torch.zeros(8, dtype=torch.bfloat16, device="cuda:0")  # never read
        say("noalloc refuses a handle beyond its scratch")
        with pytest.raises(L.LfattnError) as e:
            L.lfattn_forward_noalloc(h, x, x, x, x.data_ptr() + 4096)
        assert e.value.status == L.LFATTN_ESCRATCH
    finally:
        L.lfattn_destroy(h)
