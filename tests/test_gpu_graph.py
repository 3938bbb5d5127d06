"""The forward and the backward under HIP graph capture: the library launches
kernels only (no allocation, memset or host sync inside a call), so a
captured call must replay to the same bits as the eager call, every replay,
with the program's own eager work in between."""

import numpy as np
import pytest

from long_context_sparse_band_amd import lfattn as L
from long_context_sparse_band_amd import workloads as W
from gpu_util import say, to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    L.load()


def test_forward_and_backward_replay_bit_exact():
    import torch
    B, H, N, D, window = 1, 2, 700, 64, 128
    dil, glob = [1, 2], [0, 5, 350]
    a = W.small_case(B, H, N, D, "bf16", window, dilation=dil, glob=glob, seed=31)
    q, k, v = to_device(a)
    rng = np.random.default_rng(32)
    g = torch.from_numpy(rng.standard_normal((B, H, N, D)).astype(np.float32)).to(q.device)
    g = g.to(torch.bfloat16)
    h = L.lfattn_create(B, H, N, D, L.LFATTN_BF16, window, dil, glob)
    try:
        s = torch.cuda.Stream()

        def run(o, lse, grads):
            L.lfattn_forward_lse(h, q, k, v, o, lse, s)
            L.lfattn_backward(h, q, k, v, o, g, lse, *grads, s)

        def bufs():
            f32 = dict(dtype=torch.float32, device=q.device)
            return (torch.empty_like(q), torch.empty((B, H, N), **f32),
                    [torch.empty((B, H, N, D), **f32) for _ in range(3)])

        eager, cap = bufs(), bufs()
        say("graph: eager reference")
        with torch.cuda.stream(s):
            run(*eager)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        say("graph: capture")
        with torch.cuda.graph(graph, stream=s):
            run(*cap)
        torch.cuda.synchronize()
        for rep in range(3):
            for t in (cap[0], cap[1], *cap[2]):
                t.fill_(float("nan"))
            say(f"graph: replay {rep}")
            graph.replay()
            torch.cuda.synchronize()
            with torch.cuda.stream(s):
                run(*bufs())  # eager work between replays
            torch.cuda.synchronize()
            assert torch.equal(cap[0], eager[0])
            assert torch.equal(cap[1], eager[1])
            for x, y in zip(cap[2], eager[2]):
                assert torch.equal(x, y)
    finally:
        torch.cuda.synchronize()
        L.lfattn_destroy(h)
