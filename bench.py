"""Benchmark: scored pairs per second of the band + global attention forward.

One step is one lfattn_forward (global-row kernel + band kernel) over the
Longformer-base workload (B 1, H 12, N 4096, D 64, bf16, window 512, global
tokens 0..31) with inputs already resident in device memory.  Prints one JSON
line.  Options: --gpus (only 1 is supported: the path runs on one GPU),
--steps, --warmup, --workload (another of the named workloads), --no-cpu.
The default warm-up (2000 forwards) runs long enough for the GPU's clock to
settle under the load (a short warm-up times part of the steps at a lower
clock).  Besides the timed steps (warm: inputs resident in the caches as well), the
line carries 20-trial medians and interquartile ranges of the warm time and
of cold-cache forwards (caches flushed by a 512 MB write before each).
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "attention scored-pairs/sec and % of bf16 MFMA peak, N=4096 Longformer-base shape"
# MI355X published dense peaks: bf16 MFMA 2.5 PFLOP/s, fp32 MFMA 157.3 TFLOP/s;
# HBM3E 8 TB/s.
PEAK_TFLOPS = {"bf16": 2500.0, "f32": 157.3}
PEAK_HBM_GBS = 8000.0


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=2000)
    p.add_argument("--workload", default="longformer_base_n4096")
    p.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    p.add_argument("--variant", default="plain",
                   choices=["plain", "global_proj", "two_sequences", "causal", "chunked",
                            "backward", "backward_causal", "backward_chunked"],
                   help="global_proj: the global rows take their own projections (a second "
                        "seeded Q, K, V); two_sequences: B = 2 with a different global set per "
                        "sequence ([CLS] + 10 seeded positions for the second), and own "
                        "projections; causal: the causal band (workloads without global "
                        "tokens, e.g. dilated_charlm_n8192); chunked: GMAT chunked attention, "
                        "chunks of --chunk keys after the workload's memory tokens "
                        "(gmat_memory_m64_l16384: (512 x 32, 64)); backward: one step is "
                        "lfattn_backward (dQ, dK, dV from a seeded upstream gradient, bf16 "
                        "workloads) after one untimed lfattn_forward_lse; backward_causal, "
                        "backward_chunked: the same for the causal band and chunked attention "
                        "(same workload conditions as causal and chunked)")
    p.add_argument("--chunk", type=int, default=512, help="chunk length of --variant chunked")
    p.add_argument("--copy-calibration", action="store_true",
                   help="only run a plain 1 GiB device copy (counter calibration)")
    return p.parse_args()


BAND_SOURCE = os.path.join(ROOT, "long_context_sparse_band_amd", "csrc", "band_bf16.hip")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")


def band_source_hash():
    import hashlib
    with open(BAND_SOURCE, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


BWD_SOURCE = os.path.join(ROOT, "long_context_sparse_band_amd", "csrc", "backward_bf16.hip")
BWD_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_backward.json")


def recorded_backward_traffic(workload):
    """HBM bytes per key-side backward launch from the recorded counter runs,
    or None when they were taken on a different kernel source."""
    import hashlib
    try:
        with open(BWD_TRAFFIC_FILE) as f:
            rec = json.load(f)
        with open(BWD_SOURCE, "rb") as f:
            sha = hashlib.sha256(f.read()).hexdigest()
    except (OSError, ValueError):
        return None
    entry = rec.get("workloads", {}).get(workload)
    if not entry or rec.get("source_sha256") != sha:
        return None
    return entry.get("traffic_bytes_per_launch")


def recorded_traffic(workload):
    """HBM bytes per band-kernel launch from the recorded FETCH_SIZE/WRITE_SIZE
    counter runs, or None when they were taken on a different kernel source."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    entry = rec.get("workloads", {}).get(workload)
    if not entry or rec.get("band_source_sha256") != band_source_hash():
        return None
    return entry.get("traffic_bytes_per_launch")


def copy_calibration():
    """A plain device-to-device copy of 1 GiB, several times: the known-size
    reference that FETCH_SIZE and WRITE_SIZE are scaled by."""
    import torch
    n = 1 << 30
    x = torch.empty(n, dtype=torch.uint8, device="cuda:0")
    x.fill_(1)
    y = torch.empty_like(x)
    for _ in range(5):
        y.copy_(x)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": n, "copies": 5}), flush=True)


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def input_record(inp):
    """Library versions and a SHA-256 of each generated input array (float32
    values as generated, before any device copy)."""
    import hashlib
    import numpy as np
    import torch
    return {"numpy": np.__version__, "torch": torch.__version__,
            "sha256": {n: hashlib.sha256(np.ascontiguousarray(a).tobytes()).hexdigest()
                       for n, a in (("q", inp.q), ("k", inp.k), ("v", inp.v))}}


def quantiles(xs):
    """(25th percentile, median, 75th percentile) of a list."""
    import numpy as np
    q = np.percentile(np.asarray(xs, dtype=np.float64), [25, 50, 75])
    return float(q[0]), float(q[1]), float(q[2])


def cpu_baseline(inp, wl, pairs_per_head_total):
    """The oracle as it stands, on this host's cores, over the whole workload
    (repeated until at least 10 s have passed; one pass is about 0.1 s at the
    Longformer-base shape)."""
    import oracle
    threads = os.cpu_count() or 1
    args = (inp.q, inp.k, inp.v, wl.window, list(inp.dilation), list(inp.glob))
    passes, t0 = 0, time.perf_counter()
    while True:
        oracle.attention(*args, nthreads=threads)
        passes += 1
        el = time.perf_counter() - t0
        if el >= 10.0:
            break
    # One thread, on the first (at most 4096) rows of the first (batch, head),
    # for at least 2 s.
    rows = list(range(min(wl.N, 4096)))
    d0 = int(inp.dilation[0])
    head_pairs = sum(len(oracle.allowed_set(wl.N, wl.window, d0, list(inp.glob), i))
                     for i in rows)
    passes1, t1 = 0, time.perf_counter()
    while True:
        oracle.attention(*args, rows=rows, nthreads=1)
        passes1 += 1
        el1 = time.perf_counter() - t1
        if el1 >= 2.0:
            break
    return {"value": pairs_per_head_total * passes / el, "unit": "pairs/s", "cores": threads,
            "kind": "oracle",
            "sample": f"the whole {wl.name} workload (all {wl.B * wl.H * wl.N} rows), "
                      f"{passes} pass(es) in {el:.2f} s, double precision, {threads} threads",
            "single_thread": {"value": head_pairs * passes1 / el1, "unit": "pairs/s",
                              "sample": f"the first {len(rows)} rows of the first (batch, head), "
                                        f"{passes1} pass(es) in {el1:.2f} s"},
            "cpu_model": cpu_model()}


def bench_backward(args, wl, inp, L, torch):
    """One step: lfattn_backward over the workload.  Algorithmic work: five
    products of 2D flops per scored pair (scores, dP = dO V^T, dV, dQ, dK);
    the key-side kernel itself does four (scores, dP, dK, dV) and the
    query-side kernel three (scores, dP, dQ)."""
    import numpy as np
    dev = torch.device("cuda:0")

    def upload(x):
        return torch.from_numpy(x).to(dev).to(torch.bfloat16).contiguous()

    q, k, v = (upload(a) for a in (inp.q, inp.k, inp.v))
    rng = np.random.default_rng(wl.seed + 7)
    g = upload(rng.standard_normal(inp.q.shape).astype(np.float32))
    o = torch.empty_like(q)
    lse = torch.empty((wl.B, wl.H, wl.N), dtype=torch.float32, device=dev)
    dq, dk, dv = (torch.empty((wl.B, wl.H, wl.N, wl.D), dtype=torch.float32, device=dev)
                  for _ in range(3))
    form = args.variant[len("backward_"):] if args.variant != "backward" else "plain"
    if form == "causal":
        h = L.lfattn_create_causal(wl.B, wl.H, wl.N, wl.D, L.LFATTN_BF16, wl.window,
                                   list(inp.dilation))
    elif form == "chunked":
        h = L.lfattn_create_chunked(wl.B, wl.H, wl.N, wl.D, L.LFATTN_BF16, args.chunk,
                                    len(wl.glob))
    else:
        h = L.lfattn_create(wl.B, wl.H, wl.N, wl.D, L.LFATTN_BF16, wl.window,
                            list(inp.dilation), list(inp.glob))
    stream = torch.cuda.current_stream()
    L.lfattn_forward_lse(h, q, k, v, o, lse, stream)

    def step():
        L.lfattn_backward(h, q, k, v, o, g, lse, dq, dk, dv, stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(args.steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    L.lfattn_set_timing(h, True)
    for _ in range(args.steps):
        step()
    rows, keys, merge, n = L.lfattn_read_backward_timing(h)
    L.lfattn_set_timing(h, False)
    rows, keys, merge = (x / max(n, 1) for x in (rows, keys, merge))
    pairs = L.lfattn_scored_pairs(h)
    L.lfattn_destroy(h)
    peak = PEAK_TFLOPS["bf16"]
    D = wl.D
    keys_tf = pairs * 8 * D / (keys * 1e-3) / 1e12
    rows_tf = pairs * 6 * D / (rows * 1e-3) / 1e12
    line = {
        "metric": "backward scored-pairs/sec (dQ, dK, dV)",
        "value": pairs / (ms * 1e-3),
        "unit": "scored pairs/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded i.i.d. Gaussian Q, K, V and upstream gradient)",
        "inputs": input_record(inp),
        "config": {"workload": wl.name, "variant": args.variant, "B": wl.B, "H": wl.H,
                   "N": wl.N, "D": D, "window": None if form == "chunked" else wl.window,
                   **({"chunk": args.chunk, "n_memory": len(wl.glob)} if form == "chunked" else {}),
                   "dilation": [int(x) for x in inp.dilation], "n_global": len(inp.glob),
                   "scored_pairs": pairs, "parallelism": "single GPU"},
        "whole_backward_tflops": pairs * 10 * D / (ms * 1e-3) / 1e12,
        "whole_backward_mfma_frac": pairs * 10 * D / (ms * 1e-3) / 1e12 / peak,
        "kernels_ms": {"rows_dq": rows, "keys_dkdv": keys, "merge": merge},
        "rows_kernel": {"achieved": rows_tf, "frac": rows_tf / peak,
                        "flops_per_launch": pairs * 6 * D},
        "roofline": {"kernel": "bwd_keys_kernel", "bound": "mfma", "achieved": keys_tf,
                     "peak": peak, "unit": "TFLOP/s", "frac": keys_tf / peak,
                     "traffic": recorded_backward_traffic(wl.name) if form == "plain" else None,
                     "algorithmic_flops_per_launch": pairs * 8 * D,
                     "ideal_bytes_per_launch": wl.B * wl.H * wl.N * 16 * D},
    }
    if not args.no_cpu and form == "plain":
        line["cpu_baseline"] = cpu_baseline_backward(inp, wl, g.float().cpu().numpy(), pairs)
    print(json.dumps(line), flush=True)


def cpu_baseline_backward(inp, wl, do, pairs):
    """The gradient oracle as it stands, on this host's cores, over the whole
    workload (repeated until at least 5 s have passed), or over its first head
    when the workload scores more than 2e8 pairs (the pairs/s rate scales by
    the head's share of the pairs)."""
    import oracle
    threads = os.cpu_count() or 1
    whole = pairs <= 2e8
    if whole:
        q, k, v, g, dil, share, what = inp.q, inp.k, inp.v, do, list(inp.dilation), pairs, \
            f"the gradients of the whole {wl.name} workload"
    else:
        q, k, v, g = (x[:1, :1] for x in (inp.q, inp.k, inp.v, do))
        dil = [int(inp.dilation[0])]
        share = oracle.count_pairs(1, 1, wl.N, wl.window, dil, list(inp.glob))
        what = f"the gradients of the first head of {wl.name} ({share} pairs)"
    passes, t0 = 0, time.perf_counter()
    while True:
        oracle.attention_grad(q, k, v, g, window=wl.window, dilation=dil, glob=list(inp.glob),
                              nthreads=threads)
        passes += 1
        el = time.perf_counter() - t0
        if el >= 5.0:
            break
    return {"value": share * passes / el, "unit": "pairs/s", "cores": threads, "kind": "oracle",
            "sample": f"{what}, {passes} pass(es) in {el:.2f} s, double precision, "
                      f"{threads} threads",
            "cpu_model": cpu_model()}


def main():
    args = parse()
    if args.copy_calibration:
        copy_calibration()
        return
    if args.gpus != 1:
        print(f"bench.py: this path runs on one GPU; --gpus {args.gpus} is not supported.",
              file=sys.stderr)
        sys.exit(2)

    import torch

    from long_context_sparse_band_amd import lfattn as L
    from long_context_sparse_band_amd import workloads as W

    import dataclasses

    import numpy as np

    wl = W.BY_NAME[args.workload]
    if args.variant in ("causal", "backward_causal") and (wl.glob or wl.n_random_glob):
        print(f"bench.py: --variant causal needs a workload without global tokens; "
              f"{wl.name} has some.", file=sys.stderr)
        sys.exit(2)
    if (args.variant in ("chunked", "backward_chunked")
            and tuple(wl.glob) != tuple(range(len(wl.glob)))):
        print(f"bench.py: --variant chunked needs memory tokens at 0..M-1; {wl.name} has "
              f"other global positions.", file=sys.stderr)
        sys.exit(2)
    if args.variant.startswith("backward") and wl.dtype != "bf16":
        print(f"bench.py: --variant backward runs on bf16 workloads; {wl.name} "
              f"is {wl.dtype}.", file=sys.stderr)
        sys.exit(2)
    if args.variant == "two_sequences":
        wl = dataclasses.replace(wl, B=2)
    inp = W.generate(wl)
    if args.variant.startswith("backward"):
        bench_backward(args, wl, inp, L, torch)
        return
    dev = torch.device("cuda:0")
    tdt = torch.bfloat16 if wl.dtype == "bf16" else torch.float32

    def upload(x):
        return torch.from_numpy(x).to(dev).to(tdt).contiguous()

    q, k, v = (upload(a) for a in (inp.q, inp.k, inp.v))
    o = torch.empty_like(q)
    dtype = L.LFATTN_BF16 if wl.dtype == "bf16" else L.LFATTN_F32
    sets = [list(inp.glob)] * wl.B
    if args.variant == "two_sequences":
        rng = np.random.default_rng(wl.seed + 2000)
        sets = [list(inp.glob),
                sorted({0} | set(rng.choice(wl.N, size=10, replace=False).tolist()))]
        mask = np.zeros((wl.B, wl.N), dtype=np.uint8)
        for b, st in enumerate(sets):
            mask[b, st] = 1
        h = L.lfattn_create_masked(wl.B, wl.H, wl.N, wl.D, dtype, wl.window,
                                   list(inp.dilation), mask)
    elif args.variant == "chunked":
        h = L.lfattn_create_chunked(wl.B, wl.H, wl.N, wl.D, dtype, args.chunk, len(wl.glob))
    elif args.variant == "causal":
        h = L.lfattn_create_causal(wl.B, wl.H, wl.N, wl.D, dtype, wl.window,
                                   list(inp.dilation))
    else:
        h = L.lfattn_create(wl.B, wl.H, wl.N, wl.D, dtype, wl.window, list(inp.dilation),
                            list(inp.glob))
    if args.variant in ("plain", "causal", "chunked"):
        def forward():
            L.lfattn_forward(h, q, k, v, o, stream)
    else:
        ginp = W.generate(dataclasses.replace(wl, seed=wl.seed + 1000))
        qg, kg, vg = (upload(a) for a in (ginp.q, ginp.k, ginp.v))

        def forward():
            L.lfattn_forward_global_proj(h, q, k, v, qg, kg, vg, o, stream)
    pairs = L.lfattn_scored_pairs(h)
    n_g = [len(st) for st in sets] if args.variant == "two_sequences" else len(inp.glob)
    # Pairs the band kernel launch scores (the band rows, and the global rows
    # where the same launch computes their partials).
    band_pairs = L.lfattn_band_launch_pairs(h)
    stream = torch.cuda.current_stream()

    for _ in range(args.warmup):
        forward()
    torch.cuda.synchronize()

    # Timed region: exactly `steps` forwards between two events on the stream.
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(args.steps):
        forward()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps

    # Per-kernel durations: the same forwards with the library's events around
    # each kernel (a second pass, so the first timing is undisturbed).
    L.lfattn_set_timing(h, True)
    for _ in range(args.steps):
        forward()
    band_ms, glob_ms, n = L.lfattn_read_timing(h)
    L.lfattn_set_timing(h, False)
    band_ms /= max(n, 1)
    glob_ms /= max(n, 1)

    # Spread of the warm time: 20 trials of R back-to-back forwards.  Cold
    # cache: before each of 20 single forwards, a 512 MB device write (more
    # than the 256 MB Infinity Cache and the L2s hold) evicts Q, K and V; the
    # events bracket the forward only.
    rep = max(1, min(args.steps, 200))
    warm = []
    for _ in range(20):
        e0.record(stream)
        for _ in range(rep):
            forward()
        e1.record(stream)
        torch.cuda.synchronize()
        warm.append(e0.elapsed_time(e1) / rep)
    scratch = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    cold = []
    for t in range(20):
        scratch.fill_(t + 1)
        e0.record(stream)
        forward()
        e1.record(stream)
        torch.cuda.synchronize()
        cold.append(e0.elapsed_time(e1))
    L.lfattn_set_timing(h, True)
    cold_band = []
    for t in range(20):
        scratch.fill_(t + 101)
        forward()
        torch.cuda.synchronize()
        b_ms, _, _ = L.lfattn_read_timing(h)
        cold_band.append(b_ms)
    L.lfattn_set_timing(h, False)
    del scratch
    L.lfattn_destroy(h)

    flops_per_pair = 4 * wl.D                       # 2D for Q.K, 2D for P.V
    band_tflops = band_pairs * flops_per_pair / (band_ms * 1e-3) / 1e12
    peak = PEAK_TFLOPS[wl.dtype]
    band_cold_ms = quantiles(cold_band)[1]
    value = pairs / (ms * 1e-3)
    elem = 2 if wl.dtype == "bf16" else 4
    line = {
        "metric": METRIC,
        "value": value,
        "unit": "scored pairs/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.dtype,
        "data": "synthetic (seeded i.i.d. Gaussian Q, K, V)",
        "inputs": input_record(inp),
        "config": {"workload": wl.name, "variant": args.variant,
                   **({"chunk": args.chunk, "n_memory": len(wl.glob)}
                      if args.variant == "chunked" else {}),
                   "B": wl.B, "H": wl.H, "N": wl.N, "D": wl.D,
                   "window": None if args.variant == "chunked" else wl.window,
                   "dilation": [int(x) for x in inp.dilation],
                   "n_global": n_g, "scored_pairs": pairs, "parallelism": "single GPU"},
        "whole_forward_tflops": pairs * flops_per_pair / (ms * 1e-3) / 1e12,
        "whole_forward_mfma_frac": pairs * flops_per_pair / (ms * 1e-3) / 1e12 / peak,
        "kernels_ms": {"band": band_ms, "global_rows": glob_ms},
        "warm_trials": {"trials": len(warm), "forwards_per_trial": rep,
                        "median_ms": quantiles(warm)[1],
                        "iqr_ms": quantiles(warm)[2] - quantiles(warm)[0]},
        "cold_cache": {"trials": len(cold), "median_ms": quantiles(cold)[1],
                       "iqr_ms": quantiles(cold)[2] - quantiles(cold)[0],
                       "band_median_ms": band_cold_ms,
                       "band_frac": band_pairs * flops_per_pair / (band_cold_ms * 1e-3) / 1e12
                       / peak},
        "roofline": {
            "kernel": "band_kernel",
            "bound": "mfma",
            "achieved": band_tflops,
            "peak": peak,
            "unit": "TFLOP/s",
            "frac": band_tflops / peak,
            "traffic": recorded_traffic(wl.name) if args.variant == "plain" else None,
            "algorithmic_flops_per_launch": band_pairs * flops_per_pair,
            "ideal_bytes_per_launch": 4 * wl.B * wl.H * wl.N * wl.D * elem,
        },
    }
    if not args.no_cpu and args.variant == "plain":
        line["cpu_baseline"] = cpu_baseline(inp, wl, pairs)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
