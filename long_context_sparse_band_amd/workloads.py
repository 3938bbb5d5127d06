"""Seeded synthetic workloads for band + global sparse attention.

This module only makes inputs: shapes, seeds, random Q/K/V and the pattern
parameters (window, per-head dilation, global positions).  It holds none of the
attention arithmetic, imports neither the GPU library nor the CPU oracle, and
serves both.

The shapes stand in for the pages' workloads, whose datasets and trained
weights are not available: the released Longformer models read 4,096 tokens
with 256 neighbours on each side (Ultralytics glossary "Longformer", opening
paragraph and the sliding-window bullet); a char-level language model uses
dilation on some heads (same page, dilated-window bullet); GMAT prefixes M
memory tokens to the main sequence ("GMAT: Global Memory Augmentation for
Transformers", section "Global Memory").  Q, K and V are i.i.d. Gaussian.

Generator recipe (fixed, so every run sees the same bytes): numpy
Generator(PCG64(seed)); Q, K, V drawn in that order with standard_normal in
float32, shape [B, H, N, D], times the config's std; then (only where the
config asks) the random global positions, drawn without replacement from
[0, N) and sorted; then the outlier key rows, drawn without replacement from
the B*H*N rows of K and multiplied by the outlier factor.  bf16 configs round
the float32 values to bfloat16 with round-to-nearest-even.
"""

from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    N: int
    D: int
    dtype: str  # "f32" or "bf16"
    window: int
    dilation: tuple  # one int per head
    glob: tuple = ()  # fixed global positions (may be empty)
    n_random_glob: int = 0  # extra global positions drawn from the seed
    std: float = 1.0
    outlier_frac: float = 0.0  # fraction of key rows scaled by outlier_mult
    outlier_mult: float = 1.0
    seed: int = 0
    note: str = field(default="", compare=False)


def _dil(H, rule=None):
    return tuple(1 for _ in range(H)) if rule is None else tuple(rule)


# The five workloads, smallest first.
SINGLE_HEAD_F32 = Workload(
    "single_head_n1024_f32", B=1, H=1, N=1024, D=64, dtype="f32", window=512,
    dilation=_dil(1), glob=(0,), seed=20261,
    note="one head, window 512, one global token at 0, scale 1/sqrt(64)")
LONGFORMER_BASE = Workload(
    "longformer_base_n4096", B=1, H=12, N=4096, D=64, dtype="bf16", window=512,
    dilation=_dil(12), glob=tuple(range(32)), seed=20262,
    note="Longformer-base shape: window 512, global token 0 plus 31 question-like tokens 1..31")
DILATED_CHARLM = Workload(
    "dilated_charlm_n8192", B=2, H=8, N=8192, D=64, dtype="bf16", window=512,
    dilation=(1, 1, 1, 1, 1, 1, 2, 2), glob=(), seed=20263,
    note="window 512; heads 0-5 dilation 1, heads 6-7 dilation 2; no global tokens")
GMAT_MEMORY = Workload(
    "gmat_memory_m64_l16384", B=1, H=16, N=16448, D=64, dtype="bf16", window=256,
    dilation=_dil(16), glob=tuple(range(64)), seed=20264,
    note="64 memory tokens prefixed to 16384 main tokens; main window 256")
LONG_STRESS = Workload(
    "long_stress_n65536_d128", B=1, H=16, N=65536, D=128, dtype="bf16", window=1024,
    dilation=_dil(16), glob=(), n_random_glob=64, std=0.5, outlier_frac=0.01,
    outlier_mult=4.0, seed=20265,
    note="std 0.5, 1% of key rows x4, window 1024, 64 global tokens at seeded positions")

WORKLOADS = (SINGLE_HEAD_F32, LONGFORMER_BASE, DILATED_CHARLM, GMAT_MEMORY, LONG_STRESS)
BY_NAME = {w.name: w for w in WORKLOADS}


def bf16_round_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns (uint16), round to nearest, ties to even.

    Textbook RNE on the top 16 bits of the IEEE-754 single; inputs are finite.
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    return ((u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns -> the float32 values they denote (exact)."""
    return (np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32)
            << np.uint32(16)).view(np.float32)


@dataclass
class Inputs:
    """One generated problem.

    q, k, v: float32 [B, H, N, D] holding exactly the values the GPU sees
    (already bf16-representable for bf16 workloads).  *_bits: the bf16 bit
    patterns (uint16) for bf16 workloads, else None.  glob: sorted int32
    positions; dilation: int32 [H].
    """
    wl: Workload
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    q_bits: np.ndarray | None
    k_bits: np.ndarray | None
    v_bits: np.ndarray | None
    glob: np.ndarray
    dilation: np.ndarray


def generate(wl: Workload) -> Inputs:
    """Draw the workload's inputs with the recipe in the module docstring."""
    rng = np.random.Generator(np.random.PCG64(wl.seed))
    shape = (wl.B, wl.H, wl.N, wl.D)
    arrs = []
    for _ in range(3):
        a = rng.standard_normal(shape, dtype=np.float32)
        if wl.std != 1.0:
            a *= np.float32(wl.std)
        arrs.append(a)
    q, k, v = arrs
    glob = set(int(g) for g in wl.glob)
    if wl.n_random_glob:
        extra = rng.choice(wl.N, size=wl.n_random_glob, replace=False)
        glob.update(int(g) for g in extra)
    if wl.outlier_frac > 0.0:
        rows = wl.B * wl.H * wl.N
        n_out = int(round(wl.outlier_frac * rows))
        pick = rng.choice(rows, size=n_out, replace=False)
        k.reshape(rows, wl.D)[pick] *= np.float32(wl.outlier_mult)
    bits = [None, None, None]
    if wl.dtype == "bf16":
        bits = [bf16_round_bits(a) for a in (q, k, v)]
        q, k, v = (bf16_bits_to_f32(b).reshape(shape) for b in bits)
        bits = [b.reshape(shape) for b in bits]
    return Inputs(wl, q, k, v, bits[0], bits[1], bits[2],
                  np.array(sorted(glob), dtype=np.int32),
                  np.array(wl.dilation, dtype=np.int32))


def small_case(B, H, N, D, dtype, window, dilation=None, glob=(), seed=0, std=1.0,
               outlier_frac=0.0, outlier_mult=1.0) -> Inputs:
    """A test-sized problem drawn with the same recipe."""
    wl = Workload("case", B=B, H=H, N=N, D=D, dtype=dtype, window=window,
                  dilation=_dil(H, dilation), glob=tuple(int(g) for g in glob), std=std,
                  outlier_frac=outlier_frac, outlier_mult=outlier_mult, seed=seed)
    return generate(wl)
