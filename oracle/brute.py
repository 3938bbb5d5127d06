"""Brute-force mask form of band + global attention, in numpy float64.

TEST INFRASTRUCTURE, NOT PART OF THE PRODUCT.  Only the test suite may use it.

This is a second, independent construction of the same pattern as the C
oracle: instead of enumerating each row's key set, it materialises the full
N x N boolean mask the way the Ultralytics glossary page "Longformer" does in
its mask-counting sample (section on how the attention works): a band
predicate on |pos_i - pos_j| against window // 2, then whole rows and columns
set to True for the global tokens.  Dilation (the page's dilated sliding-window
bullet gives no formula) is read as: key j is in row i's band when
(j - i) is a multiple of d and |j - i| <= d * (window // 2).

Attention values follow Eq. (1) of "Unlimiformer: Long-Range Transformers with
Unlimited Length Input", section 2.3, as an additive mask with entries 0 or
-inf (the binary mask B of "GMAT: Global Memory Augmentation for Transformers",
section "Global-Memory Augmented Transformers"), then a row softmax.  Only for
tiny N: it costs N*N memory per head.
"""

from __future__ import annotations

import numpy as np


def band_global_mask(n: int, window: int, dilation: int = 1, glob=()) -> np.ndarray:
    """Boolean [n, n] mask: True where query row i scores key column j."""
    pos = np.arange(n, dtype=np.int64)
    diff = pos[:, None] - pos[None, :]
    hw = window // 2
    mask = (np.abs(diff) <= dilation * hw) & (diff % dilation == 0)
    for g in glob:
        mask[g, :] = True
        mask[:, g] = True
    return mask


def attention(q, k, v, window: int, dilation=None, glob=(), scale: float | None = None):
    """Masked softmax attention in float64.

    q, k, v: arrays [B, H, N, D].  dilation: H ints or None (all 1).
    Returns float64 [B, H, N, D].
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, H, N, D = q.shape
    if scale is None or scale <= 0:
        scale = 1.0 / np.sqrt(D)
    out = np.empty((B, H, N, D), dtype=np.float64)
    for h in range(H):
        d = 1 if dilation is None else int(dilation[h])
        mask = band_global_mask(N, window, d, glob)
        additive = np.where(mask, 0.0, -np.inf)
        for b in range(B):
            z = scale * (q[b, h] @ k[b, h].T) + additive
            z = z - z.max(axis=1, keepdims=True)
            w = np.exp(z)
            out[b, h] = (w @ v[b, h]) / w.sum(axis=1, keepdims=True)
    return out
