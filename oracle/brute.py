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


def attention_ex(q, k, v, window: int, dilation=None, batch_glob=None, qg=None, kg=None,
                 vg=None, scale: float | None = None):
    """The general form: one global set per batch element (batch_glob: B lists)
    and separate projections qg, kg, vg (None: q, k, v) for the global rows.

    Same mask construction per batch element; a global row's scores are
    qg_i . kg_j over every key, weighting vg (the Longformer glossary page's
    global-attention bullet: global attention has its own query, key and value
    projections); every other row keeps q, k, v and its mask row.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    qg = q if qg is None else np.asarray(qg, dtype=np.float64)
    kg = k if kg is None else np.asarray(kg, dtype=np.float64)
    vg = v if vg is None else np.asarray(vg, dtype=np.float64)
    B, H, N, D = q.shape
    if batch_glob is None:
        batch_glob = [[]] * B
    if scale is None or scale <= 0:
        scale = 1.0 / np.sqrt(D)
    out = np.empty((B, H, N, D), dtype=np.float64)
    for b in range(B):
        gset = sorted(set(int(x) for x in batch_glob[b]))
        for h in range(H):
            d = 1 if dilation is None else int(dilation[h])
            additive = np.where(band_global_mask(N, window, d, gset), 0.0, -np.inf)
            z = scale * (q[b, h] @ k[b, h].T) + additive
            z = z - z.max(axis=1, keepdims=True)
            w = np.exp(z)
            out[b, h] = (w @ v[b, h]) / w.sum(axis=1, keepdims=True)
            if gset:
                zg = scale * (qg[b, h][gset] @ kg[b, h].T)
                zg = zg - zg.max(axis=1, keepdims=True)
                wg = np.exp(zg)
                out[b, h][gset] = (wg @ vg[b, h]) / wg.sum(axis=1, keepdims=True)
    return out


def causal_band_mask(n: int, window: int, dilation: int = 1) -> np.ndarray:
    """Boolean [n, n] mask of the causal band: key j <= i with (i - j) a
    multiple of d and i - j <= d * (window // 2) (the symmetric band's lower
    triangle, diagonal included)."""
    pos = np.arange(n, dtype=np.int64)
    diff = pos[:, None] - pos[None, :]
    hw = window // 2
    return (diff >= 0) & (diff <= dilation * hw) & (diff % dilation == 0)


def attention_causal(q, k, v, window: int, dilation=None, scale: float | None = None):
    """Masked softmax attention over the causal band, float64 [B, H, N, D]."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, H, N, D = q.shape
    if scale is None or scale <= 0:
        scale = 1.0 / np.sqrt(D)
    out = np.empty((B, H, N, D), dtype=np.float64)
    for h in range(H):
        d = 1 if dilation is None else int(dilation[h])
        additive = np.where(causal_band_mask(N, window, d), 0.0, -np.inf)
        for b in range(B):
            z = scale * (q[b, h] @ k[b, h].T) + additive
            z = z - z.max(axis=1, keepdims=True)
            w = np.exp(z)
            out[b, h] = (w @ v[b, h]) / w.sum(axis=1, keepdims=True)
    return out


def chunked_mask(n: int, chunk: int, n_memory: int) -> np.ndarray:
    """Boolean [n, n] mask of GMAT's C x k chunked attention with n_memory
    memory tokens prefixed: block-diagonal chunks of the main sequence (which
    starts at n_memory), plus the memory rows and columns set to True."""
    pos = np.arange(n, dtype=np.int64)
    blk = np.where(pos >= n_memory, (pos - n_memory) // chunk, -1)
    mask = (blk[:, None] == blk[None, :]) & (blk[:, None] >= 0)
    mask[:n_memory, :] = True
    mask[:, :n_memory] = True
    return mask


def attention_chunked(q, k, v, chunk: int, n_memory: int, qg=None, kg=None, vg=None,
                      scale: float | None = None):
    """Masked softmax attention over the chunked pattern, float64; the memory
    rows take qg, kg, vg when given."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    qg = q if qg is None else np.asarray(qg, dtype=np.float64)
    kg = k if kg is None else np.asarray(kg, dtype=np.float64)
    vg = v if vg is None else np.asarray(vg, dtype=np.float64)
    B, H, N, D = q.shape
    if scale is None or scale <= 0:
        scale = 1.0 / np.sqrt(D)
    additive = np.where(chunked_mask(N, chunk, n_memory), 0.0, -np.inf)
    out = np.empty((B, H, N, D), dtype=np.float64)
    for b in range(B):
        for h in range(H):
            z = scale * (q[b, h] @ k[b, h].T) + additive
            z = z - z.max(axis=1, keepdims=True)
            w = np.exp(z)
            out[b, h] = (w @ v[b, h]) / w.sum(axis=1, keepdims=True)
            if n_memory:
                zg = scale * (qg[b, h][:n_memory] @ kg[b, h].T)
                zg = zg - zg.max(axis=1, keepdims=True)
                wg = np.exp(zg)
                out[b, h][:n_memory] = (wg @ vg[b, h]) / wg.sum(axis=1, keepdims=True)
    return out
