"""Plain float64 softmax attention, the definition FlashAttention reproduces.

TEST INFRASTRUCTURE ONLY (see the package docstring).

For one (batch, head) with queries Q, keys K and values V (rows are tokens):

    z[s, j]  = scale * <Q[s], K[j]>
    z[s, j]  = -inf   where the 128x128 tile (s // 128, j // 128) is masked
    P[s, j]  = exp(z[s, j] - max_j z[s, j]) / sum_j exp(z[s, j] - max_j z[s, j])
    O[s]     = sum_j P[s, j] V[j]

A row whose keys are all masked has no softmax; its output is defined as 0.
Sources: X-Stage abstract (CatalyzeX / fugumt pages) -- FlashAttention inside
Ulysses sequence-parallel attention; ScalingAttention abstract (CatalyzeX
page) -- bit-wise block-sparse attention where masked tiles are skipped.
Query rows are processed in blocks of ``row_block`` only to bound memory: each
block is the full definition over all keys.
"""
from __future__ import annotations

from typing import Optional, Sequence

import numpy as np

MASK_TILE = 128


def unpack_mask(words: np.ndarray, S: int) -> np.ndarray:
    """uint64 [H][nT][W] -> bool [H][nT][nT]: tile (i, j) of head h is kept
    when bit (j % 64) of word (j // 64) in row (h, i) is set."""
    words = np.asarray(words, dtype=np.uint64)
    H, nT, W = words.shape
    if nT != (S + MASK_TILE - 1) // MASK_TILE or W != (nT + 63) // 64:
        raise ValueError("mask shape does not match S")
    keep = np.zeros((H, nT, nT), dtype=bool)
    for j in range(nT):
        bit = (words[:, :, j // 64] >> np.uint64(j % 64)) & np.uint64(1)
        keep[:, :, j] = bit.astype(bool)
    return keep


def _row_blocks(S: int, rows: Optional[Sequence[int]], row_block: int):
    if rows is None:
        for r0 in range(0, S, row_block):
            yield np.arange(r0, min(S, r0 + row_block))
    else:
        rows = np.asarray(rows, dtype=np.int64)
        for r0 in range(0, len(rows), row_block):
            yield rows[r0:r0 + row_block]


def attention_probs(q: np.ndarray, k: np.ndarray, scale: float,
                    keep: Optional[np.ndarray] = None,
                    rows: Optional[np.ndarray] = None) -> np.ndarray:
    """Softmax probabilities P[rows, :] of one (batch, head).

    q, k: float64 [S][D]; keep: bool [nT][nT] or None; rows: query indices
    (default all).  Fully masked rows come back as all-zero rows.
    """
    S = k.shape[0]
    rows = np.arange(S) if rows is None else np.asarray(rows, dtype=np.int64)
    z = (q[rows] @ k.T) * scale
    if keep is not None:
        allowed = keep[rows // MASK_TILE][:, np.arange(S) // MASK_TILE]
        z = np.where(allowed, z, -np.inf)
    m = z.max(axis=1, keepdims=True)
    dead = ~np.isfinite(m[:, 0])
    m[dead] = 0.0
    e = np.exp(z - m)
    l = e.sum(axis=1, keepdims=True)
    l[dead] = 1.0
    p = e / l
    p[dead] = 0.0
    return p


def attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float,
              mask_words: Optional[np.ndarray] = None,
              rows: Optional[Sequence[int]] = None,
              row_block: int = 128) -> np.ndarray:
    """softmax(scale Q K^T) V for every (batch, head).

    q, k: float64 [B][H][S][D] (the exact values of the bf16 inputs); v:
    float64 [B][H][S][Dv], the values averaged (Dv = D for attention itself;
    any width, since each output column is the same weighted sum of its own
    value column).  mask_words: optional uint64 [H][nT][ceil(nT/64)] tile
    keep-mask, shared by every batch index.  rows: optional query indices;
    the result then has shape [B][H][len(rows)][Dv] instead of [B][H][S][Dv].
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, H, S, D = q.shape
    if k.shape != q.shape or v.ndim != 4 or v.shape[:3] != q.shape[:3]:
        raise ValueError("q, k must share one [B][H][S][D] shape, v [B][H][S][Dv]")
    keep = None if mask_words is None else unpack_mask(mask_words, S)
    n_out = S if rows is None else len(rows)
    out = np.zeros((B, H, n_out, v.shape[3]), dtype=np.float64)
    for b in range(B):
        for h in range(H):
            kh = None if keep is None else keep[h]
            pos = 0
            for blk in _row_blocks(S, rows, row_block):
                p = attention_probs(q[b, h], k[b, h], scale, kh, blk)
                out[b, h, pos:pos + len(blk)] = p @ v[b, h]
                pos += len(blk)
    return out
