"""Head-to-sequence re-layout (the post-attention All-to-All seen from one GPU).

TEST INFRASTRUCTURE ONLY (see the package docstring).

Ulysses sequence parallelism (X-Stage abstract, CatalyzeX / fugumt pages)
gives each GPU a share of the heads over the full sequence for attention and
returns afterwards to sequence sharding.  With P destinations, destination p
owns the contiguous tokens [p*S/P, (p+1)*S/P).  On one GPU the P destinations
are P local slabs, and slab p holds its tokens token-major with the local
heads inside each token:

    out[p][b][t][h][d] = O[b][h][p * S/P + t][d]

Two derivations that share nothing but this statement:
  * ``relayout_split``: slice the sequence into P chunks, swap the head and
    token axes of each chunk, stack the chunks;
  * ``relayout_index``: scatter every element of O to the flat offset
    (((p*B + b)*S/P + t)*H + h)*D + d.
"""
from __future__ import annotations

import numpy as np


def _check(o: np.ndarray, P: int):
    if o.ndim != 4:
        raise ValueError("O must be [B][H][S][D]")
    S = o.shape[2]
    if P <= 0 or S % P != 0:
        raise ValueError("S must be a positive multiple of P")
    return o.shape


def relayout_split(o: np.ndarray, P: int) -> np.ndarray:
    """[B][H][S][D] -> [P][B][S/P][H][D] by split, transpose and stack."""
    B, H, S, D = _check(o, P)
    Sp = S // P
    chunks = [o[:, :, p * Sp:(p + 1) * Sp, :] for p in range(P)]
    return np.stack([np.transpose(c, (0, 2, 1, 3)) for c in chunks], axis=0)


def relayout_index(o: np.ndarray, P: int) -> np.ndarray:
    """[B][H][S][D] -> [P][B][S/P][H][D] by scattering each source element to
    its closed-form destination offset."""
    B, H, S, D = _check(o, P)
    Sp = S // P
    b = np.arange(B)[:, None, None, None]
    h = np.arange(H)[None, :, None, None]
    s = np.arange(S)[None, None, :, None]
    d = np.arange(D)[None, None, None, :]
    p, t = s // Sp, s % Sp
    dest = (((p * B + b) * Sp + t) * H + h) * D + d
    flat = np.empty(B * H * S * D, dtype=o.dtype)
    flat[dest.reshape(-1)] = o.reshape(-1)
    return flat.reshape(P, B, Sp, H, D)


def plain_layout(o: np.ndarray) -> np.ndarray:
    """The plain [B][H][S][D] output layout, unchanged (the baseline the fused
    store is measured against)."""
    return np.ascontiguousarray(o)
