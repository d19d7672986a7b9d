"""Seeded synthetic inputs for the fused attention + Ulysses re-layout path.

This module is shared by the CPU oracle's tests, the GPU parity tests and the
benchmark.  It holds input construction only -- shapes, random draws, the
block-sparse tile mask and its bit packing, integer-tagged inputs -- and none
of the attention or re-layout arithmetic.

Workload shapes stand in for the diffusion-transformer (DiT) attention the
X-Stage pages describe (abstract on the CatalyzeX and fugumt pages; "Technical
Summary: X-Stage in DiT Inference", Key Contributions 3).  The pages give no
sequence lengths, head counts or head dimension, so the shapes are DiT-like:
an image latent of 64x64 patches and video latents of 21x30x52 and 21x60x60
patches, each seen as one GPU's head share of a Ulysses-sharded layer.  The
block-sparse case follows the bit-wise 128x128 tile mask of the ScalingAttention
abstract (CatalyzeX page), with the mask drawn from a seed instead of being
extracted from model weights.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np
import torch

TILE = 128  # mask tile edge, in tokens (queries and keys)


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    S: int
    D: int
    P: int
    seed: int
    kscale: Optional[tuple] = None      # per-head K multiplier ~ U(lo, hi)
    keep_prob: Optional[float] = None   # block-sparse: P(keep off-diagonal tile)

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.D)

    @property
    def n_tiles(self) -> int:
        return (self.S + TILE - 1) // TILE

    @property
    def slab_tokens(self) -> int:
        return self.S // self.P


# The workloads, in a fixed order; the base seed of entry i is 1000 + i.  The
# last is the Video share at head dimension 64 (the pages name no head
# dimension; DiT models use both 64 and 128).
WORKLOADS = {
    "tiny": Workload("tiny", B=1, H=1, S=256, D=64, P=2, seed=1000),
    "image": Workload("image", B=1, H=3, S=4096, D=128, P=8, seed=1001),
    "video": Workload("video", B=1, H=5, S=32760, D=128, P=8, seed=1002,
                      kscale=(0.5, 2.0)),
    "long": Workload("long", B=1, H=5, S=75600, D=128, P=8, seed=1003),
    "sparse": Workload("sparse", B=1, H=5, S=32760, D=128, P=8, seed=1004,
                       keep_prob=0.3),
    "video64": Workload("video64", B=1, H=5, S=32760, D=64, P=8, seed=1005,
                        kscale=(0.5, 2.0)),
}

DESCRIPTIONS = {
    "tiny": "Tiny: B=1 H=1 S=256 D=64 P=2",
    "image": "Image-DiT share: B=1 H=3 S=4096 (64x64 latent) D=128 P=8",
    "video": "Video-DiT share: B=1 H=5 S=32760 (21x30x52 latent) D=128 P=8, "
             "per-head K scale U(0.5,2)",
    "long": "Long video share: B=1 H=5 S=75600 (21x60x60 latent) D=128 P=8",
    "sparse": "Block-sparse video: B=1 H=5 S=32760 D=128 P=8, 128x128 tiles, "
              "70% sparsity, diagonal kept",
    "video64": "Video-DiT share at head dimension 64: B=1 H=5 S=32760 D=64 P=8, "
               "per-head K scale U(0.5,2)",
}


@dataclasses.dataclass
class Inputs:
    """bf16 tensors on the host plus their exact float64 values."""
    q: torch.Tensor          # bf16 [B][H][S][D], contiguous, CPU
    k: torch.Tensor
    v: torch.Tensor
    mask: Optional[np.ndarray]   # uint64 [H][nT][W] or None (dense)

    def f64(self, name: str) -> np.ndarray:
        return getattr(self, name).to(torch.float64).numpy()


def _streams(seed: int):
    kids = np.random.SeedSequence(seed).spawn(5)
    return [np.random.Generator(np.random.PCG64(s)) for s in kids]


def to_bf16(x: np.ndarray) -> torch.Tensor:
    """fp32 array -> bf16 tensor, round-to-nearest-even (torch's cast)."""
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)


def random_qkv(B: int, H: int, S: int, D: int, seed: int,
               kscale: Optional[tuple] = None):
    """Q, K, V drawn i.i.d. N(0,1) in fp32 from independent streams, cast to bf16.

    With ``kscale=(lo, hi)`` one factor per head is drawn after K from U(lo, hi)
    and multiplies that head's fp32 K before the cast, which varies how sharp
    each head's softmax is.
    """
    gq, gk, gv, gs, _ = _streams(seed)
    q = gq.standard_normal((B, H, S, D), dtype=np.float32)
    k = gk.standard_normal((B, H, S, D), dtype=np.float32)
    v = gv.standard_normal((B, H, S, D), dtype=np.float32)
    if kscale is not None:
        c = gs.uniform(kscale[0], kscale[1], size=H).astype(np.float32)
        k *= c[None, :, None, None]
    return to_bf16(q), to_bf16(k), to_bf16(v)


def tile_mask_bool(H: int, S: int, keep_prob: float, seed: int) -> np.ndarray:
    """Per-head [H][nT][nT] keep-flags: diagonal tiles always kept, every other
    tile kept independently with probability ``keep_prob``."""
    nT = (S + TILE - 1) // TILE
    g = _streams(seed)[4]
    keep = g.random((H, nT, nT)) < keep_prob
    idx = np.arange(nT)
    keep[:, idx, idx] = True
    return keep


def pack_mask(keep: np.ndarray) -> np.ndarray:
    """[H][nT][nT] bool -> uint64 [H][nT][ceil(nT/64)]; tile (i, j) of head h is
    bit (j % 64) of word (j // 64) in row (h, i)."""
    H, nT, nT2 = keep.shape
    assert nT == nT2
    W = (nT + 63) // 64
    words = np.zeros((H, nT, W), dtype=np.uint64)
    for j in range(nT):
        words[:, :, j // 64] |= keep[:, :, j].astype(np.uint64) << np.uint64(j % 64)
    return words


def make(name_or_wl, seed: Optional[int] = None) -> Inputs:
    wl = WORKLOADS[name_or_wl] if isinstance(name_or_wl, str) else name_or_wl
    s = wl.seed if seed is None else seed
    q, k, v = random_qkv(wl.B, wl.H, wl.S, wl.D, s, wl.kscale)
    mask = None
    if wl.keep_prob is not None:
        mask = pack_mask(tile_mask_bool(wl.H, wl.S, wl.keep_prob, s))
    return Inputs(q, k, v, mask)


# ---------------------------------------------------------------- tag inputs
def tag_digits(S: int, D: int):
    """Smallest digit count n (and base b) with b**n >= S and n*b <= D."""
    for n in range(1, 9):
        b = max(2, math.ceil(S ** (1.0 / n)))
        while b ** n < S:
            b += 1
        if n * b <= D:
            return b, n
    raise ValueError(f"no tag code for S={S}, D={D}")


def tag_inputs(B: int, H: int, S: int, D: int) -> Inputs:
    """Integer-tagged inputs whose attention output is exactly V.

    Token s is written in base b with n digits; Q[s] and K[s] carry 16 at the
    one-hot position of each digit (one block of b dims per digit).  Then
    q_s . k_s = 256 n while every other key shares at most n-1 digits and
    scores at most 256 (n-1): after the 1/sqrt(D) scale that is a gap of at
    least 22 nats, so each softmax row is one-hot on its own key up to ~1e-8.
    V holds small positive integers (exact in bf16) that encode (b, h, s, d),
    so the attention output equals V bit-for-bit after bf16 rounding and any
    misplaced row, head, batch or column is visible in the re-layout.
    """
    b_, n = tag_digits(S, D)
    s = np.arange(S)
    qk = np.zeros((S, D), dtype=np.float32)
    rem = s.copy()
    for i in range(n):
        dig = rem % b_
        rem //= b_
        qk[s, i * b_ + dig] = 16.0
    q = np.broadcast_to(qk, (B, H, S, D)).copy()
    v = np.empty((B, H, S, D), dtype=np.float32)
    d = np.arange(D)
    for bi in range(B):
        for h in range(H):
            t = np.empty((S, D), dtype=np.float32)
            t[:] = 1 + (d[None, :] * 7 + s[:, None] * 3) % 251
            t[:, 0] = 1 + s % 128
            t[:, 1] = 1 + (s >> 7) % 128
            t[:, 2] = 1 + (s >> 14)
            if D > 3:
                t[:, 3] = 1 + h
            if D > 4:
                t[:, 4] = 1 + bi
            v[bi, h] = t
    return Inputs(to_bf16(q), to_bf16(q), to_bf16(v), None)


def flop_count(B: int, H: int, S: int, D: int, keep: Optional[np.ndarray] = None) -> float:
    """Algorithmic FLOP of softmax(Q K^T) V: 4 D per (query, kept key) pair.

    ``keep`` ([H][nT][nT] bool) restricts the count to kept 128x128 tiles, with
    ragged tail tiles counted at their true size."""
    if keep is None:
        return 4.0 * B * H * S * S * D
    nT = keep.shape[1]
    sizes = np.full(nT, TILE, dtype=np.float64)
    sizes[-1] = S - TILE * (nT - 1)
    pairs = np.einsum("hij,i,j->", keep.astype(np.float64), sizes, sizes)
    return 4.0 * B * D * pairs
