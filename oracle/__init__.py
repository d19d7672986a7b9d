"""CPU oracle for fused attention + Ulysses head-to-sequence re-layout.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path imports this package:
only the test suite, the smoke check in ``__graft_entry__`` and the CPU
baseline leg of ``bench.py`` may use it.  It shares no code, headers, tables
or helpers with the HIP library; the two meet only in the seeded input
generators of the ``workloads`` package, which hold no attention arithmetic.

What it computes, in float64 and in the plainest form:

* ``attention`` -- softmax(scale * Q K^T) V per (batch, head), non-causal,
  with an optional per-head 128x128 tile keep-mask (masked tiles contribute
  nothing to the softmax).  FlashAttention's tiled online softmax is an exact
  reformulation of this, so the oracle is the definition itself with no
  tiling over keys, no online rescaling and no reordering.
* ``relayout_split`` and ``relayout_index`` -- the post-attention All-to-All of
  Ulysses sequence parallelism seen from one GPU: the output [B][H][S][D] is
  split along the sequence into P contiguous token ranges, one per destination
  slab, each slab holding [B][S/P][H][D].  Two independent derivations (split
  then transpose; scatter by the closed-form index) that must agree exactly.

Sources: the X-Stage abstract (CatalyzeX and fugumt pages) names Ulysses
sequence-parallel attention with the post-attention All-to-All fused into
FlashAttention; "Technical Summary: X-Stage in DiT Inference", Key
Contributions 3 (FlashAttention-A2A piggybacking) says the output-tile owner
stores the tile to its destination and resumes the next tile's Q-loop.  The
ScalingAttention abstract (CatalyzeX page) describes the bit-wise block-sparse
kernel.  For attention and the re-layout the pages print no formula, layout
or worked example; every reading taken where they are silent is listed with
the design notes.

* ``burst_gap`` -- the one formula the pages do print: the Burst-Gap model of
  sender-visible store-issue time (Methodology section of the technical
  summary), used to check the fit of the store-burst microbenchmark.

Pins (tests/test_oracle_pins.py): hand-derived exact examples
(tests/golden/), identical keys -> mean of V, one dominant score -> that V
row, V == 1 -> 1, torch's fp64 scaled_dot_product_attention on small cases,
row-permutation / key-shift / linearity invariants, block-diagonal masks
against independent per-block attention, a hand-written re-layout example,
and planted mistakes that the pins must catch.  Every function here is pinned.
"""
from .attn import attention, attention_probs, unpack_mask
from .relayout import relayout_split, relayout_index, plain_layout
from . import burst_gap

__all__ = ["attention", "attention_probs", "unpack_mask",
           "relayout_split", "relayout_index", "plain_layout", "burst_gap"]
