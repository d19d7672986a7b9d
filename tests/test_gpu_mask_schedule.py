"""GPU: the schedule of block-masked launches.

Every workgroup derives the same schedule from the mask: the rounds of G
units of the plain order (G = the persistent grid), each dealt in decreasing
kept-tile count K (ties by index) in snake order -- in even rounds slot w
takes the w-th costliest unit, in odd rounds the (G - 1 - w)-th, where the
workgroup with block id b holds slot (b mod 8) G/8 + floor(b / 8) when 8
divides G (the XCD-aware order: the hardware deals blocks to the 8 XCDs
round-robin), else slot b.  The timestamped instances record which
workgroup ran each unit (include/fa_instrument.h), so the test compares that
assignment with the schedule computed here from its definition; beyond the
schedule's limits (more mask rows than kb0 holds as int counts, 8192 at D =
128, or more than 256 rounds) the launch keeps the plain order, unit u on
slot u mod G.
The outputs equal the product kernel's bit for bit and meet the float64
oracle on sampled rows.
"""
import math
import sys

import numpy as np
import pytest
import torch

import flashattention_output_re_amd as fa
from flashattention_output_re_amd import binding, tile_stamps
import oracle
import workloads as wl
from gpu_util import assert_close, mask_to_dev, sample_rows, slab_rows, to_dev

pytestmark = pytest.mark.gpu


def _cus():
    return torch.cuda.get_device_properties(0).multi_processor_count


def slot_of_block(b, G):
    """The XCD-aware slot of block id b on a grid of G."""
    return (b % 8) * (G // 8) + b // 8 if G % 8 == 0 else b


def expected_schedule(kept, G):
    """Slot of each unit under the round-wise snake rule."""
    units = len(kept)
    wg_of = np.full(units, -1, dtype=np.int64)
    for r, base in enumerate(range(0, units, G)):
        us = np.arange(base, min(units, base + G))
        by_k = us[np.lexsort((us, -kept[us]))]           # decreasing K, ties by index
        for rank, u in enumerate(by_k):
            wg_of[u] = rank if r % 2 == 0 else G - 1 - rank
    return wg_of


def _rows_mask(H, nT):
    """Rows with nothing kept, everything kept, and every other tile."""
    m = np.zeros((H, nT, nT), dtype=bool)
    for h in range(H):
        for i in range(nT):
            kind = (h + i) % 3
            if kind == 1:
                m[h, i] = True
            elif kind == 2:
                m[h, i] = np.arange(nT) % 2 == i % 2
    return m


# (B, H, S, P, keep probability or "rows"); D = 128 (timestamped instances).
CASES = {
    "fewer units than workgroups, ragged S": (1, 1, 1000, 4, 0.4),
    "several rounds, B=2, last round partial": (2, 3, 8000, 4, 0.3),
    "empty rows and full rows": (1, 4, 6144, 2, "rows"),
    "block-sparse video shape": (1, 5, 32760, 8, 0.3),
    "beyond the limit: plain order": (1, 33, 32768, 8, 0.02),
}


@pytest.mark.parametrize("case", sorted(CASES))
def test_masked_schedule(case):
    B, H, S, P, keep = CASES[case]
    D = 128
    print(f"[mask schedule] {case}: B={B} H={H} S={S} D={D} P={P}", file=sys.stderr, flush=True)
    nT = (S + 127) // 128
    keepm = _rows_mask(H, nT) if keep == "rows" else wl.tile_mask_bool(H, S, keep, seed=S)
    words = wl.pack_mask(keepm)
    q, k, v = wl.random_qkv(B, H, S, D, seed=S + 7 * H)
    qd, kd, vd = to_dev(q), to_dev(k), to_dev(v)
    m = mask_to_dev(words)
    scale = 1.0 / math.sqrt(D)
    ref = torch.empty((P, B, S // P, H, D), dtype=torch.bfloat16, device=qd.device)
    fa.attn_fwd_relayout_async(qd, kd, vd, ref, B, H, S, D, P, scale, m)
    out = torch.full_like(ref, float("nan"))
    stamps = torch.zeros(binding.attn_instrumented_stamp_words(B, H, S), dtype=torch.int32,
                         device=qd.device)
    launch = binding.attn_fwd_relayout_instrumented_async(qd, kd, vd, out, B, H, S, D, P, scale,
                                                          m, 0, stamps)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), ref.view(torch.int16))
    units = B * H * nT
    assert list(launch) == [units, 0]
    (rec,) = tile_stamps.records(stamps.cpu().numpy().view(np.uint32), launch)
    G = min(units, _cus())
    ran_on = slot_of_block(rec[:, 0, 6].astype(np.int64), G)
    kept = np.tile(keepm.sum(-1).reshape(-1), B).astype(np.int64)
    if H * nT > 8192 or (units + G - 1) // G > 256:
        want = np.arange(units) % G
    else:
        want = expected_schedule(kept, G)
    assert np.array_equal(ran_on, want), \
        f"{int((ran_on != want).sum())} of {units} units on another workgroup"
    # The schedule's balance: the busiest workgroup's cost (K + 7 stage
    # times a unit, the fit of the timestamps) against the mean.
    load = np.bincount(ran_on, weights=kept + 7, minlength=G)
    print(f"[mask schedule] {case}: busiest/mean cost {load.max() / load.mean():.4f}",
          file=sys.stderr, flush=True)
    rows = sample_rows(S, P, seed=S, n_random=8)
    want_o = oracle.attention(q.double().numpy(), k.double().numpy(), v.double().numpy(), scale,
                              words, rows=rows[:40])
    assert_close(slab_rows(out, rows[:40], S, P), want_o, f"masked schedule {case}")
