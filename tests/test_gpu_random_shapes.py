"""GPU: a seeded sweep of shapes through every attention entry point.

Each case draws B, H, S, D, P, a scale and optionally a block mask from a
fixed seed, so that the launch plans the ABI picks -- whole rounds, split
half tiles, the spread last round (lead and helper pieces), half tiles cut
into key pieces, masked schedules and their plain-order fallback -- meet
shapes no hand-written case names; a second sweep draws longer sequences
sized so that the _ws_ entry points run the dynamic schedule (the last
round's tiles in key pieces handed out from a counter).  The output must meet the float64 oracle
on sampled rows (tile and slab edges, the ragged tail, random rows) -- the
element-wise bound from the arithmetic in every case, the workload gate in
the cases at the workloads' scale 1/sqrt(D) -- fill every slab element, and
repeat bit for bit on a second call.
"""
import math
import sys

import numpy as np
import pytest
import torch

import flashattention_output_re_amd as fa
import oracle
import workloads as wl
from gpu_util import (Guarded, assert_close, assert_within_bound, mask_to_dev, sample_rows,
                      slab_rows)

pytestmark = pytest.mark.gpu

ENTRIES = ["relayout", "relayout_ws", "plain_ws", "slab_to_slab_ws"]


def _case(i):
    r = np.random.default_rng(7000 + i)
    D = int(r.choice([64, 128]))
    P = int(r.choice([1, 2, 3, 4, 8]))
    entry = ENTRIES[i % len(ENTRIES)]
    lo = 64 * P if entry == "slab_to_slab_ws" else 1
    S = P * int(r.integers(max(1, lo // P), 12000 // P + 1))
    B = int(r.choice([1, 1, 2]))
    H = int(r.integers(1, 7))
    keep = None if r.random() < 0.6 else float(r.choice([0.1, 0.5]))
    scale = float(r.choice([1.0 / math.sqrt(D), 0.3, -0.3]))
    return dict(B=B, H=H, S=S, D=D, P=P, keep=keep, scale=scale, entry=entry, seed=7000 + i)


def _run(c, q, k, v, mask):
    B, H, S, D, P, scale = c["B"], c["H"], c["S"], c["D"], c["P"], c["scale"]
    e = c["entry"]
    if e == "plain_ws":
        out = torch.full((B, H, S, D), float("nan"), dtype=torch.bfloat16, device="cuda:0")
        fa.attn_fwd_plain_ws_async(q, k, v, out, B, H, S, D, scale, mask)
        torch.cuda.synchronize()
        assert not torch.isnan(out.float()).any(), "output left unwritten"
        # [B][H][S][D] -> slabs [P][B][S/P][H][D]
        return out.permute(0, 2, 1, 3).reshape(B, P, S // P, H, D).permute(1, 0, 2, 3, 4).contiguous()
    g = Guarded((P, B, S // P, H, D))
    if e == "relayout":
        fa.attn_fwd_relayout_async(q, k, v, g.out, B, H, S, D, P, scale, mask)
    elif e == "relayout_ws":
        fa.attn_fwd_relayout_ws_async(q, k, v, g.out, B, H, S, D, P, scale, mask)
    else:
        def to_slabs(t):
            return t.view(B, H, P, S // P, D).permute(2, 0, 3, 1, 4).contiguous()
        fa.attn_fwd_slab_to_slab_ws_async(to_slabs(q), to_slabs(k), to_slabs(v), g.out, B, H, S, D,
                                          P, scale, mask)
    torch.cuda.synchronize()
    g.check_guards()
    assert g.unwritten() == 0, "slab elements left unwritten"
    return g.out.clone()


@pytest.mark.parametrize("i", range(24))
def test_random_shape(i):
    c = _case(i)
    print(f"[random shapes] {i}: {c}", file=sys.stderr, flush=True)
    B, H, S, D, P = c["B"], c["H"], c["S"], c["D"], c["P"]
    q, k, v = wl.random_qkv(B, H, S, D, seed=c["seed"])
    words = None
    if c["keep"] is not None:
        words = wl.pack_mask(wl.tile_mask_bool(H, S, c["keep"], seed=c["seed"]))
    mask = None if words is None else mask_to_dev(words)
    qd, kd, vd = (t.to("cuda:0") for t in (q, k, v))
    got = _run(c, qd, kd, vd, mask)
    again = _run(c, qd, kd, vd, mask)
    assert torch.equal(got.view(torch.int16), again.view(torch.int16)), "second call differs"
    rows = sample_rows(S, P, seed=c["seed"], n_random=8)
    vv = np.concatenate([v.double().numpy(), np.abs(v.double().numpy())], axis=-1)
    both = oracle.attention(q.double().numpy(), k.double().numpy(), vv, c["scale"], words,
                            rows=rows)
    ref, absv = both[..., :D], both[..., D:]
    g = slab_rows(got, rows, S, P)
    # The element-wise bound from the arithmetic holds at every scale; the
    # workload gate (absolute max/mean) is defined at the workloads' scale
    # 1/sqrt(D), where the outputs average many keys.
    assert_within_bound(g, ref, absv, f"case {i}")
    if c["scale"] == 1.0 / math.sqrt(D):
        assert_close(g, ref, f"case {i}")


def _dyn_case(i, n):
    """A seeded shape on which the _ws_ entry points run the dynamic
    schedule on n CUs: at least one full round of whole 256-query tiles, a
    last round at least half full, at least 256 key stages per tile."""
    r = np.random.default_rng(9000 + i)
    D = int(r.choice([64, 128]))
    P = int(r.choice([2, 4, 8]))
    B = int(r.choice([1, 2]))
    S = P * int(r.integers(16384 // P + 1, 40000 // P + 1))
    tiles = -(-S // 256)
    H = next(h for h in range(1, 64)
             if B * h * tiles >= n + (B * h * tiles) % n and 2 * ((B * h * tiles) % n) >= n)
    entry = ENTRIES[1 + i % 3]
    scale = float(r.choice([1.0 / math.sqrt(D), -0.3]))
    return dict(B=B, H=H, S=S, D=D, P=P, keep=None, scale=scale, entry=entry, seed=9000 + i)


@pytest.mark.parametrize("i", range(6))
def test_random_dynamic_schedule_shape(i):
    """Seeded shapes that reach the dynamic schedule (last round in key
    pieces from a counter) through each _ws_ entry point: the float64 oracle
    on sampled rows, every slab element written, a second call bit-equal."""
    c = _dyn_case(i, torch.cuda.get_device_properties(0).multi_processor_count)
    print(f"[dynamic shapes] {i}: {c}", file=sys.stderr, flush=True)
    B, H, S, D, P = c["B"], c["H"], c["S"], c["D"], c["P"]
    q, k, v = wl.random_qkv(B, H, S, D, seed=c["seed"])
    qd, kd, vd = (t.to("cuda:0") for t in (q, k, v))
    got = _run(c, qd, kd, vd, None)
    again = _run(c, qd, kd, vd, None)
    assert torch.equal(got.view(torch.int16), again.view(torch.int16)), "second call differs"
    rows = sample_rows(S, P, seed=c["seed"], n_random=4)
    vv = np.concatenate([v.double().numpy(), np.abs(v.double().numpy())], axis=-1)
    both = oracle.attention(q.double().numpy(), k.double().numpy(), vv, c["scale"], None,
                            rows=rows)
    ref, absv = both[..., :D], both[..., D:]
    g = slab_rows(got, rows, S, P)
    assert_within_bound(g, ref, absv, f"dynamic case {i}")
    if c["scale"] == 1.0 / math.sqrt(D):
        assert_close(g, ref, f"dynamic case {i}")
