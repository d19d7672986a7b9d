"""GPU: the whole Ulysses step on one GPU (attn_fwd_slab_to_slab), with Q, K
and V read straight from sequence-sharded slabs [P][B][S/P][H][D].

The slab inputs are built by the oracle's re-layout of [B][H][S][D] tensors
(the pre-attention exchange is its inverse), so the expected output is the
oracle's attention on the unsharded tensors, re-laid into slabs.  Beyond the
oracle bound, the result must equal attn_fwd_relayout on the unsharded
tensors bit for bit: only the load addressing differs, not the arithmetic.
"""
import math
import sys

import numpy as np
import pytest
import torch

import flashattention_output_re_amd as fa
import oracle
import workloads as wl
from gpu_util import (Guarded, assert_close, assert_within_bound, f64, mask_to_dev, run_slabs,
                      to_dev)

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def _cus():
    return torch.cuda.get_device_properties(0).multi_processor_count


def to_slabs(t: torch.Tensor, P: int) -> torch.Tensor:
    """[B][H][S][D] bf16 (host) -> [P][B][S/P][H][D] on the device, by the
    oracle's closed-form re-layout (on the 16-bit patterns, so exact)."""
    raw = oracle.relayout_index(t.view(torch.int16).numpy(), P)
    return torch.from_numpy(np.ascontiguousarray(raw)).view(torch.bfloat16).to("cuda:0")


def run_s2s(qs, ks, vs, B, H, S, D, P, scale, mask=None):
    g = Guarded((P, B, S // P, H, D))
    fa.attn_fwd_slab_to_slab_async(qs, ks, vs, g.out, B, H, S, D, P, scale, mask)
    torch.cuda.synchronize()
    g.check_guards()
    assert g.unwritten() == 0, "slab elements left unwritten"
    return g.out


CASES = {
    # name: (B, H, S, D, P, mask keep probability or None)
    "whole + split tiles": lambda n: (1, n + 5, 300, 128, 3, None),
    "stages cross slab ends, B = 1": lambda n: (1, 3, 8190, 128, 2, None),
    "B = 2, slab crossings": lambda n: (2, 3, 1000, 128, 4, None),
    "B = 3, ragged S, D = 64": lambda n: (3, 2, 777, 64, 7, None),
    "split tiles only, D = 64": lambda n: (2, 2, 650, 64, 2, None),
    "block mask, B = 2": lambda n: (2, 3, 1000, 128, 4, 0.4),
    "block mask, ragged, D = 64": lambda n: (1, 4, 777, 64, 7, 0.3),
}


@pytest.mark.parametrize("case", sorted(CASES))
def test_slab_inputs_equal_unsharded_inputs(case):
    B, H, S, D, P, keep_p = CASES[case](_cus())
    say(f"[slab-in] {case}: B={B} H={H} S={S} D={D} P={P} mask={keep_p}")
    q, k, v = wl.random_qkv(B, H, S, D, seed=S + 7 * H)
    mask = None
    if keep_p is not None:
        mask = mask_to_dev(wl.pack_mask(wl.tile_mask_bool(H, S, keep_p, seed=S)))
    scale = 1.0 / math.sqrt(D)
    got = run_s2s(to_slabs(q, P), to_slabs(k, P), to_slabs(v, P), B, H, S, D, P, scale, mask)
    want = run_slabs(to_dev(q), to_dev(k), to_dev(v), P, scale, mask)
    assert torch.equal(got.view(torch.int16), want.view(torch.int16))


@pytest.mark.parametrize("B,H,S,D,P,keep_p", [(2, 3, 1000, 128, 4, None), (1, 3, 777, 64, 7, 0.5)])
def test_slab_inputs_against_oracle(B, H, S, D, P, keep_p):
    say(f"[slab-in oracle] B={B} H={H} S={S} D={D} P={P} mask={keep_p}")
    q, k, v = wl.random_qkv(B, H, S, D, seed=S + 3)
    words = None if keep_p is None else wl.pack_mask(wl.tile_mask_bool(H, S, keep_p, seed=S + 1))
    scale = 0.11
    got = f64(run_s2s(to_slabs(q, P), to_slabs(k, P), to_slabs(v, P), B, H, S, D, P, scale,
                      mask_to_dev(words)))
    qd, kd, vd = q.double().numpy(), k.double().numpy(), v.double().numpy()
    ref = oracle.relayout_split(oracle.attention(qd, kd, vd, scale, words), P)
    absv = oracle.relayout_split(oracle.attention(qd, kd, np.abs(vd), scale, words), P)
    assert_close(got, ref, "slab inputs")
    assert_within_bound(got, ref, absv, "slab inputs")


@pytest.mark.parametrize("B,H,S,D,P", [(1, 3, 4096, 128, 8), (2, 2, 1000, 64, 4)])
def test_slab_inputs_integer_tags(B, H, S, D, P):
    """Integer tags: every output row is its own V row, so the output slabs
    are exactly the input V slabs."""
    say(f"[slab-in tags] B={B} H={H} S={S} D={D} P={P}")
    t = wl.tag_inputs(B, H, S, D)
    vs = to_slabs(t.v, P)
    got = run_s2s(to_slabs(t.q, P), to_slabs(t.k, P), vs, B, H, S, D, P, 1.0 / math.sqrt(D))
    assert torch.equal(got.view(torch.int16), vs.view(torch.int16))


def test_slab_inputs_blocking_entry_point():
    B, H, S, D, P = 1, 2, 512, 128, 4
    q, k, v = wl.random_qkv(B, H, S, D, seed=31)
    qs, ks, vs = to_slabs(q, P), to_slabs(k, P), to_slabs(v, P)
    a = torch.empty((P, B, S // P, H, D), dtype=torch.bfloat16, device="cuda:0")
    fa.attn_fwd_slab_to_slab(qs, ks, vs, a, B, H, S, D, P, 0.125)
    b = run_slabs(to_dev(q), to_dev(k), to_dev(v), P, 0.125)
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


WS_CASES = {
    # name: (B, H, S, D, P, mask keep probability or None); the last round
    # in key pieces from the dynamic schedule's counter, spread (lead and
    # helper pieces), cut into half-tile pieces, or masked (256 CUs).
    "last round spread, slices on tile bounds": (1, 1, 16384, 128, 2, None),
    "whole round + spread last round": (1, 4, 20000, 128, 4, None),
    "dynamic schedule": (1, 5, 20000, 128, 4, None),
    "dynamic schedule, D = 64, B = 2": (2, 3, 16400, 64, 4, None),
    "half tiles in pieces (Image share)": (1, 3, 4096, 128, 8, None),
    "half tiles in pieces, D = 64, B = 2": (2, 1, 3000, 64, 4, None),
    "block mask, B = 2": (2, 3, 1000, 128, 4, 0.4),
}


@pytest.mark.parametrize("case", sorted(WS_CASES))
def test_slab_inputs_workspace_form_equals_unsharded(case):
    """attn_fwd_slab_to_slab_ws_async equals attn_fwd_relayout_ws_async on
    the unsharded tensors bit for bit (same schedule and merge, only the
    load addressing differs), and meets the oracle on sampled rows."""
    from gpu_util import sample_rows, slab_rows
    B, H, S, D, P, keep_p = WS_CASES[case]
    say(f"[slab-in ws] {case}: B={B} H={H} S={S} D={D} P={P} mask={keep_p}")
    q, k, v = wl.random_qkv(B, H, S, D, seed=S + 11 * H)
    words = None if keep_p is None else wl.pack_mask(wl.tile_mask_bool(H, S, keep_p, seed=S))
    mask = None if words is None else mask_to_dev(words)
    scale = 1.0 / math.sqrt(D)
    g = Guarded((P, B, S // P, H, D))
    fa.attn_fwd_slab_to_slab_ws_async(to_slabs(q, P), to_slabs(k, P), to_slabs(v, P), g.out,
                                      B, H, S, D, P, scale, mask)
    want = torch.empty((P, B, S // P, H, D), dtype=torch.bfloat16, device="cuda:0")
    fa.attn_fwd_relayout_ws_async(to_dev(q), to_dev(k), to_dev(v), want, B, H, S, D, P, scale,
                                  mask)
    torch.cuda.synchronize()
    g.check_guards()
    assert g.unwritten() == 0
    assert torch.equal(g.out.view(torch.int16), want.view(torch.int16))
    rows = sample_rows(S, P, seed=S, n_random=8)
    ref = oracle.attention(q.double().numpy(), k.double().numpy(), v.double().numpy(), scale,
                           words, rows=rows)
    assert_close(slab_rows(g.out, rows, S, P), ref, case)
