"""GPU parity: the HIP path through the C ABI against the float64 oracle.

Gate (attention values, bf16 outputs vs the unrounded float64 reference):
max-abs <= 1e-2 and mean-abs <= 1e-3 over every compared element.  The
re-layout is checked bit-exactly with integer-tagged inputs, with canary-filled
output buffers inside guard bands (every slab element written, nothing
outside).  Full-size workloads are compared on sampled rows (tile edges, slab
edges, the ragged tail, random rows) that the oracle computes row by row.
"""
import math
import sys

import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from gpu_util import (assert_close, assert_within_bound, f64, mask_to_dev, run_plain, run_slabs, sample_rows,
                      slab_rows, to_dev)

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def _upload(inp):
    return to_dev(inp.q), to_dev(inp.k), to_dev(inp.v), mask_to_dev(inp.mask)


# ------------------------------------------------------------ full oracle
@pytest.mark.parametrize("name", ["tiny", "image"])
def test_workload_full_parity(name):
    w = wl.WORKLOADS[name]
    say(f"[parity] {name} B={w.B} H={w.H} S={w.S} D={w.D} P={w.P}")
    inp = wl.make(name)
    q, k, v, m = _upload(inp)
    slabs = run_slabs(q, k, v, w.P, w.scale, m)
    plain = run_plain(q, k, v, w.scale, m)
    ref = oracle.attention(inp.f64("q"), inp.f64("k"), inp.f64("v"), w.scale, inp.mask)
    e = assert_close(f64(slabs), oracle.relayout_index(ref, w.P), name)
    assert_close(f64(plain), ref, name + " plain")
    absv = oracle.attention(inp.f64("q"), inp.f64("k"), np.abs(inp.f64("v")), w.scale, inp.mask)
    assert_within_bound(f64(plain), ref, absv, name)
    # Same arithmetic, two store layouts: identical bits.
    assert torch.equal(slabs.view(torch.int16).cpu(),
                       torch.from_numpy(oracle.relayout_split(
                           plain.view(torch.int16).cpu().numpy(), w.P)))
    say(f"[parity] {name}: {e}")


@pytest.mark.parametrize("name", ["video", "long", "sparse", "video64"])
def test_workload_sampled_parity(name):
    w = wl.WORKLOADS[name]
    say(f"[parity] {name} sampled rows B={w.B} H={w.H} S={w.S} D={w.D} P={w.P}")
    inp = wl.make(name)
    q, k, v, m = _upload(inp)
    slabs = run_slabs(q, k, v, w.P, w.scale, m)
    rows = sample_rows(w.S, w.P, seed=w.seed)
    ref = oracle.attention(inp.f64("q"), inp.f64("k"), inp.f64("v"), w.scale, inp.mask,
                           rows=rows)
    got = slab_rows(slabs, rows, w.S, w.P)
    e = assert_close(got, ref, name)
    absv = oracle.attention(inp.f64("q"), inp.f64("k"), np.abs(inp.f64("v")), w.scale, inp.mask,
                            rows=rows)
    assert_within_bound(got, ref, absv, name)
    say(f"[parity] {name}: {len(rows)} rows x {w.H} heads: {e}")
    # The plain twin equals the slabs bit for bit at full size.
    plain = run_plain(q, k, v, w.scale, m)
    re = torch.from_numpy(oracle.relayout_split(plain.view(torch.int16).cpu().numpy(), w.P))
    assert torch.equal(slabs.view(torch.int16).cpu(), re)


# ------------------------------------------------------ bit-exact re-layout
@pytest.mark.parametrize("name", ["tiny", "image", "video", "long", "sparse", "video64"])
def test_tags_bit_exact(name):
    w = wl.WORKLOADS[name]
    say(f"[tags] {name} S={w.S} H={w.H} D={w.D} P={w.P}")
    t = wl.tag_inputs(w.B, w.H, w.S, w.D)
    mask = None
    if w.keep_prob is not None:
        mask = wl.pack_mask(wl.tile_mask_bool(w.H, w.S, w.keep_prob, w.seed))
    q, k, v = to_dev(t.q), to_dev(t.k), to_dev(t.v)
    slabs = run_slabs(q, k, v, w.P, w.scale, mask_to_dev(mask))
    want = oracle.relayout_index(t.v.view(torch.int16).numpy(), w.P)
    got = slabs.view(torch.int16).cpu().numpy()
    bad = np.argwhere(got != want)
    assert bad.size == 0, f"{len(bad)} mismatches, first at {bad[:5].tolist()}"


@pytest.mark.parametrize("B,H,S,D,P", [
    (2, 3, 256, 64, 2), (2, 2, 1000, 128, 8), (1, 4, 4095 * 2, 128, 2), (3, 1, 384, 128, 3),
    (1, 2, 129, 64, 1), (1, 1, 1, 128, 1), (2, 2, 17, 64, 17),
])
def test_tags_shapes(B, H, S, D, P):
    t = wl.tag_inputs(B, H, S, D)
    q, k, v = to_dev(t.q), to_dev(t.k), to_dev(t.v)
    slabs = run_slabs(q, k, v, P, 1.0 / math.sqrt(D))
    want = oracle.relayout_index(t.v.view(torch.int16).numpy(), P)
    assert np.array_equal(slabs.view(torch.int16).cpu().numpy(), want)


# ---------------------------------------------------------------- edges
EDGE_SHAPES = [
    (1, 1, 1, 64, 1), (1, 1, 2, 128, 2), (1, 2, 16, 64, 4), (1, 1, 63, 128, 1),
    (1, 1, 64, 128, 1), (1, 1, 65, 64, 5), (1, 2, 127, 128, 1), (1, 1, 128, 64, 8),
    (1, 2, 129, 128, 3), (2, 2, 200, 64, 8), (2, 1, 255, 128, 5), (1, 3, 257, 128, 1),
    (2, 3, 640, 128, 8), (1, 2, 1000, 64, 8),
]


@pytest.mark.parametrize("B,H,S,D,P", EDGE_SHAPES)
def test_edge_shapes(B, H, S, D, P):
    q, k, v = wl.random_qkv(B, H, S, D, seed=S * 7 + D)
    scale = 1.0 / math.sqrt(D)
    slabs = run_slabs(to_dev(q), to_dev(k), to_dev(v), P, scale)
    qd, kd, vd = q.double().numpy(), k.double().numpy(), v.double().numpy()
    ref = oracle.attention(qd, kd, vd, scale)
    absv = oracle.attention(qd, kd, np.abs(vd), scale)
    assert_within_bound(f64(slabs), oracle.relayout_split(ref, P), oracle.relayout_split(absv, P),
                        f"{(B, H, S, D, P)}")


def _cus():
    return torch.cuda.get_device_properties(0).multi_processor_count


# Dense launches run whole 256-query tiles, one workgroup per CU per round; a
# last round that would fill at most half the CUs runs as half-tiles whose
# keys are split between the two wave groups of a workgroup.  Shapes for each
# schedule, from the CU count: (B, H, S, D, P).
SCHEDULES = {
    "half-tiles only, even stages": lambda n: (1, 3, 600, 128, 4),
    "half-tiles only, odd stages": lambda n: (2, 2, 650, 64, 2),
    "half-tiles only, two stages": lambda n: (1, 2, 100, 128, 2),
    "whole tiles, full rounds": lambda n: (1, n, 256, 128, 2),
    "whole tiles, partial round": lambda n: (1, (3 * n) // 4, 256, 64, 4),
    "whole tiles + half-tiles": lambda n: (1, n + 5, 300, 128, 3),
    "whole tiles + half-tiles, odd stages": lambda n: (2, n // 2 + 3, 520, 64, 8),
}


@pytest.mark.parametrize("sched", sorted(SCHEDULES))
def test_dense_schedules(sched):
    B, H, S, D, P = SCHEDULES[sched](_cus())
    say(f"[sched] {sched}: B={B} H={H} S={S} D={D} P={P}")
    q, k, v = wl.random_qkv(B, H, S, D, seed=H * 31 + S)
    scale = 1.0 / math.sqrt(D)
    slabs = run_slabs(to_dev(q), to_dev(k), to_dev(v), P, scale)
    qd, kd, vd = q.double().numpy(), k.double().numpy(), v.double().numpy()
    ref = oracle.relayout_split(oracle.attention(qd, kd, vd, scale), P)
    absv = oracle.relayout_split(oracle.attention(qd, kd, np.abs(vd), scale), P)
    assert_close(f64(slabs), ref, sched)
    assert_within_bound(f64(slabs), ref, absv, sched)
    t = wl.tag_inputs(B, H, S, D)
    tags = run_slabs(to_dev(t.q), to_dev(t.k), to_dev(t.v), P, scale)
    assert np.array_equal(tags.view(torch.int16).cpu().numpy(),
                          oracle.relayout_index(t.v.view(torch.int16).numpy(), P))


@pytest.mark.parametrize("scale", [0.0, -0.125, 0.5, -1.0 / math.sqrt(128)])
def test_scales(scale):
    B, H, S, D, P = 1, 2, 300, 128, 3
    q, k, v = wl.random_qkv(B, H, S, D, seed=11)
    slabs = run_slabs(to_dev(q), to_dev(k), to_dev(v), P, scale)
    qd, kd, vd = q.double().numpy(), k.double().numpy(), v.double().numpy()
    ref = oracle.attention(qd, kd, vd, scale)
    absv = oracle.attention(qd, kd, np.abs(vd), scale)
    assert_within_bound(f64(slabs), oracle.relayout_split(ref, P), oracle.relayout_split(absv, P),
                        f"scale={scale}")


def test_scale_zero_is_mean_of_v():
    B, H, S, D, P = 1, 2, 333, 64, 3
    q, k, v = wl.random_qkv(B, H, S, D, seed=12)
    slabs = run_slabs(to_dev(q), to_dev(k), to_dev(v), P, 0.0)
    mean = v.double().numpy().mean(axis=2, keepdims=True)
    assert_close(f64(slabs), oracle.relayout_split(np.broadcast_to(mean, (B, H, S, D)), P))


def test_ones_v_gives_ones():
    B, H, S, D = 1, 3, 4096, 128
    q, k, _ = wl.random_qkv(B, H, S, D, seed=13, kscale=(0.5, 2.0))
    v = torch.ones((B, H, S, D), dtype=torch.bfloat16)
    out = f64(run_plain(to_dev(q), to_dev(k), to_dev(v), 1.0 / math.sqrt(D)))
    assert np.abs(out - 1.0).max() <= 2 ** -7


# ---------------------------------------------------------------- masks
def test_full_mask_equals_dense():
    """A mask that keeps every tile gives the dense result.  Masked calls run
    on 128-query tiles with the keys split between two wave groups and dense
    ones on 256-query tiles, so the two sum in different orders: both must
    meet the bound against the oracle, and the tag re-layout must be
    identical."""
    B, H, S, D, P = 1, 3, 1000, 128, 8
    qh, kh, vh = wl.random_qkv(B, H, S, D, seed=14)
    q, k, v = to_dev(qh), to_dev(kh), to_dev(vh)
    keep = np.ones((H, 8, 8), dtype=bool)
    a = run_slabs(q, k, v, P, 0.09, mask_to_dev(wl.pack_mask(keep)))
    b = run_slabs(q, k, v, P, 0.09)
    qd, kd, vd = qh.double().numpy(), kh.double().numpy(), vh.double().numpy()
    ref = oracle.relayout_split(oracle.attention(qd, kd, vd, 0.09), P)
    absv = oracle.relayout_split(oracle.attention(qd, kd, np.abs(vd), 0.09), P)
    for got, what in ((a, "full mask"), (b, "dense")):
        assert_close(f64(got), ref, what)
        assert_within_bound(f64(got), ref, absv, what)
    t = wl.tag_inputs(B, H, S, D)
    tq, tk, tv = to_dev(t.q), to_dev(t.k), to_dev(t.v)
    ta = run_slabs(tq, tk, tv, P, 1.0 / math.sqrt(D), mask_to_dev(wl.pack_mask(keep)))
    tb = run_slabs(tq, tk, tv, P, 1.0 / math.sqrt(D))
    assert torch.equal(ta.view(torch.int16), tb.view(torch.int16))


@pytest.mark.parametrize("S,p_keep,B,D,scale", [
    (1000, 0.0, 1, 128, 0.088), (1000, 0.3, 1, 128, 0.088), (32760 // 4, 0.3, 1, 128, 0.088),
    (700, 0.7, 1, 128, 0.088), (1000, 0.5, 2, 64, 0.125), (777, 0.4, 3, 128, -0.09),
    (129, 0.5, 2, 64, 0.2), (9000, 0.3, 1, 128, 0.088),
])
def test_masked_parity(S, p_keep, B, D, scale):
    H, P = 3, 4 if S % 4 == 0 else 1
    q, k, v = wl.random_qkv(B, H, S, D, seed=S + 1)
    keep = wl.tile_mask_bool(H, S, p_keep, seed=S)
    words = wl.pack_mask(keep)
    slabs = run_slabs(to_dev(q), to_dev(k), to_dev(v), P, scale, mask_to_dev(words))
    rows = None if S <= 1000 else sample_rows(S, P, seed=S)
    qd, kd, vd = q.double().numpy(), k.double().numpy(), v.double().numpy()
    ref = oracle.attention(qd, kd, vd, scale, words, rows=rows)
    absv = oracle.attention(qd, kd, np.abs(vd), scale, words, rows=rows)
    if rows is None:
        got, ref, absv = f64(slabs), oracle.relayout_split(ref, P), oracle.relayout_split(absv, P)
    else:
        got = slab_rows(slabs, rows, S, P)
    assert_close(got, ref, f"mask S={S}")
    assert_within_bound(got, ref, absv, f"mask S={S}")


def test_identical_keys_with_mask_is_mean_over_kept():
    B, H, S, D, P = 1, 2, 500, 64, 4
    q, _, v = wl.random_qkv(B, H, S, D, seed=15)
    k = q[:, :, :1].expand(B, H, S, D).contiguous()
    keep = wl.tile_mask_bool(H, S, 0.5, seed=15)
    out = f64(run_plain(to_dev(q), to_dev(k), to_dev(v), 0.125, mask_to_dev(wl.pack_mask(keep))))
    vv = v.double().numpy()
    tile = np.arange(S) // 128
    for h in range(H):
        for i in range(keep.shape[1]):
            cols = keep[h, i][tile]
            want = vv[0, h][cols].mean(axis=0)
            got = out[0, h][tile == i]
            assert np.abs(got - want).max() <= 1e-2


def test_fully_masked_rows_are_zero():
    B, H, S, D = 1, 1, 384, 128
    q, k, v = wl.random_qkv(B, H, S, D, seed=16)
    keep = np.zeros((1, 3, 3), dtype=bool)
    keep[0, 0, 0] = keep[0, 2, 1] = True      # tile row 1 keeps nothing
    words = wl.pack_mask(keep)
    out = f64(run_plain(to_dev(q), to_dev(k), to_dev(v), 0.1, mask_to_dev(words)))
    assert np.all(out[0, 0, 128:256] == 0.0)
    ref = oracle.attention(q.double().numpy(), k.double().numpy(), v.double().numpy(), 0.1, words)
    assert_close(out, ref)


def test_mask_stream_edges():
    """Masked units split a row's kept stages between two wave groups.  Edge
    rows at S = 300 (three mask tiles, the last holding 44 keys): only the
    short last tile kept, so the second group's only stage has no key at all;
    nothing kept; two tiles kept; every tile kept.  Bits for tiles past the
    row's end are ignored (the same call with them set gives the same bits)."""
    B, H, S, D, P = 1, 2, 300, 128, 3
    q, k, v = wl.random_qkv(B, H, S, D, seed=19)
    keep = np.zeros((H, 3, 3), dtype=bool)
    keep[0, 0, 2] = True                 # one short tile: K = 1
    keep[0, 2, [0, 2]] = True            # K = 2, its last stage empty
    keep[1] = True                       # head 1: every tile
    words = wl.pack_mask(keep)           # row 1 of head 0 keeps nothing
    qd, kd, vd = q.double().numpy(), k.double().numpy(), v.double().numpy()
    ref = oracle.attention(qd, kd, vd, 0.1, words)
    absv = oracle.attention(qd, kd, np.abs(vd), 0.1, words)
    qg, kg, vg = to_dev(q), to_dev(k), to_dev(v)
    out = run_plain(qg, kg, vg, 0.1, mask_to_dev(words))
    got = f64(out)
    assert np.all(got[0, 0, 128:256] == 0.0)
    assert_close(got, ref, "mask edges")
    assert_within_bound(got, ref, absv, "mask edges")
    junk = words.copy()
    junk[..., 0] |= np.uint64(0xF0F0) << np.uint64(3)   # tiles 3 and up do not exist
    out2 = run_plain(qg, kg, vg, 0.1, mask_to_dev(junk))
    assert torch.equal(out.view(torch.int16), out2.view(torch.int16))


# ------------------------------------------------------------ invariants
def test_key_shift_and_permutation_invariance():
    B, H, S, D = 1, 2, 1000, 128
    r = np.random.default_rng(17)
    # Quarter-integers: K and K + c are both exact in bf16.
    q = wl.to_bf16(r.integers(-4, 5, (B, H, S, D)) / 4.0)
    k = r.integers(-4, 5, (B, H, S, D)) / 4.0
    v = wl.to_bf16(r.standard_normal((B, H, S, D)))
    c = r.integers(-3, 4, (1, 1, 1, D)).astype(np.float64)
    scale = 0.05
    base = f64(run_plain(to_dev(q), to_dev(wl.to_bf16(k)), to_dev(v), scale))
    shifted = f64(run_plain(to_dev(q), to_dev(wl.to_bf16(k + c)), to_dev(v), scale))
    assert np.abs(base - shifted).max() <= 1e-2
    perm = torch.from_numpy(r.permutation(S))
    kp = wl.to_bf16(k)[:, :, perm].contiguous()
    vp = v[:, :, perm].contiguous()
    permuted = f64(run_plain(to_dev(q), to_dev(kp), to_dev(vp), scale))
    assert np.abs(base - permuted).max() <= 1e-2


def test_deterministic_and_stream():
    w = wl.WORKLOADS["image"]
    inp = wl.make("image")
    q, k, v, m = _upload(inp)
    a = run_slabs(q, k, v, w.P, w.scale)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        b = run_slabs(q, k, v, w.P, w.scale, stream=s)
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


@pytest.mark.parametrize("case", ["video share", "image share", "whole tiles + half-tiles",
                                  "block-sparse video share", "block mask, head dim 64"])
def test_repeated_calls_bit_identical(case):
    """Repeated calls on the same inputs return the same bits.  Waves that
    race on an LDS buffer (a refill landing while another wave still reads
    the stage) show up as run-to-run differences, so this covers the whole-
    and split-tile launches and the masked units over many calls."""
    import flashattention_output_re_amd as fa
    shapes = {"video share": (1, 5, 32760, 128, 8, None), "image share": (1, 3, 4096, 128, 8, None),
              "whole tiles + half-tiles": (1, _cus() + 5, 300, 128, 3, None),
              "block-sparse video share": (1, 5, 32760, 128, 8, 0.3),
              "block mask, head dim 64": (2, 3, 9000, 64, 4, 0.5)}
    B, H, S, D, P, keep = shapes[case]
    say(f"[repeat] {case}: B={B} H={H} S={S} D={D} P={P} keep={keep}")
    q, k, v = (to_dev(t) for t in wl.random_qkv(B, H, S, D, seed=S + H))
    mask = None if keep is None else mask_to_dev(wl.pack_mask(wl.tile_mask_bool(H, S, keep, seed=S + H)))
    scale = 1.0 / math.sqrt(D)
    first = torch.empty((P, B, S // P, H, D), dtype=torch.bfloat16, device=q.device)
    fa.attn_fwd_relayout_async(q, k, v, first, B, H, S, D, P, scale, mask)
    out = torch.empty_like(first)
    calls = 10 if S > 10000 else 30
    for i in range(calls):
        out.fill_(0)
        fa.attn_fwd_relayout_async(q, k, v, out, B, H, S, D, P, scale, mask)
        assert torch.equal(out.view(torch.int16), first.view(torch.int16)), f"{case}: call {i + 1} differs"
    torch.cuda.synchronize()


@pytest.mark.parametrize("case", ["dense, whole and split launches", "block mask"])
def test_graph_capture_replays(case):
    """A fused call allocates nothing and issues only kernel launches, so a
    serving loop can record it in a HIP graph.  Each replay, with eager work
    on the stream between replays, gives the eager result bit for bit."""
    import flashattention_output_re_amd as fa
    if case == "block mask":
        B, H, S, D, P = 1, 3, 1000, 128, 4
        keep = wl.tile_mask_bool(H, S, 0.4, seed=21)
        mask = mask_to_dev(wl.pack_mask(keep))
    else:
        B, H, S, D, P = 1, _cus() + 5, 300, 128, 3
        mask = None
    say(f"[graph] {case}: B={B} H={H} S={S} D={D} P={P}")
    q, k, v = (to_dev(t) for t in wl.random_qkv(B, H, S, D, seed=22))
    scale = 1.0 / math.sqrt(D)
    eager = torch.empty((P, B, S // P, H, D), dtype=torch.bfloat16, device=q.device)
    fa.attn_fwd_relayout_async(q, k, v, eager, B, H, S, D, P, scale, mask)
    out = torch.zeros_like(eager)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fa.attn_fwd_relayout_async(q, k, v, out, B, H, S, D, P, scale, mask)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        fa.attn_fwd_relayout_async(q, k, v, out, B, H, S, D, P, scale, mask)
    for i in range(4):
        out.fill_(0)
        busy = (q.float() * 2.0).sum()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.isfinite(busy)
        assert torch.equal(out.view(torch.int16), eager.view(torch.int16)), f"{case}: replay {i}"


def test_output_past_2_31_elements():
    """Slab element offsets beyond 2^31 (64-bit store addressing, 64-bit head
    offsets): 66560 heads of 256 tokens, integer-tagged so that every output
    row is its own V row bit for bit.  The head index is spread over V's dims
    3-5 (base 128, exact in bf16).  Rows sampled on both sides of the 2^31
    boundary are compared with the tag values."""
    import flashattention_output_re_amd as fa
    B, H, S, D, P = 1, 66560, 256, 128, 2
    Sp = S // P
    assert B * H * S * D > 2 ** 31
    say(f"[2^31] B={B} H={H} S={S} D={D} P={P}")
    one = wl.tag_inputs(1, 1, S, D)
    dev = torch.device("cuda:0")
    q = one.q.to(dev).expand(B, H, S, D).contiguous()
    v = one.v.to(dev).expand(B, H, S, D).contiguous()
    hh = torch.arange(H, device=dev)
    for col, val in ((3, 1 + hh % 128), (4, 1 + (hh // 128) % 128), (5, 1 + hh // 16384)):
        v[0, :, :, col] = val[:, None].to(torch.bfloat16)
    out = torch.full((P, B, Sp, H, D), -1, dtype=torch.int16, device=dev).view(torch.bfloat16)
    fa.attn_fwd_relayout_async(q, q, v, out, B, H, S, D, P, 1.0 / math.sqrt(D), None)
    torch.cuda.synchronize()
    del q, v
    base = one.v[0, 0].view(torch.int16).numpy()
    # Slab row index (p * Sp + t) * H + h; the first row past 2^31 elements and
    # its neighbours, the last row, and rows far below.
    r0 = 2 ** 31 // D
    p0, rem = divmod(r0, Sp * H)
    t0, h0 = divmod(rem, H)
    where = [(0, 0, 0), (0, Sp - 1, H - 1), (1, 0, 0), (p0, t0, h0 - 1), (p0, t0, h0),
             (p0, t0, h0 + 1), (p0, t0 + 1, 7), (P - 1, Sp - 1, H - 1)]
    past = 0
    for p, t, h in where:
        got = out[p, 0, t, h].view(torch.int16).cpu().numpy()
        want = base[p * Sp + t].copy()
        want[3:6] = torch.tensor([1 + h % 128, 1 + (h // 128) % 128, 1 + h // 16384],
                                 dtype=torch.bfloat16).view(torch.int16).numpy()
        off = ((p * Sp + t) * H + h) * D
        past += off >= 2 ** 31
        assert np.array_equal(got, want), f"p={p} t={t} h={h}: element offset {off}"
    assert past >= 4


def test_blocking_entry_points():
    import flashattention_output_re_amd as fa
    B, H, S, D, P = 1, 2, 512, 64, 4
    q, k, v = (to_dev(t) for t in wl.random_qkv(B, H, S, D, seed=18))
    a = torch.empty((P, B, S // P, H, D), dtype=torch.bfloat16, device=q.device)
    fa.attn_fwd_relayout(q, k, v, a, B, H, S, D, P, 0.125)
    b = torch.empty((B, H, S, D), dtype=torch.bfloat16, device=q.device)
    fa.attn_fwd_plain(q, k, v, b, B, H, S, D, 0.125)
    re = oracle.relayout_split(b.view(torch.int16).cpu().numpy(), P)
    assert np.array_equal(a.view(torch.int16).cpu().numpy(), re)
