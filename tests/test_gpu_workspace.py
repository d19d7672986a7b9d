"""GPU: the workspace entry points, whose dense calls spread the last, partial
round of whole tiles over every workgroup and merge the partial results in a
second launch (include/fa_relayout.h, the _ws_ forms).

Each schedule shape -- all tiles in the tail round, a whole round plus a
tail, slices on tile bounds and slices that cut tiles at unaligned stages,
D = 64 with B = 2, a ragged sequence -- is compared with the float64 oracle
(every row of one head, sampled rows otherwise) under the gate and the
element-wise bound, and with integer tags bit for bit inside canary guard
bands.  Every row of the Video share's all-tail head is compared too.  The
plain twin equals the slab form bit for bit; repeated calls, HIP-graph
replays, calls of different shapes and plans sharing one workspace, and two
calls in flight on two streams with their own workspaces are bit-identical
to the calls made alone; a workspace that is too small or misaligned is
rejected before any launch.
"""
import math
import sys

import numpy as np
import pytest
import torch

import flashattention_output_re_amd as fa
from flashattention_output_re_amd import binding
import oracle
import workloads as wl
from gpu_util import (CANARY, Guarded, assert_close, assert_within_bound, f64, mask_to_dev,
                      sample_rows, slab_rows, to_dev)

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def _cus():
    return torch.cuda.get_device_properties(0).multi_processor_count


def run_ws(q, k, v, P, scale, mask=None, workspace=None):
    B, H, S, D = q.shape
    g = Guarded((P, B, S // P, H, D))
    fa.attn_fwd_relayout_ws_async(q, k, v, g.out, B, H, S, D, P, scale, mask, workspace)
    torch.cuda.synchronize()
    g.check_guards()
    assert g.unwritten() == 0, "slab elements left unwritten"
    return g.out


def run_plain_ws(q, k, v, scale, mask=None):
    B, H, S, D = q.shape
    g = Guarded((B, H, S, D))
    fa.attn_fwd_plain_ws_async(q, k, v, g.out, B, H, S, D, scale, mask)
    torch.cuda.synchronize()
    g.check_guards()
    assert g.unwritten() == 0
    return g.out


# (B, H, S, D, P) from the CU count n (slice lengths for 256 CUs).  Calls of
# at least one full round and a last round at least half full, of tiles of at
# least 256 key stages, run the dynamic schedule (the last round's t tiles in
# min(6, 4 n / t) key pieces of falling length, handed out from a counter);
# other tail rounds are spread as whole-tile pieces when a slice holds at
# least 64 stages; shorter tails run as half tiles, cut into key pieces of at
# least 16 stages when that leaves workgroups idle.
SHAPES = {
    "all tail, slices on tile bounds": lambda n: (1, 1, 16384, 128, 2),        # L = 64
    "all tail, unaligned slices, ragged S": lambda n: (1, 1, 20000, 128, 8),   # L = 97
    "whole round + tail, unaligned": lambda n: (1, 4, 20000, 128, 4),          # L = 74
    "all tail, D=64, B=2": lambda n: (2, 1, 20000, 64, 4),                     # L = 194
    "dynamic, ragged S": lambda n: (1, 5 * n // 256, 20000, 128, 4),           # t = 139
    "dynamic, D=64, B=2": lambda n: (2, 3 * n // 256, 16400, 64, 4),           # t = 134
    "half tiles in 2 pieces (Image share)": lambda n: (1, 3, 4096, 128, 8),
    "half tiles in 4 pieces": lambda n: (1, 1, 4096, 128, 2),
    "half tiles in 2 pieces, D=64, B=2, ragged S": lambda n: (2, 1, 3000, 64, 4),
    "whole rounds + half tiles in pieces": lambda n: (1, n + 3, 2048, 128, 4),
}


@pytest.mark.parametrize("name", sorted(SHAPES))
def test_ws_against_oracle(name):
    B, H, S, D, P = SHAPES[name](_cus())
    need = binding.attn_fwd_workspace_bytes(B, H, S, D)
    say(f"[ws] {name}: B={B} H={H} S={S} D={D} P={P}, workspace {need} bytes")
    assert need > 0, "the shape should have a tail round"
    q, k, v = wl.random_qkv(B, H, S, D, seed=S + 3 * H)
    scale = 1.0 / math.sqrt(D)
    slabs = run_ws(to_dev(q), to_dev(k), to_dev(v), P, scale)
    qd, kd, vd = q.double().numpy(), k.double().numpy(), v.double().numpy()
    vv = np.concatenate([vd, np.abs(vd)], axis=-1)
    rows = None if B * H * S <= 40_000 else sample_rows(S, P, seed=S)
    both = oracle.attention(qd, kd, vv, scale, rows=rows)
    ref, absv = both[..., :D], both[..., D:]
    if rows is None:
        got = f64(slabs)
        ref, absv = oracle.relayout_split(ref, P), oracle.relayout_split(absv, P)
    else:
        got = slab_rows(slabs, rows, S, P)
    e = assert_close(got, ref, name)
    assert_within_bound(got, ref, absv, name)
    say(f"[ws] {name}: {e}")
    plain = run_plain_ws(to_dev(q), to_dev(k), to_dev(v), scale)
    re = torch.from_numpy(oracle.relayout_split(plain.view(torch.int16).cpu().numpy(), P))
    assert torch.equal(slabs.view(torch.int16).cpu(), re), "plain twin differs from the slabs"
    t = wl.tag_inputs(B, H, S, D)
    tags = run_ws(to_dev(t.q), to_dev(t.k), to_dev(t.v), P, scale)
    assert np.array_equal(tags.view(torch.int16).cpu().numpy(),
                          oracle.relayout_index(t.v.view(torch.int16).numpy(), P))


@pytest.mark.parametrize("name", ["video", "long"])
def test_ws_full_size_sampled(name):
    w = wl.WORKLOADS[name]
    inp = wl.make(name)
    need = binding.attn_fwd_workspace_bytes(w.B, w.H, w.S, w.D)
    say(f"[ws] {name}: workspace {need / 2**20:.1f} MiB")
    assert need > 0
    q, k, v = to_dev(inp.q), to_dev(inp.k), to_dev(inp.v)
    slabs = run_ws(q, k, v, w.P, w.scale)
    rows = sample_rows(w.S, w.P, seed=w.seed)
    vv = np.concatenate([inp.f64("v"), np.abs(inp.f64("v"))], axis=-1)
    both = oracle.attention(inp.f64("q"), inp.f64("k"), vv, w.scale, rows=rows)
    ref, absv = both[..., :w.D], both[..., w.D:]
    got = slab_rows(slabs, rows, w.S, w.P)
    e = assert_close(got, ref, name)
    assert_within_bound(got, ref, absv, name)
    say(f"[ws] {name}: {len(rows)} rows x {w.H} heads: {e}")
    t = wl.tag_inputs(w.B, w.H, w.S, w.D)
    tags = run_ws(to_dev(t.q), to_dev(t.k), to_dev(t.v), w.P, w.scale)
    assert np.array_equal(tags.view(torch.int16).cpu().numpy(),
                          oracle.relayout_index(t.v.view(torch.int16).numpy(), w.P))


def test_ws_every_row_of_a_tail_tile():
    """Every row of the Video share's last head, whose 128 tiles all run as
    key pieces (spread over the workgroups and merged), against the
    oracle."""
    w = wl.WORKLOADS["video"]
    inp = wl.make("video")
    q, k, v = to_dev(inp.q), to_dev(inp.k), to_dev(inp.v)
    a = run_ws(q, k, v, w.P, w.scale)
    got = a.permute(1, 3, 0, 2, 4).reshape(w.B, w.H, w.S, w.D)
    h = w.H - 1          # tiles of the last head are all in the tail round
    vv = np.concatenate([inp.f64("v")[:, h:h + 1], np.abs(inp.f64("v")[:, h:h + 1])], axis=-1)
    both = oracle.attention(inp.f64("q")[:, h:h + 1], inp.f64("k")[:, h:h + 1], vv, w.scale,
                            row_block=512)
    g = got[:, h:h + 1].to(torch.float64).cpu().numpy()
    assert_close(g, both[..., :w.D], "video tail head")
    assert_within_bound(g, both[..., :w.D], both[..., w.D:], "video tail head")


def test_ws_repeated_calls_and_masked_calls():
    B, H, S, D, P = 1, 5, 20000, 128, 4
    q, k, v = (to_dev(t) for t in wl.random_qkv(B, H, S, D, seed=5))
    ws = torch.empty(binding.attn_fwd_workspace_bytes(B, H, S, D), dtype=torch.uint8,
                     device=q.device)
    first = run_ws(q, k, v, P, 0.09, workspace=ws)
    for i in range(8):
        again = run_ws(q, k, v, P, 0.09, workspace=ws)
        assert torch.equal(again.view(torch.int16), first.view(torch.int16)), f"call {i}"
    # Masked calls need no workspace and equal the call without one.
    keep = wl.tile_mask_bool(H, S, 0.5, seed=5)
    m = mask_to_dev(wl.pack_mask(keep))
    assert binding.attn_fwd_workspace_bytes(B, H, S, D) > 0
    out = torch.empty((P, B, S // P, H, D), dtype=torch.bfloat16, device=q.device)
    fa.attn_fwd_relayout_ws_async(q, k, v, out, B, H, S, D, P, 0.09, m,
                                  workspace=torch.empty(16, dtype=torch.uint8, device=q.device))
    ref = torch.empty_like(out)
    fa.attn_fwd_relayout_async(q, k, v, ref, B, H, S, D, P, 0.09, m)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), ref.view(torch.int16))


def test_ws_rejects_small_or_misaligned_workspace():
    B, H, S, D, P = 1, 1, 16384, 128, 2
    q, k, v = (to_dev(t) for t in wl.random_qkv(B, H, S, D, seed=6))
    need = binding.attn_fwd_workspace_bytes(B, H, S, D)
    lib = binding.load_library()
    out = torch.full((P, B, S // P, H, D), CANARY, dtype=torch.int16, device=q.device)
    ws = torch.empty(need + 64, dtype=torch.uint8, device=q.device)
    args = [q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), B, H, S, D, P, 0.1, None]
    s = torch.cuda.current_stream().cuda_stream
    assert lib.attn_fwd_relayout_ws_async(*args, ws.data_ptr(), need - 1, s) == -5
    assert lib.attn_fwd_relayout_ws_async(*args, ws.data_ptr() + 8, need, s) == -4
    assert lib.attn_fwd_relayout_ws_async(*args, None, need, s) == -1
    torch.cuda.synchronize()
    assert bool((out == CANARY).all()), "a rejected call wrote its output"
    assert lib.attn_fwd_relayout_ws_async(*args, ws.data_ptr(), need, s) == 0
    torch.cuda.synchronize()
    # Sizes that fill whole rounds need no workspace and run as without one;
    # the Image share's half tiles, cut into pieces, need one.
    n = _cus()
    assert binding.attn_fwd_workspace_bytes(1, n, 256, 128) == 0
    assert binding.attn_fwd_workspace_bytes(1, 3, 4096, 128) > 0
    a = torch.empty((8, 1, 256, n, 128), dtype=torch.bfloat16, device=q.device)
    b = torch.empty_like(a)
    qi, ki, vi = (to_dev(t) for t in wl.random_qkv(1, n, 2048, 128, seed=8))
    fa.attn_fwd_relayout_ws_async(qi, ki, vi, a, 1, n, 2048, 128, 8, 0.1, None,
                                  torch.empty(16, dtype=torch.uint8, device=q.device))
    fa.attn_fwd_relayout_async(qi, ki, vi, b, 1, n, 2048, 128, 8, 0.1, None)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


@pytest.mark.parametrize("shape", [(1, 1, 16384, 128, 2), (1, 5, 20000, 128, 4)],
                         ids=["spread tail", "dynamic"])
def test_ws_graph_capture_replays(shape):
    """A _ws_ call (two launches; the dynamic schedule's counter reset makes
    three) recorded in a HIP graph with a preallocated workspace replays
    bit-identically to the eager call, with eager work between replays."""
    B, H, S, D, P = shape
    q, k, v = (to_dev(t) for t in wl.random_qkv(B, H, S, D, seed=7))
    ws = torch.empty(binding.attn_fwd_workspace_bytes(B, H, S, D), dtype=torch.uint8,
                     device=q.device)
    eager = torch.empty((P, B, S // P, H, D), dtype=torch.bfloat16, device=q.device)
    fa.attn_fwd_relayout_ws_async(q, k, v, eager, B, H, S, D, P, 0.1, None, ws)
    out = torch.zeros_like(eager)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fa.attn_fwd_relayout_ws_async(q, k, v, out, B, H, S, D, P, 0.1, None, ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        fa.attn_fwd_relayout_ws_async(q, k, v, out, B, H, S, D, P, 0.1, None, ws)
    for i in range(4):
        out.fill_(0)
        busy = (q.float() * 2.0).sum()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.isfinite(busy)
        assert torch.equal(out.view(torch.int16), eager.view(torch.int16)), f"replay {i}"


def test_ws_shared_between_shapes_and_plans():
    """One workspace serves calls of different shapes and launch plans in
    turn -- the dynamic schedule (its counter after the partial slots), the
    spread last round and split half tiles in pieces -- and each call equals
    the same call on a fresh workspace bit for bit: nothing a call leaves in
    the workspace reaches the next."""
    shapes = [(1, 5, 20000, 128, 4), (1, 1, 16384, 128, 2), (1, 3, 4096, 128, 8),
              (2, 3, 16400, 64, 4)]
    need = max(binding.attn_fwd_workspace_bytes(B, H, S, D) for B, H, S, D, _ in shapes)
    shared = torch.empty(need, dtype=torch.uint8, device="cuda:0")
    cases = []
    for i, (B, H, S, D, P) in enumerate(shapes):
        q, k, v = (to_dev(t) for t in wl.random_qkv(B, H, S, D, seed=300 + i))
        fresh = torch.empty(binding.attn_fwd_workspace_bytes(B, H, S, D), dtype=torch.uint8,
                            device="cuda:0")
        ref = torch.empty((P, B, S // P, H, D), dtype=torch.bfloat16, device="cuda:0")
        fa.attn_fwd_relayout_ws_async(q, k, v, ref, B, H, S, D, P, 0.1, None, fresh)
        cases.append((q, k, v, ref, (B, H, S, D, P)))
    torch.cuda.synchronize()
    for rnd in range(3):
        for q, k, v, ref, (B, H, S, D, P) in cases:
            out = torch.full_like(ref, float("nan"))
            fa.attn_fwd_relayout_ws_async(q, k, v, out, B, H, S, D, P, 0.1, None, shared)
            torch.cuda.synchronize()
            assert torch.equal(out.view(torch.int16), ref.view(torch.int16)), \
                f"round {rnd}, shape {(B, H, S, D, P)}"


def test_ws_concurrent_calls_on_two_streams():
    """Two dynamic-schedule calls in flight at once on two streams, each with
    its own workspace (its own counter), give the results of the same calls
    made one at a time."""
    B, H, S, D, P = 1, 5, 20000, 128, 4
    ins = [tuple(to_dev(t) for t in wl.random_qkv(B, H, S, D, seed=400 + i)) for i in range(2)]
    need = binding.attn_fwd_workspace_bytes(B, H, S, D)
    wss = [torch.empty(need, dtype=torch.uint8, device="cuda:0") for _ in range(2)]
    refs = []
    for (q, k, v), ws in zip(ins, wss):
        r = torch.empty((P, B, S // P, H, D), dtype=torch.bfloat16, device="cuda:0")
        fa.attn_fwd_relayout_ws_async(q, k, v, r, B, H, S, D, P, 0.1, None, ws)
        refs.append(r)
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream() for _ in range(2)]
    outs = [torch.full_like(refs[0], float("nan")) for _ in range(2)]
    for rep in range(3):
        for (q, k, v), ws, o, st in zip(ins, wss, outs, streams):
            st.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(st):
                fa.attn_fwd_relayout_ws_async(q, k, v, o, B, H, S, D, P, 0.1, None, ws)
        torch.cuda.synchronize()
        for o, r in zip(outs, refs):
            assert torch.equal(o.view(torch.int16), r.view(torch.int16)), f"repeat {rep}"
