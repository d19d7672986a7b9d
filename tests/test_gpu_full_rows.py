"""GPU parity at full size on every row: the fused call through the C ABI
against the float64 oracle on every output element of the Video-DiT share
and of the block-sparse Video share (5 heads x 32760 rows each), and on one
whole head of the long video share (75600 rows); then the workspace entry
point (the headline call, whose last round runs as key pieces from the
dynamic schedule) on every row of the long share's last head, which holds
that round's tiles.

Each element meets the workload gate (max-abs <= 1e-2, mean-abs <= 1e-3) and
the element-wise bound from the arithmetic (gpu_util.assert_within_bound).
The oracle computes the output for V and for |V| from one softmax by taking
[V | |V|] as the value rows.  The sampled-row tests in test_gpu_parity.py
cover the same workloads for every head of the long share.
"""
import sys
import time

import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from gpu_util import assert_close, assert_within_bound, mask_to_dev, run_slabs, to_dev

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, file=sys.stderr, flush=True)


@pytest.mark.parametrize("name,heads", [("video", None), ("sparse", None), ("long", (0,))])
def test_every_row(name, heads):
    w = wl.WORKLOADS[name]
    inp = wl.make(name)
    say(f"[full rows] {name} B={w.B} H={w.H} S={w.S} D={w.D} P={w.P}")
    slabs = run_slabs(to_dev(inp.q), to_dev(inp.k), to_dev(inp.v), w.P, w.scale,
                      mask_to_dev(inp.mask))
    # [P][B][S/P][H][D] -> [B][H][S][D]
    got_all = slabs.permute(1, 3, 0, 2, 4).reshape(w.B, w.H, w.S, w.D)
    q, k, v = inp.f64("q"), inp.f64("k"), inp.f64("v")
    for h in (range(w.H) if heads is None else heads):
        t0 = time.perf_counter()
        mask = None if inp.mask is None else inp.mask[h:h + 1]
        vv = np.concatenate([v[:, h:h + 1], np.abs(v[:, h:h + 1])], axis=-1)
        both = oracle.attention(q[:, h:h + 1], k[:, h:h + 1], vv, w.scale, mask, row_block=512)
        ref, absv = both[..., :w.D], both[..., w.D:]
        got = got_all[:, h:h + 1].to(torch.float64).cpu().numpy()
        e = assert_close(got, ref, f"{name} head {h}")
        assert_within_bound(got, ref, absv, f"{name} head {h}")
        say(f"[full rows] {name} head {h}: {w.S} rows, max_abs {e['max_abs']:.3e} "
            f"mean_abs {e['mean_abs']:.3e} ({time.perf_counter() - t0:.1f} s)")


def test_every_row_of_the_long_share_last_head_workspace_form():
    """The workspace entry point on the long share (the headline call): its
    last round -- 200 tiles, all of the last head's last 200 query tiles --
    runs as key pieces handed out from a counter and merged by a second
    launch; every row of that head against the oracle."""
    import flashattention_output_re_amd as fa
    w = wl.WORKLOADS["long"]
    inp = wl.make("long")
    h = w.H - 1
    say(f"[full rows] long, workspace form, head {h}")
    q, k, v = to_dev(inp.q), to_dev(inp.k), to_dev(inp.v)
    out = torch.empty((w.P, w.B, w.S // w.P, w.H, w.D), dtype=torch.bfloat16, device=q.device)
    fa.attn_fwd_relayout_ws_async(q, k, v, out, w.B, w.H, w.S, w.D, w.P, w.scale)
    torch.cuda.synchronize()
    got = out.permute(1, 3, 0, 2, 4).reshape(w.B, w.H, w.S, w.D)[:, h:h + 1]
    got = got.to(torch.float64).cpu().numpy()
    t0 = time.perf_counter()
    qd, kd, vd = inp.f64("q"), inp.f64("k"), inp.f64("v")
    vv = np.concatenate([vd[:, h:h + 1], np.abs(vd[:, h:h + 1])], axis=-1)
    both = oracle.attention(qd[:, h:h + 1], kd[:, h:h + 1], vv, w.scale, row_block=512)
    ref, absv = both[..., :w.D], both[..., w.D:]
    e = assert_close(got, ref, f"long head {h}, workspace form")
    assert_within_bound(got, ref, absv, f"long head {h}, workspace form")
    say(f"[full rows] long head {h} (workspace form): {w.S} rows, max_abs {e['max_abs']:.3e} "
        f"mean_abs {e['mean_abs']:.3e} ({time.perf_counter() - t0:.1f} s)")
