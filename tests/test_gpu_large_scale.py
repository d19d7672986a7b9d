"""GPU: scales at the accepted bound |scale| <= 2^16 (include/fa_relayout.h).

At such scales softmax(scale * Q K^T) is a hard arg-max (arg-min for a
negative scale): a query whose best key beats the runner-up by a margin g
weighs the runner-up by exp(-g |scale|), below 2^-900 here, so the exact
output is that key's V row.  The kernel forms scale * log2(e) * (q . k) in
fp32; the largest product stays below 2^24 for these inputs (|q . k| < 100),
so the row's common weight factor (the rounding of its running max) stays in
[1/2, 2] and the output meets the bf16 error bound against the exact V row:
|out - V| <= 1.1 * 2^-8 * 2 |V| + 1e-5 element-wise (the probability's and
the output's roundings).  Rows whose two best scores lie closer than 1e-2
(where the fp32 score rounding could pick either key) have more than one
valid answer; for them the output must be a weighted mean of the V rows of
the keys within that margin.  The float64 oracle confirms the clear rows'
reference at the same scale.
"""
import math
import sys

import numpy as np
import pytest

import oracle
import workloads as wl
from gpu_util import mask_to_dev, run_slabs, slab_rows, to_dev

pytestmark = pytest.mark.gpu

MARGIN = 1e-2


def _bound(v):
    return 1.1 * 2.0 ** -8 * 2.0 * np.abs(v) + 1e-5


@pytest.mark.parametrize("scale", [2.0 ** 12, 2.0 ** 16, -(2.0 ** 16)])
@pytest.mark.parametrize("masked", [False, True])
def test_hard_argmax_limit(scale, masked):
    B, H, S, D, P = 1, 2, 1000, 128, 4
    print(f"[large scale] scale={scale:g} masked={masked}", file=sys.stderr, flush=True)
    q, k, v = wl.random_qkv(B, H, S, D, seed=77)
    words = wl.pack_mask(wl.tile_mask_bool(H, S, 0.5, seed=78)) if masked else None
    slabs = run_slabs(to_dev(q), to_dev(k), to_dev(v), P, scale,
                      None if words is None else mask_to_dev(words))
    got = slab_rows(slabs, np.arange(S), S, P)            # [B][H][S][D] float64
    qd, kd, vd = q.double().numpy(), k.double().numpy(), v.double().numpy()
    keep = None if words is None else oracle.unpack_mask(words, S)
    clear = 0
    clear_rows = np.ones(S, dtype=bool)
    for h in range(H):
        z = qd[0, h] @ kd[0, h].T * math.copysign(1.0, scale)   # larger is better
        assert np.abs(z).max() * abs(scale) * math.log2(math.e) < 2.0 ** 24
        if keep is not None:
            allowed = keep[h][np.arange(S)[:, None] // 128, np.arange(S)[None, :] // 128]
            z = np.where(allowed, z, -np.inf)
        order = np.argsort(-z, axis=1)
        best, second = order[:, 0], order[:, 1]
        gap = z[np.arange(S), best] - z[np.arange(S), second]
        clear_rows &= gap >= MARGIN
        for s in range(S):
            if gap[s] >= MARGIN:
                clear += 1
                want = vd[0, h, best[s]]
                assert np.all(np.abs(got[0, h, s] - want) <= _bound(want)), f"head {h} row {s}"
            else:
                # A weighted mean of the near-best keys' V rows (one of them
                # when their scaled scores differ, a mix on an fp32 tie).
                vn = vd[0, h, np.nonzero(z[s] >= z[s, best[s]] - MARGIN)[0]]
                tol = _bound(np.abs(vn).max(axis=0))
                assert np.all(got[0, h, s] >= vn.min(axis=0) - tol) and \
                    np.all(got[0, h, s] <= vn.max(axis=0) + tol), f"head {h} row {s}"
    assert clear >= 0.99 * H * S
    # The oracle, at the same scale, gives V of the best key on a sample of
    # the clear rows.
    rows = np.nonzero(clear_rows)[0][::37]
    ref = oracle.attention(qd, kd, vd, scale, words, rows=rows)
    assert np.all(np.abs(got[:, :, rows] - ref) <= _bound(ref))
