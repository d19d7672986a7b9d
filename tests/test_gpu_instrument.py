"""GPU: the timestamped instances of the fused kernel (include/fa_instrument.h).

In every form of the tile boundary (piggybacked, completion-coupled, stores
then prologue) the output equals the product kernel's bit for bit, every
(unit, wave) record is written once, and its stamps are in program order:
wait returned <= Q-loop started <= last stage done <= last store issued
(<= stores complete, coupled form only).
"""
import math
import sys

import numpy as np
import pytest
import torch

import flashattention_output_re_amd as fa
from flashattention_output_re_amd import binding, tile_stamps
import workloads as wl
from gpu_util import mask_to_dev, to_dev

pytestmark = pytest.mark.gpu


def _cus():
    return torch.cuda.get_device_properties(0).multi_processor_count


CASES = {
    "dense, whole and split launches": lambda n: (1, n + 5, 300, 128, 3, None),
    "dense, several rounds": lambda n: (1, 2 * n + 3, 700, 128, 4, None),
    "block mask": lambda n: (1, 3, 1000, 128, 4, 0.4),
    "block mask, several units per workgroup": lambda n: (1, n // 8 + 2, 2048, 128, 4, 0.5),
}


@pytest.mark.parametrize("case", sorted(CASES))
@pytest.mark.parametrize("boundary", [0, 1, 2])
def test_instrumented_output_and_records(case, boundary):
    B, H, S, D, P, keep = CASES[case](_cus())
    print(f"[instr] {case} boundary={boundary}: B={B} H={H} S={S} D={D} P={P} keep={keep}",
          file=sys.stderr, flush=True)
    q, k, v = (to_dev(t) for t in wl.random_qkv(B, H, S, D, seed=S + H))
    mask = None if keep is None else mask_to_dev(wl.pack_mask(wl.tile_mask_bool(H, S, keep, seed=S)))
    scale = 1.0 / math.sqrt(D)
    ref = torch.empty((P, B, S // P, H, D), dtype=torch.bfloat16, device=q.device)
    fa.attn_fwd_relayout_async(q, k, v, ref, B, H, S, D, P, scale, mask)
    out = torch.full_like(ref, float("nan"))
    words = binding.attn_instrumented_stamp_words(B, H, S)
    stamps = torch.zeros(words, dtype=torch.int32, device=q.device)
    units = binding.attn_fwd_relayout_instrumented_async(q, k, v, out, B, H, S, D, P, scale, mask,
                                                         boundary, stamps)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), ref.view(torch.int16))
    recs = tile_stamps.records(stamps.cpu().numpy().view(np.uint32), units)
    assert len(recs) == (1 if units[1] == 0 else 2)
    if keep is None and case.startswith("dense, whole and split"):
        assert units[1] > 0, "expected a split-key second launch"
    m32 = 1 << 32
    for r in recs:
        n = r.shape[0]
        assert np.array_equal(r[:, :, 5], np.broadcast_to(np.arange(n)[:, None], (n, 8)))
        assert np.all(r[:, :, 6] == r[:, :1, 6]), "one workgroup per unit"
        d = lambda a, b: (r[:, :, b].astype(np.int64) - r[:, :, a].astype(np.int64)) % m32
        for a, b in ((0, 1), (1, 2), (2, 3)):
            assert np.all(d(a, b) < (1 << 30)), f"stamps {a} -> {b} out of order"
        if boundary == 1:
            assert np.all(d(3, 4) < (1 << 30)) and np.all(r[:, :, 4] != 0)
        else:
            assert np.all(r[:, :, 4] == 0)
        b = tile_stamps.boundaries(r)
        assert np.all(b["resume_wait"] >= 0) and np.all(b["resume_wait"] < (1 << 30))
