"""GPU: the allocation-free entry point (attn_fwd_relayout_noalloc_async,
the library's static workspace) against the workspace entry point it is a
variant of (attn_fwd_relayout_ws_async, a workspace from the caller), through
the C ABI, on two calls in a row, the second with a smaller input: the same
kernels and schedule, so identical bits, and the output meets the oracle
gate on sampled rows.
"""
import math
import sys

import numpy as np
import pytest
import torch

from flashattention_output_re_amd import binding
import oracle
import workloads as wl
from gpu_util import Guarded, assert_close, sample_rows, slab_rows, to_dev

pytestmark = pytest.mark.gpu


def test_no_alloc_matches_workspace_entry_on_two_calls():
    for B, H, S, D, P in [(1, 5, 20000, 128, 4), (1, 1, 16384, 128, 2)]:
        print(f"[no-alloc] B={B} H={H} S={S} D={D} P={P}", file=sys.stderr, flush=True)
        assert binding.attn_fwd_workspace_bytes(B, H, S, D) > 0
        q, k, v = wl.random_qkv(B, H, S, D, seed=S + H)
        qd, kd, vd = to_dev(q), to_dev(k), to_dev(v)
        scale = 1.0 / math.sqrt(D)
        ref = torch.empty((P, B, S // P, H, D), dtype=torch.bfloat16, device=qd.device)
        binding.attn_fwd_relayout_ws_async(qd, kd, vd, ref, B, H, S, D, P, scale)
        g = Guarded((P, B, S // P, H, D))
        binding.attn_fwd_relayout_noalloc_async(qd, kd, vd, g.out, B, H, S, D, P, scale)
        torch.cuda.synchronize()
        g.check_guards()
        assert g.unwritten() == 0
        assert torch.equal(g.out.view(torch.int16), ref.view(torch.int16))
        rows = sample_rows(S, P, seed=S)
        want = oracle.attention(q.double().numpy(), k.double().numpy(), v.double().numpy(), scale,
                                rows=rows)
        assert_close(slab_rows(g.out, rows, S, P), want, f"no-alloc S={S}")


def test_no_alloc_masked_matches_workspace_entry_on_two_calls():
    """Block-masked calls: the schedule lives in the static array as well."""
    from gpu_util import mask_to_dev
    for B, H, S, D, P in [(1, 5, 20000, 128, 4), (1, 2, 3000, 128, 2)]:
        print(f"[no-alloc masked] B={B} H={H} S={S} D={D} P={P}", file=sys.stderr, flush=True)
        q, k, v = wl.random_qkv(B, H, S, D, seed=S + 3)
        qd, kd, vd = to_dev(q), to_dev(k), to_dev(v)
        words = wl.pack_mask(wl.tile_mask_bool(H, S, 0.3, seed=S))
        m = mask_to_dev(words)
        scale = 1.0 / math.sqrt(D)
        ref = torch.empty((P, B, S // P, H, D), dtype=torch.bfloat16, device=qd.device)
        binding.attn_fwd_relayout_ws_async(qd, kd, vd, ref, B, H, S, D, P, scale, m)
        g = Guarded((P, B, S // P, H, D))
        binding.attn_fwd_relayout_noalloc_async(qd, kd, vd, g.out, B, H, S, D, P, scale, m)
        torch.cuda.synchronize()
        g.check_guards()
        assert g.unwritten() == 0
        assert torch.equal(g.out.view(torch.int16), ref.view(torch.int16))
        rows = sample_rows(S, P, seed=S, n_random=8)
        want = oracle.attention(q.double().numpy(), k.double().numpy(), v.double().numpy(), scale,
                                words, rows=rows)
        assert_close(slab_rows(g.out, rows, S, P), want, f"no-alloc masked S={S}")
