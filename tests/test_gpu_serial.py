"""GPU: the standalone re-layout copy (the exchange half of the serial
baseline) against the oracle's re-layout, bit for bit, and the serial path
(plain attention, then the copy) against the fused kernel."""
import sys

import numpy as np
import pytest
import torch

import flashattention_output_re_amd as fa
import oracle
import workloads as wl
from gpu_util import CANARY, Guarded, dev, to_dev

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def random_bits(B, H, S, D, seed):
    """Every 16-bit pattern but the canary, as bf16 (NaN payloads included:
    the copy moves bits, it does no arithmetic)."""
    r = np.random.default_rng(seed)
    bits = r.integers(-32768, 32768, size=(B, H, S, D), dtype=np.int64).astype(np.int16)
    bits[bits == CANARY] = 0
    return bits


def run_copy(plain, B, H, S, D, P, stream=None):
    g = Guarded((P, B, S // P, H, D))
    fa.relayout_to_slabs_async(plain, g.out, B, H, S, D, P, stream)
    torch.cuda.synchronize()
    g.check_guards()
    assert g.unwritten() == 0, "slab elements left unwritten"
    return g.out


@pytest.mark.parametrize("B,H,S,D,P", [
    (1, 1, 1, 64, 1), (1, 1, 2, 128, 2), (2, 3, 256, 128, 2), (3, 2, 1000, 64, 8),
    (1, 4, 17, 128, 17), (2, 1, 640, 128, 5), (1, 3, 4096, 128, 8), (1, 5, 32760, 128, 8),
    (1, 5, 75600, 128, 8), (4, 7, 96, 64, 96),
])
def test_relayout_copy_bit_exact(B, H, S, D, P):
    say(f"[copy] B={B} H={H} S={S} D={D} P={P}")
    bits = random_bits(B, H, S, D, seed=B * 7919 + H * 131 + S + D + P)
    plain = to_dev(torch.from_numpy(bits).view(torch.bfloat16))
    out = run_copy(plain, B, H, S, D, P)
    want = oracle.relayout_split(bits, P)
    got = out.view(torch.int16).cpu().numpy()
    bad = np.argwhere(got != want)
    assert bad.size == 0, f"{len(bad)} mismatches, first at {bad[:5].tolist()}"


def test_relayout_copy_blocking_and_stream():
    B, H, S, D, P = 2, 2, 512, 128, 4
    bits = random_bits(B, H, S, D, seed=5)
    plain = to_dev(torch.from_numpy(bits).view(torch.bfloat16))
    a = torch.empty((P, B, S // P, H, D), dtype=torch.bfloat16, device=dev())
    fa.relayout_to_slabs(plain, a, B, H, S, D, P)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        b = run_copy(plain, B, H, S, D, P, stream=s)
    want = oracle.relayout_split(bits, P)
    assert np.array_equal(a.view(torch.int16).cpu().numpy(), want)
    assert np.array_equal(b.view(torch.int16).cpu().numpy(), want)


@pytest.mark.parametrize("name", ["tiny", "image", "video"])
def test_serial_equals_fused(name):
    """Plain attention followed by the copy gives the fused kernel's slabs bit
    for bit (the two attention layouts share their arithmetic)."""
    w = wl.WORKLOADS[name]
    say(f"[serial] {name}")
    inp = wl.make(name)
    q, k, v = (to_dev(t) for t in (inp.q, inp.k, inp.v))
    fused = torch.empty((w.P, w.B, w.S // w.P, w.H, w.D), dtype=torch.bfloat16, device=dev())
    fa.attn_fwd_relayout_async(q, k, v, fused, w.B, w.H, w.S, w.D, w.P, w.scale)
    plain = torch.empty((w.B, w.H, w.S, w.D), dtype=torch.bfloat16, device=dev())
    fa.attn_fwd_plain_async(q, k, v, plain, w.B, w.H, w.S, w.D, w.scale)
    serial = run_copy(plain, w.B, w.H, w.S, w.D, w.P)
    assert torch.equal(fused.view(torch.int16), serial.view(torch.int16))
