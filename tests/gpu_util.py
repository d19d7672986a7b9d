"""Helpers shared by the GPU tests: device placement, comparison against the
oracle, canary-guarded output buffers."""
from __future__ import annotations

import numpy as np
import torch

import flashattention_output_re_amd as fa

MAX_ABS = 1e-2    # workload gate: max |gpu - oracle| over every compared element
MEAN_ABS = 1e-3   # workload gate: mean |gpu - oracle|
# Element-wise bound from the arithmetic.  bf16 keeps 8 significant bits, so
# round-to-nearest has relative error <= u = 2^-8.  The kernel rounds each
# softmax weight fed to the PV product to bf16 (the output moves by at most
# u * sum_j P_j |V_j|) and rounds the output to bf16 (<= u |O|); fp32
# accumulation, exp2 and the division add far less (the floor and slack).
BOUND_REL = 2.0 ** -8
BOUND_SLACK = 1.1
BOUND_FLOOR = 1e-5
CANARY = -1       # 0xFFFF as int16: a bf16 NaN pattern the kernel never writes
GUARD = 4096      # guard elements on each side of an output buffer


def dev():
    return torch.device("cuda:0")


def to_dev(t: torch.Tensor) -> torch.Tensor:
    return t.contiguous().to(dev())


def mask_to_dev(words):
    if words is None:
        return None
    return torch.from_numpy(np.ascontiguousarray(words).view(np.int64)).to(dev())


class Guarded:
    """A bf16 output buffer of `shape` inside canary-filled guard bands."""

    def __init__(self, shape):
        self.shape = tuple(shape)
        n = int(np.prod(self.shape))
        self.raw = torch.full((n + 2 * GUARD,), CANARY, dtype=torch.int16, device=dev())
        self.n = n

    @property
    def out(self) -> torch.Tensor:
        return self.raw[GUARD:GUARD + self.n].view(torch.bfloat16).view(self.shape)

    def check_guards(self):
        r = self.raw
        assert bool((r[:GUARD] == CANARY).all()), "write below the output buffer"
        assert bool((r[GUARD + self.n:] == CANARY).all()), "write above the output buffer"

    def unwritten(self) -> int:
        return int((self.raw[GUARD:GUARD + self.n] == CANARY).sum())


def run_slabs(q, k, v, P, scale, mask=None, stream=None):
    B, H, S, D = q.shape
    g = Guarded((P, B, S // P, H, D))
    fa.attn_fwd_relayout_async(q, k, v, g.out, B, H, S, D, P, scale, mask, stream)
    torch.cuda.synchronize()
    g.check_guards()
    assert g.unwritten() == 0, "slab elements left unwritten"
    return g.out


def run_plain(q, k, v, scale, mask=None, stream=None):
    B, H, S, D = q.shape
    g = Guarded((B, H, S, D))
    fa.attn_fwd_plain_async(q, k, v, g.out, B, H, S, D, scale, mask, stream)
    torch.cuda.synchronize()
    g.check_guards()
    assert g.unwritten() == 0, "output elements left unwritten"
    return g.out


def f64(t: torch.Tensor) -> np.ndarray:
    return t.to(torch.float64).cpu().numpy()


def errors(got: np.ndarray, want: np.ndarray) -> dict:
    diff = np.abs(got - want)
    rms = float(np.sqrt(np.mean(want ** 2))) or 1.0
    return {"max_abs": float(diff.max()), "mean_abs": float(diff.mean()),
            "max_rel_rms": float(diff.max()) / rms}


def assert_close(got: np.ndarray, want: np.ndarray, what: str = ""):
    assert got.shape == want.shape, (got.shape, want.shape)
    assert np.isfinite(got).all(), f"{what}: non-finite output"
    e = errors(got, want)
    assert e["max_abs"] <= MAX_ABS and e["mean_abs"] <= MEAN_ABS, f"{what}: {e}"
    return e


def assert_within_bound(got: np.ndarray, ref: np.ndarray, ref_absv: np.ndarray, what: str = ""):
    """|got - ref| <= 1.1 * 2^-8 * (|ref| + sum_j P_j |V_j|) + 1e-5 element-wise;
    ``ref_absv`` is the oracle's attention output for |V|."""
    assert got.shape == ref.shape == ref_absv.shape
    assert np.isfinite(got).all(), f"{what}: non-finite output"
    bound = BOUND_SLACK * BOUND_REL * (np.abs(ref) + ref_absv) + BOUND_FLOOR
    excess = np.abs(got - ref) - bound
    worst = np.unravel_index(np.argmax(excess), excess.shape)
    assert excess.max() <= 0.0, (f"{what}: |err| {abs(got - ref)[worst]:.3e} > bound "
                                 f"{bound[worst]:.3e} at {worst}")


def slab_rows(slabs: torch.Tensor, rows, S: int, P: int) -> np.ndarray:
    """Rows `rows` of every (b, h) from a slab tensor, as [B][H][len(rows)][D]."""
    Sp = S // P
    rows = np.asarray(rows)
    p, t = rows // Sp, rows % Sp
    idx_p = torch.as_tensor(p, device=slabs.device)
    idx_t = torch.as_tensor(t, device=slabs.device)
    sel = slabs[idx_p, :, idx_t]                    # [R][B][H][D]
    return f64(sel.permute(1, 2, 0, 3).contiguous())


def sample_rows(S: int, P: int, seed: int = 0, n_random: int = 24) -> np.ndarray:
    """Rows at tile edges, slab edges, the ragged tail and some random ones."""
    Sp = S // P
    cand = {0, 1, 31, 32, 63, 64, 127, 128, 129, 255, 256, 257, 383, 384, S - 1, S - 2, S - 33}
    for tile in (128, 256):        # the last tile of each tiling, and its halves
        last = ((S - 1) // tile) * tile
        cand |= {last, last - 1, last + 1, last + tile // 2 - 1, last + tile // 2}
    for p in range(1, P):
        cand |= {p * Sp - 1, p * Sp, p * Sp + 1}
    r = np.random.default_rng(seed)
    cand |= set(r.integers(0, S, size=n_random).tolist())
    return np.array(sorted(x for x in cand if 0 <= x < S))
