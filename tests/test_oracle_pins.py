"""Pins of the CPU oracle to facts outside itself (CPU only).

Each pin is a fact fixed by mathematics or by hand derivation, not a retyping
of the oracle's formula: exact rational examples, closed forms (identical
keys, one dominant score, V == 1), torch's independent fp64 attention,
invariants of softmax attention, a hand-written re-layout example and the
bijection property.  The planted-mistake tests at the end show that plausible
slips in the oracle (a dropped scale, a wrong softmax axis, a transposed mask,
a wrong tile size, K in place of V, a swapped re-layout axis, strided slabs)
each break at least one pin.
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
import oracle.attn as oatt
import oracle.relayout as orel
import workloads as wl

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rng(seed):
    return np.random.default_rng(seed)


def _bf16_values(x):
    """float array -> float64 values of its bf16 (RNE) rounding."""
    return wl.to_bf16(np.asarray(x, dtype=np.float32)).to(torch.float64).numpy()


# ---------------------------------------------------------------------------
# Pin functions.  Each takes the attention and re-layout implementations under
# test and raises AssertionError when the implementation violates the pin.
# ---------------------------------------------------------------------------
def pin_hand_attention(attn, relayout):
    with open(os.path.join(GOLDEN, "hand_attention.json")) as f:
        g = json.load(f)
    for case in g["cases"]:
        scale = {"ln2": math.log(2.0), "-ln2": -math.log(2.0)}[case["scale"]]
        q = np.array(case["q"], dtype=np.float64)
        k = np.array(case["k"], dtype=np.float64)
        v = np.array(case["v"], dtype=np.float64)
        want = np.vectorize(lambda s: float(Fraction(s)))(np.array(case["out"]))
        got = attn(q, k, v, scale)
        np.testing.assert_allclose(got, want, rtol=0, atol=1e-13, err_msg=case["name"])


def pin_hand_relayout(attn, relayout):
    with open(os.path.join(GOLDEN, "hand_relayout.json")) as f:
        g = json.load(f)
    B, H, S, D, P = (g[x] for x in "BHSDP")
    o = np.zeros((B, H, S, D))
    for b in range(B):
        for h in range(H):
            for s in range(S):
                o[b, h, s, 0] = 1000 * b + 100 * h + s
    got = relayout(o, P)
    assert got.shape == (P, B, S // P, H, D)
    assert got.reshape(-1).tolist() == g["out_flat"]


def pin_identical_keys(attn, relayout):
    """All keys equal -> every score in a row is equal -> O[s] = mean of the
    V rows the row may see (all of them, or those of its kept tiles)."""
    r = _rng(1)
    B, H, S, D = 2, 2, 300, 16
    q = r.standard_normal((B, H, S, D))
    k = np.broadcast_to(r.standard_normal((B, H, 1, D)), (B, H, S, D)).copy()
    v = r.standard_normal((B, H, S, D))
    got = attn(q, k, v, 0.3)
    want = np.broadcast_to(v.mean(axis=2, keepdims=True), got.shape)
    np.testing.assert_allclose(got, want, atol=1e-12)
    # With a tile mask: mean over the keys of kept tiles.
    keep = wl.tile_mask_bool(H, S, 0.5, seed=7)
    got = attn(q, k, v, 0.3, wl.pack_mask(keep))
    nT = keep.shape[1]
    tile_of = np.arange(S) // 128
    for h in range(H):
        for i in range(nT):
            cols = keep[h, i][tile_of]
            rows = tile_of == i
            want = v[:, h][:, cols].mean(axis=1)
            np.testing.assert_allclose(got[:, h][:, rows], np.broadcast_to(
                want[:, None, :], got[:, h][:, rows].shape), atol=1e-12)


def pin_scale_zero(attn, relayout):
    r = _rng(2)
    q, k, v = (r.standard_normal((1, 3, 130, 8)) for _ in range(3))
    got = attn(q, k, v, 0.0)
    np.testing.assert_allclose(got, np.broadcast_to(v.mean(axis=2, keepdims=True),
                                                    got.shape), atol=1e-12)


def pin_dominant_score(attn, relayout):
    """Integer-tagged inputs: each query's own key wins by >= 22 nats, so the
    output is that key's V row (and rounds to it exactly in bf16)."""
    for (B, H, S, D) in [(1, 1, 256, 64), (2, 3, 300, 64), (1, 2, 1000, 128)]:
        t = wl.tag_inputs(B, H, S, D)
        q, k, v = t.f64("q"), t.f64("k"), t.f64("v")
        got = attn(q, k, v, 1.0 / math.sqrt(D))
        np.testing.assert_allclose(got, v, rtol=0, atol=1e-4)
        assert np.array_equal(_bf16_values(got), v)


def pin_rows_sum_to_one(attn, relayout):
    r = _rng(3)
    q, k = (r.standard_normal((2, 2, 200, 32)) for _ in range(2))
    v = np.ones((2, 2, 200, 32))
    np.testing.assert_allclose(attn(q, k, v, 0.7), 1.0, atol=1e-12)
    keep = wl.tile_mask_bool(2, 200, 0.5, seed=3)
    np.testing.assert_allclose(attn(q, k, v, 0.7, wl.pack_mask(keep)), 1.0, atol=1e-12)


def pin_torch_sdpa(attn, relayout):
    """torch's own fp64 attention (an independent implementation) on small
    cases, dense and with a tile mask, ragged tails included."""
    r = _rng(4)
    for (B, H, S, D, masked) in [(1, 1, 1, 4, False), (1, 2, 5, 8, False),
                                 (2, 2, 16, 16, False), (1, 2, 200, 16, True),
                                 (1, 1, 300, 8, True)]:
        q, k, v = (r.standard_normal((B, H, S, D)) for _ in range(3))
        scale = 0.37
        mask_words, tmask = None, None
        if masked:
            keep = wl.tile_mask_bool(H, S, 0.4, seed=S)
            mask_words = wl.pack_mask(keep)
            tile = np.arange(S) // 128
            tmask = torch.from_numpy(keep[:, tile][:, :, tile])[None]
        want = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v),
            attn_mask=tmask, scale=scale).numpy()
        got = attn(q, k, v, scale, mask_words)
        np.testing.assert_allclose(got, want, atol=1e-12, rtol=1e-12)


def pin_invariants(attn, relayout):
    r = _rng(5)
    B, H, S, D = 1, 2, 150, 16
    q, k, v, v2 = (r.standard_normal((B, H, S, D)) for _ in range(4))
    base = attn(q, k, v, 0.5)
    # A joint permutation of the key/value rows changes nothing (dense).
    perm = r.permutation(S)
    np.testing.assert_allclose(attn(q, k[:, :, perm], v[:, :, perm], 0.5), base, atol=1e-12)
    # Adding one vector to every key shifts each score row by a constant.
    c = r.standard_normal((1, 1, 1, D))
    np.testing.assert_allclose(attn(q, k + c, v, 0.5), base, atol=1e-10)
    # Linear in V.
    np.testing.assert_allclose(attn(q, k, 2.0 * v - 3.0 * v2, 0.5),
                               2.0 * base - 3.0 * attn(q, k, v2, 0.5), atol=1e-11)


def pin_block_diagonal(attn, relayout):
    """A diagonal-only tile mask splits attention into independent 128-token
    blocks, each equal to dense attention on that block alone."""
    r = _rng(6)
    B, H, S, D = 1, 2, 300, 8
    q, k, v = (r.standard_normal((B, H, S, D)) for _ in range(3))
    nT = 3
    keep = np.zeros((H, nT, nT), dtype=bool)
    keep[:, np.arange(nT), np.arange(nT)] = True
    got = attn(q, k, v, 0.4, wl.pack_mask(keep))
    for i in range(nT):
        sl = slice(128 * i, min(S, 128 * i + 128))
        want = attn(q[:, :, sl], k[:, :, sl], v[:, :, sl], 0.4)
        np.testing.assert_allclose(got[:, :, sl], want, atol=1e-12)


def pin_relayout_bijection(attn, relayout):
    """Every source element lands exactly once, slab p holds exactly tokens
    [p S/P, (p+1) S/P), heads stay inside their token row."""
    for (B, H, S, D, P) in [(1, 1, 8, 2, 1), (2, 3, 12, 4, 3), (1, 5, 40, 8, 8)]:
        o = np.arange(B * H * S * D, dtype=np.float64).reshape(B, H, S, D)
        got = relayout(o, P)
        assert got.shape == (P, B, S // P, H, D)
        assert np.array_equal(np.sort(got.reshape(-1)), o.reshape(-1))
        Sp = S // P
        for p in range(P):
            src = o[:, :, p * Sp:(p + 1) * Sp]          # [B][H][Sp][D]
            for t in range(Sp):
                for h in range(H):
                    assert np.array_equal(got[p, :, t, h], src[:, h, t])


PINS = [pin_hand_attention, pin_hand_relayout, pin_identical_keys, pin_scale_zero,
        pin_dominant_score, pin_rows_sum_to_one, pin_torch_sdpa, pin_invariants,
        pin_block_diagonal, pin_relayout_bijection]


def _attn(q, k, v, scale, mask_words=None):
    return oracle.attention(q, k, v, scale, mask_words)


def failing_pins(attn, relayout):
    bad = []
    for pin in PINS:
        try:
            pin(attn, relayout)
        except Exception:  # a crash is as much a failed pin as a wrong value
            bad.append(pin.__name__)
    return bad


# ---------------------------------------------------------------- the oracle
@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
@pytest.mark.parametrize("relayout", [oracle.relayout_split, oracle.relayout_index],
                         ids=["split", "index"])
def test_oracle_pin(pin, relayout):
    pin(_attn, relayout)


def test_relayout_derivations_agree():
    r = _rng(8)
    for (B, H, S, D, P) in [(1, 1, 256, 64, 2), (2, 3, 96, 8, 8), (1, 5, 4095 * 8, 2, 8)]:
        o = r.standard_normal((B, H, S, D))
        a, b = oracle.relayout_split(o, P), oracle.relayout_index(o, P)
        assert a.shape == b.shape and np.array_equal(a, b)


def test_probs_rows_sum_to_one():
    r = _rng(9)
    q, k = r.standard_normal((2, 333, 16)), r.standard_normal((2, 333, 16))
    keep = wl.tile_mask_bool(1, 333, 0.5, seed=1)[0]
    for kk in (None, keep):
        p = oatt.attention_probs(q[0], k[0], 1.3, kk)
        np.testing.assert_allclose(p.sum(axis=1), 1.0, atol=1e-12)
        assert (p >= 0).all()


def test_fully_masked_row_is_zero():
    r = _rng(10)
    q, k, v = (r.standard_normal((1, 1, 200, 8)) for _ in range(3))
    keep = np.zeros((1, 2, 2), dtype=bool)
    keep[0, 1, 1] = True          # tile row 0 keeps nothing
    out = oracle.attention(q, k, v, 0.5, wl.pack_mask(keep))
    assert np.all(out[0, 0, :128] == 0.0)
    assert np.isfinite(out).all()


def test_mask_bit_convention():
    """The oracle's unpacking inverts the input generator's packing, including
    rows wider than one 64-bit word."""
    for S in (1, 128, 129, 8192 + 5, 32760):
        keep = wl.tile_mask_bool(2, S, 0.3, seed=S)
        assert np.array_equal(oatt.unpack_mask(wl.pack_mask(keep), S), keep)
    keep = np.zeros((1, 70, 70), dtype=bool)
    keep[0, 3, 65] = True
    w = wl.pack_mask(keep)
    assert w[0, 3, 1] == np.uint64(1 << 1) and w[0, 3, 0] == 0


def test_rows_subset_matches_full():
    r = _rng(11)
    q, k, v = (r.standard_normal((1, 2, 400, 16)) for _ in range(3))
    rows = [0, 5, 127, 128, 255, 399]
    full = oracle.attention(q, k, v, 0.2)
    sub = oracle.attention(q, k, v, 0.2, rows=rows)
    np.testing.assert_allclose(sub, full[:, :, rows], rtol=0, atol=1e-13)


# ------------------------------------------------------- planted mistakes
def _mut_no_scale(q, k, v, scale, mask_words=None):
    return oracle.attention(q, k, v, 1.0, mask_words)


def _mut_k_as_v(q, k, v, scale, mask_words=None):
    return oracle.attention(q, k, k, scale, mask_words)


def _mut_transposed_mask(q, k, v, scale, mask_words=None):
    if mask_words is None:
        return oracle.attention(q, k, v, scale)
    keep = oatt.unpack_mask(mask_words, q.shape[2])
    return oracle.attention(q, k, v, scale, wl.pack_mask(keep.transpose(0, 2, 1)))


def _mut_sign(q, k, v, scale, mask_words=None):
    return oracle.attention(q, k, v, -scale, mask_words)


def _mut_transposed_scores(q, k, v, scale, mask_words=None):
    # Q and K swapped: z[s, j] = <K[s], Q[j]>.
    return oracle.attention(k, q, v, scale, mask_words)


def _relayout_swapped(o, P):
    B, H, S, D = o.shape
    Sp = S // P
    return o.reshape(B, H, P, Sp, D).transpose(2, 0, 1, 3, 4).reshape(P, B, Sp, H, D)


def _relayout_strided(o, P):
    B, H, S, D = o.shape
    Sp = S // P
    return np.stack([o[:, :, p::P].transpose(0, 2, 1, 3) for p in range(P)])


@pytest.mark.parametrize("mutant", [_mut_no_scale, _mut_k_as_v, _mut_transposed_mask,
                                    _mut_sign, _mut_transposed_scores])
def test_planted_attention_mistakes_are_caught(mutant):
    assert failing_pins(mutant, oracle.relayout_split)


def test_planted_softmax_axis_mistake_is_caught(monkeypatch):
    def wrong_axis(q, k, scale, keep=None, rows=None):
        S = k.shape[0]
        rows = np.arange(S) if rows is None else np.asarray(rows)
        z = (q[rows] @ k.T) * scale
        e = np.exp(z - z.max(axis=0, keepdims=True))
        return e / e.sum(axis=0, keepdims=True)
    monkeypatch.setattr(oatt, "attention_probs", wrong_axis)
    assert failing_pins(_attn, oracle.relayout_split)


def test_planted_tile_size_mistake_is_caught(monkeypatch):
    monkeypatch.setattr(oatt, "MASK_TILE", 64)
    bad = failing_pins(_attn, oracle.relayout_split)
    assert bad


def test_planted_relayout_mistakes_are_caught():
    for mut in (_relayout_swapped, _relayout_strided):
        assert failing_pins(_attn, mut)


def test_oracle_passes_every_pin():
    assert failing_pins(_attn, oracle.relayout_split) == []
    assert failing_pins(_attn, oracle.relayout_index) == []


def test_values_wider_than_keys_match_torch_sdpa():
    """Value rows of another width than the keys (used to get the output for
    V and for |V| from one softmax): torch's fp64 attention, which also takes
    Dv != D, agrees, dense and with a tile mask."""
    r = _rng(12)
    for (B, H, S, D, Dv, masked) in [(1, 2, 40, 8, 24, False), (2, 1, 260, 16, 32, True)]:
        q, k = (r.standard_normal((B, H, S, D)) for _ in range(2))
        v = r.standard_normal((B, H, S, Dv))
        mask_words, tmask = None, None
        if masked:
            keep = wl.tile_mask_bool(H, S, 0.5, seed=S)
            mask_words = wl.pack_mask(keep)
            tile = np.arange(S) // 128
            tmask = torch.from_numpy(keep[:, tile][:, :, tile])[None]
        want = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v),
            attn_mask=tmask, scale=0.3).numpy()
        got = oracle.attention(q, k, v, 0.3, mask_words)
        assert got.shape == (B, H, S, Dv)
        np.testing.assert_allclose(got, want, atol=1e-12, rtol=1e-12)
