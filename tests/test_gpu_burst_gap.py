"""GPU: the store-burst microbenchmark.

* It writes exactly its documented pattern and reports ordered, plausible
  timestamps (correctness of the measurement tool).
* The Burst-Gap equation of the pages ("Technical Summary: X-Stage in DiT
  Inference", Methodology), as the oracle writes it (oracle.burst_gap.t_iss),
  predicts the measured steady-state issue time of points it was not fitted
  on.  For each burst volume, T0 is the issue time at the largest gap and
  V / R the issue time plus gap at G = 0; the equation must then give the
  other gaps of that volume: the drain-dominated middle (V / R - G at least
  twice T0), where the issue time falls with slope -1, and backpressure-free
  gaps (G >= 1.5 V / R) short of the largest.  R is fitted per volume
  because on one GPU the L2 and MALL write-back absorb a burst smaller than
  their capacity faster than a burst that must stream to HBM.
* The completion-coupled issuer (each burst made visible device-wide before
  the next) is never faster than the decoupled one at any gap.
"""
import sys

import numpy as np
import pytest
import torch

from flashattention_output_re_amd import burst_gap as bg
from oracle import burst_gap as model

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("K,Vp,bursts,gap,nt,cp", [(8, 4096, 3, 10, 0, 0), (37, 12288, 5, 200, 1, 0),
                                                   (256, 65536, 6, 0, 0, 0),
                                                   (64, 16384, 4, 100, 0, 1)])
def test_pattern_and_timestamps(K, Vp, bursts, gap, nt, cp):
    print(f"[burst-gap] K={K} Vp={Vp} bursts={bursts} gap={gap} nt={nt} coupled={cp}",
          file=sys.stderr, flush=True)
    n = bursts * K * Vp // 4
    dst = torch.full((n + 1024,), -1, dtype=torch.int32, device="cuda:0")
    issue, gapt, clock, complete = bg.run(dst, K, Vp, bursts, gap, bool(nt), bool(cp))
    got = dst[:n].cpu().numpy().view(np.uint32).reshape(bursts, K, Vp // 16, 4)
    assert np.array_equal(got, bg.expected_chunks(K, Vp, bursts))
    assert bool((dst[n:] == -1).all()), "write past the bursts"
    assert issue.shape == (K, bursts) and gapt.shape == (K, bursts)
    assert np.all(issue > 0) and np.all(gapt >= 0)
    assert 0.3e9 < clock < 3.5e9
    assert complete > 0


# Relative error allowed between the equation and a measured steady-state
# issue time.  The per-volume fits have left residuals of a few per cent at
# these points; 25% still separates the regimes, whose values differ 3-10x
# there.
TOL = 0.25


def test_issue_time_follows_the_burst_gap_equation():
    K = torch.cuda.get_device_properties(0).multi_processor_count
    small, big = 64 << 10, 1 << 20
    cfg = [(K, small, g, False) for g in (0, 10, 30, 3000, 30000)] + \
          [(K, big, g, False) for g in (0, 300, 1000, 3000, 10000, 30000)] + \
          [(K, big, g, False, True) for g in (0, 3000, 30000)]
    print(f"[burst-gap model] K={K}", file=sys.stderr, flush=True)
    rows = bg.measure(cfg, bursts=16)
    dec = [r for r in rows if not r["coupled"]]
    checked = 0
    for vp in (small, big):
        sel = [r for r in dec if r["bytes_per_producer"] == vp]
        V = sel[0]["volume"]
        far = max(sel, key=lambda r: r["gap_s"])
        near = next(r for r in sel if r["gap_iters"] == 0)
        T0 = far["t_iss_s"]
        R = V / (near["t_iss_s"] + near["gap_s"])
        assert 1e12 < R < 3e13, R          # bytes per second, local HBM
        for r in sel:
            if r is far or r is near:
                continue                   # fitting points
            G = r["gap_s"]
            drain = V / R - G >= 2 * T0
            free = G >= 1.5 * V / R
            if not (drain or free):
                continue                   # near the regime boundary
            pred = float(model.t_iss(G, T0, V, R))
            assert model.regime(G, T0, V, R) == ("drain-dominated" if drain else "backpressure-free")
            err = abs(pred - r["t_iss_s"]) / r["t_iss_s"]
            print(f"  Vp={vp >> 10} KiB G={G * 1e6:.2f} us: measured {r['t_iss_s'] * 1e6:.3f} us, "
                  f"model {pred * 1e6:.3f} us ({err:.1%})", file=sys.stderr, flush=True)
            assert err <= TOL, (vp, G, r["t_iss_s"], pred)
            checked += 1
    assert checked >= 4
    # Completion-coupled issue times, per gap, against the decoupled ones.
    cp = {r["gap_iters"]: r["t_iss_s"] for r in rows if r["coupled"]}
    de = {r["gap_iters"]: r["t_iss_s"] for r in dec if r["bytes_per_producer"] == big}
    for g in cp:
        print(f"  coupled Vp={big >> 10} KiB gap_iters={g}: {cp[g] * 1e6:.3f} us "
              f"(decoupled {de[g] * 1e6:.3f} us)", file=sys.stderr, flush=True)
        assert cp[g] >= 0.95 * de[g], (g, cp, de)
