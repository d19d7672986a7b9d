"""GPU: the store-burst microbenchmark writes exactly its documented pattern
and reports ordered, plausible timestamps (correctness of the measurement
tool; its numbers are reported by the driver module, not asserted here)."""
import sys

import numpy as np
import pytest
import torch

from flashattention_output_re_amd import burst_gap as bg

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("K,Vp,bursts,gap,nt", [(8, 4096, 3, 10, 0), (37, 12288, 5, 200, 1),
                                                (256, 65536, 6, 0, 0)])
def test_pattern_and_timestamps(K, Vp, bursts, gap, nt):
    print(f"[burst-gap] K={K} Vp={Vp} bursts={bursts} gap={gap} nt={nt}", file=sys.stderr,
          flush=True)
    n = bursts * K * Vp // 4
    dst = torch.full((n + 1024,), -1, dtype=torch.int32, device="cuda:0")
    issue, gapt, clock, complete = bg.run(dst, K, Vp, bursts, gap, bool(nt))
    got = dst[:n].cpu().numpy().view(np.uint32).reshape(bursts, K, Vp // 16, 4)
    assert np.array_equal(got, bg.expected_chunks(K, Vp, bursts))
    assert bool((dst[n:] == -1).all()), "write past the bursts"
    assert issue.shape == (K, bursts) and gapt.shape == (K, bursts)
    assert np.all(issue > 0) and np.all(gapt >= 0)
    assert 0.3e9 < clock < 3.5e9
    assert complete > 0
