"""Burst-Gap model of sender-visible store-issue time (TEST INFRASTRUCTURE
ONLY, like the rest of this package).

The pages ("Technical Summary: X-Stage in DiT Inference", Methodology: the
X-Stage abstraction and the Burst-Gap model) give the issue time of a burst
of aggregate volume V from K producers, after a producer-side compute gap G
since the previous burst, as the larger of the backpressure-free issue time
T0(K, V) and the time the drain path still needs, V / R - G, with R the
effective drain rate.  Two regimes follow: drain-dominated when G is short,
backpressure-free when G covers the drain.  The outstanding capacity Q is the
volume that may be accepted but not yet drained: a stream of back-to-back
bursts (G = 0) issues at the backpressure-free pace until Q is outstanding,
then at the drain rate.

Functions (scalars or numpy arrays, seconds, bytes, bytes per second):
  t_iss(G, T0, V, R)   the model's issue time
  period(G, T0, V, R)  one burst plus its gap in steady state
  regime(G, T0, V, R)  "backpressure-free" or "drain-dominated"
  cumulative_issue_times(n, T0, V, R, Q)
                       end times of n back-to-back bursts (G = 0) issued at
                       V per T0 while less than Q is outstanding, at the
                       drain rate once Q is full (the capacity reading).
"""
from __future__ import annotations

import numpy as np


def t_iss(G, T0, V, R):
    return np.maximum(T0, V / R - G)


def period(G, T0, V, R):
    return t_iss(G, T0, V, R) + G


def regime(G, T0, V, R):
    return "backpressure-free" if V / R - G <= T0 else "drain-dominated"


def cumulative_issue_times(n, T0, V, R, Q):
    """End time of each of n back-to-back bursts.  Bytes leave at rate R from
    time 0; a burst of V bytes takes T0 to issue unless issuing it would leave
    more than Q bytes outstanding, in which case it ends when the drain has
    made room for its last byte."""
    ends = []
    t = 0.0
    for i in range(1, n + 1):
        t_fast = t + T0
        sent = i * V
        t_room = (sent - Q) / R        # the drain must have taken sent - Q bytes
        t = max(t_fast, t_room)
        ends.append(t)
    return np.array(ends)
