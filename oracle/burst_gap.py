"""Plain definition of the Burst-Gap model (CPU oracle; test infrastructure only).

Follows Section 3 of "X-Stage: An Overlooked Pipeline Stage for Communication-Computation
Overlap in DiT Inference" (the Burst-Gap characterisation, Sections 3.2-3.5, and the design
test that opens Section 4). K producers each write B bytes in one burst, V = K * B in all;
between bursts each producer computes for a gap G. Three calibrated quantities describe the
sender-visible behaviour:

  t_iss0   backpressure-free issue time of a recovered burst (seconds)
  r        effective aggregate drain rate (bytes / second)
  q        effective outstanding capacity (bytes)

The page's display equations were lost in extraction; these are the plainest forms that its
prose states (and that its worked numbers satisfy, see the tests):

  steady state, drain-dominated:   period = V / r                  (flow conservation)
  a period is issue then gap:      period = t_iss + G
  issue is never faster than t_iss0, so
      t_iss  = max(t_iss0, V / r - G)
      period = max(V / r, t_iss0 + G)                              (the "max law")
  issue overhead:                  max(V / r - G - t_iss0, 0)
  recovery gap (plateau reached):  G* = V / r - t_iss0
  isolated burst: outstanding volume at the end of a backpressure-free issue is
      q_peak0 = V - r * t_iss0;  t_iss = t_iss0 if q_peak0 <= q, else (V - q) / r
  design test for recurring bursts (no modelled backpressure):
      V / r <= t_iss0 + G   (rate)   and   V - r * t_iss0 <= q   (capacity)

Every function is the formula written out, in float64.
"""
from __future__ import annotations

import numpy as np


def steady_period_zero_gap(v, r):
    """Zero-gap periodic bursts reach the drain-dominated steady state: period = V / r."""
    return np.asarray(v, np.float64) / float(r)


def issue_time(v, r, t_iss0, gap):
    """Periodic steady state: t_iss = max(t_iss0, V / r - G)."""
    return np.maximum(float(t_iss0), np.asarray(v, np.float64) / float(r) - np.asarray(gap, np.float64))


def period(v, r, t_iss0, gap):
    """Periodic steady state: period = max(V / r, t_iss0 + G) (= issue + gap)."""
    return np.maximum(np.asarray(v, np.float64) / float(r), float(t_iss0) + np.asarray(gap, np.float64))


def issue_overhead(v, r, t_iss0, gap):
    """Extra issue time caused by the previous burst: [V / r - G - t_iss0]_+."""
    return np.maximum(np.asarray(v, np.float64) / float(r) - np.asarray(gap, np.float64) - float(t_iss0), 0.0)


def recovery_gap(v, r, t_iss0):
    """The gap at which issue returns to t_iss0: G* = V / r - t_iss0."""
    return np.asarray(v, np.float64) / float(r) - float(t_iss0)


def isolated_peak(v, r, t_iss0):
    """Outstanding volume at the end of a backpressure-free isolated issue: V - r * t_iss0."""
    return np.asarray(v, np.float64) - float(r) * float(t_iss0)


def isolated_issue_time(v, r, t_iss0, q):
    """Isolated burst: t_iss0 while V - r t_iss0 <= q, else (V - q) / r."""
    v = np.asarray(v, np.float64)
    return np.where(isolated_peak(v, r, t_iss0) <= float(q), float(t_iss0), (v - float(q)) / float(r))


def capacity_from_knee(v_knee, r, t_iss0):
    """The capacity that puts the isolated-burst knee at v_knee: q = v_knee - r * t_iss0."""
    return float(v_knee) - float(r) * float(t_iss0)


def design_test(v, r, t_iss0, q, gap):
    """(rate bound holds, capacity bound holds) for recurring bursts of volume V and gap G."""
    v = float(v)
    return v / float(r) <= float(t_iss0) + float(gap), v - float(r) * float(t_iss0) <= float(q)
