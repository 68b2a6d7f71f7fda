"""The Burst-Gap fitting code (mixture_experts_ffn_dispatch_amd/xstage.py, host logic) against
the model oracle (oracle/burst_gap.py): the product's predictions equal the oracle's formulas,
and its three fits recover known parameters from measurements the oracle generates (X-Stage
paper, Section 3: drain rate from zero-gap periods, issue floor from the large-gap plateau,
capacity from the isolated-burst knee)."""
import numpy as np
import pytest

from mixture_experts_ffn_dispatch_amd import xstage as X
from oracle import burst_gap as M

MIB = 1 << 20
R, T0, Q = 5.2e12, 1.3e-6, 48 * MIB


def test_predictions_equal_the_model():
    v = np.array([1, 8, 64, 512]) * MIB
    gaps = np.linspace(0, 2e-4, 41)
    for vv in v:
        np.testing.assert_allclose(X.predict_issue(vv, R, T0, gaps), M.issue_time(vv, R, T0, gaps), rtol=0, atol=0)
        np.testing.assert_allclose(X.predict_period(vv, R, T0, gaps), M.period(vv, R, T0, gaps), rtol=0, atol=0)
    np.testing.assert_allclose(X.predict_isolated(v, R, T0, Q), M.isolated_issue_time(v, R, T0, Q), rtol=0, atol=0)
    for g in (0.0, 1e-6, 1e-4):
        d = X.design_test(16 * MIB, R, T0, Q, g)
        assert (d["rate_bound"], d["capacity_bound"]) == M.design_test(16 * MIB, R, T0, Q, g)
        assert d["recovery_gap_s"] == pytest.approx(float(M.recovery_gap(16 * MIB, R, T0)))


def test_fits_recover_known_parameters():
    rng = np.random.default_rng(7)
    noise = lambda x: x * (1 + 0.005 * rng.standard_normal(np.shape(x)))  # 0.5% measurement noise
    # zero-gap periodic bursts in the drain-dominated regime
    v = np.array([64, 128, 256, 512, 1024]) * MIB
    r = X.fit_drain_rate(v, noise(M.steady_period_zero_gap(v, R)))
    assert r == pytest.approx(R, rel=0.01)
    # gap sweep of one volume: the plateau gives the floor
    vol = 32 * MIB
    gaps = np.linspace(0, 3 * vol / R, 25)
    t0 = X.fit_issue_floor(gaps, noise(M.issue_time(vol, R, T0, gaps)))
    assert t0 == pytest.approx(T0, rel=0.02)
    # isolated bursts across the knee give the capacity and the knee: before the knee a burst
    # issues at an absorb rate S (its backpressure-free issue time is V / S), after it on the
    # drain-limited branch; the oracle gives each point with t_iss0 = V / S
    S = 4.0 * R
    vi = np.array([1, 4, 16, 32, 64, 128, 256, 512]) * MIB
    t = noise(np.array([float(M.isolated_issue_time(v, R, v / S, Q)) for v in vi]))
    q = X.fit_capacity(vi, t, R)
    assert q == pytest.approx(Q, rel=0.03)
    s_abs, v_knee = X.fit_knee(vi, t, R, q)
    assert s_abs == pytest.approx(S, rel=0.02)
    # the knee is where V - R * (V / S) reaches Q
    assert v_knee == pytest.approx(Q / (1 - R / S), rel=0.04)
    assert float(M.isolated_peak(v_knee, R, v_knee / s_abs)) == pytest.approx(q, rel=1e-9)
    # absorbing no faster than the drain: no knee
    assert X.fit_knee(vi, vi / (0.5 * R), R, q)[1] is None
