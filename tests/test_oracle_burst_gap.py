"""Pins of the Burst-Gap model oracle (oracle/burst_gap.py) against the numbers the X-Stage
page works through (Section 3.5, isolated bursts; Section 4.3, the FlashAttention-4 output
tile) and against identities the model's prose fixes (a period is issue followed by gap; the
knee is continuous; the recovery gap is where the plateau starts)."""
import numpy as np
import pytest

from oracle import burst_gap as M

KIB, MIB = 1024, 1024 * 1024

# Section 3.5: K = 148 producers, knee at about 33 KiB per producer, R ~ 717 GB/s (fitted in
# Section 3.3), backpressure-free issue floor ~ 0.76 us at B = 32 KiB; capacity ~ 4.25 MiB.
K, B_KNEE, R, T0 = 148, 33 * KIB, 717e9, 0.76e-6


def test_knee_volume_and_capacity_match_the_page():
    v_knee = K * B_KNEE
    assert v_knee == 5_001_216
    assert v_knee / MIB == pytest.approx(4.77, abs=0.005)
    q = M.capacity_from_knee(v_knee, R, T0)
    assert R * T0 == pytest.approx(544_920.0)
    assert q == pytest.approx(4_456_296.0)
    assert q / MIB == pytest.approx(4.25, abs=0.005)


def test_fa4_output_tile_sits_below_the_knee():
    # Section 4.3: a 128 x 128 bf16 output tile is 32 KiB; 148 aligned producers give ~4.6 MiB
    tile = 128 * 128 * 2
    assert tile == 32 * KIB
    v = K * tile
    assert v / MIB == pytest.approx(4.625)
    q = M.capacity_from_knee(K * B_KNEE, R, T0)
    assert M.isolated_issue_time(v, R, T0, q) == pytest.approx(T0)  # no isolated backpressure
    assert M.design_test(v, R, T0, q, gap=1.0)[1]


def test_isolated_issue_time_is_continuous_at_the_knee_and_drain_limited_beyond():
    q = 3.0 * MIB
    v_knee = q + R * T0
    eps = 1.0
    assert M.isolated_issue_time(v_knee - eps, R, T0, q) == pytest.approx(T0)
    assert M.isolated_issue_time(v_knee + eps, R, T0, q) == pytest.approx(T0 + eps / R, rel=1e-12)
    # far beyond the knee: (V - q) / R, slope 1 / R
    v = np.array([2, 4, 8]) * v_knee
    t = M.isolated_issue_time(v, R, T0, q)
    np.testing.assert_allclose(t, (v - q) / R)
    np.testing.assert_allclose(np.diff(t) / np.diff(v), 1.0 / R)


@pytest.mark.parametrize("v", [64 * KIB, 4 * MIB, 256 * MIB])
def test_max_law_identities(v):
    gaps = np.linspace(0.0, 3.0 * v / R + 5e-6, 97)
    t_iss = M.issue_time(v, R, T0, gaps)
    per = M.period(v, R, T0, gaps)
    # a period is issue followed by gap
    np.testing.assert_allclose(per, t_iss + gaps, rtol=1e-12, atol=1e-18)
    # issue is never faster than the backpressure-free floor, overhead is the excess
    assert np.all(t_iss >= T0)
    np.testing.assert_allclose(M.issue_overhead(v, R, T0, gaps), t_iss - T0, atol=1e-18)
    # zero gap: the drain-dominated steady state V / R (whenever that exceeds the floor)
    assert M.period(v, R, T0, 0.0) == pytest.approx(max(v / R, T0))
    assert M.steady_period_zero_gap(v, R) == pytest.approx(v / R)
    # the period never drops below either branch, and the gap is not simply added on
    assert np.all(per >= v / R - 1e-18) and np.all(per >= T0 + gaps - 1e-18)
    assert np.all(per <= v / R + gaps + T0)


def test_recovery_gap_starts_the_plateau():
    v = 32 * MIB
    g_star = M.recovery_gap(v, R, T0)
    assert g_star == pytest.approx(v / R - T0)
    assert M.issue_time(v, R, T0, g_star) == pytest.approx(T0)
    assert M.issue_time(v, R, T0, g_star * 0.5) > T0
    assert M.issue_time(v, R, T0, g_star * 2.0) == pytest.approx(T0)
    # below G* the stall falls one for one with the gap (slope -1)
    g = np.array([0.1, 0.2, 0.3]) * g_star
    np.testing.assert_allclose(np.diff(M.issue_time(v, R, T0, g)), -np.diff(g))


def test_design_test_rate_bound_is_zero_overhead():
    q = 4.25 * MIB
    for v in (1 * MIB, 16 * MIB, 128 * MIB):
        for gap in (0.0, 1e-6, 1e-5, 1e-4):
            rate_ok, cap_ok = M.design_test(v, R, T0, q, gap)
            assert rate_ok == (M.issue_overhead(v, R, T0, gap) == 0.0)
            assert cap_ok == (M.isolated_issue_time(v, R, T0, q) == T0)
