"""The MOE_SCHED_AUTO rule's host model on the CPU: what it picks for the named workloads with
this GPU's own memory as the store path, and with a slow link (the pages' remote path), and
that its X-Stage part is the Burst-Gap oracle's arithmetic."""
import numpy as np
import pytest

import moe_workloads as W
from oracle import burst_gap as BG
from oracle import moe_ref as R
from tests.auto_rule import auto_choice, calibration

GRID = 256  # resident workgroups of the 256-row kernel on 256 CUs


def counts_of(name):
    s = W.shape(name)
    d = W.generate(s)
    ids, _ = R.route(d["logits"], s.k)
    return s, R.plan(ids, s.E)[0]


@pytest.mark.parametrize("name", ["dsv3_share", "qwen3_30b_a3b"])
def test_local_memory_path_picks_every_linear1_tile_first(name):
    # stores to this GPU's own memory never backpressure (6.6 TB/s drain, 31 MiB capacity),
    # the Expert-Wave order pays a dependency stall per wave, and no lead keeps more than the
    # cache holds: every interleaved lead that meets the dependency costs nothing, and the
    # largest wins the tie
    s, counts = counts_of(name)
    sched, lead, prices = auto_choice(counts, s.experts_per_wave, s.H, s.I, 256, -(-s.I // 128),
                                      -(-s.H // 256), GRID, calibration())
    assert sched == 1 and lead == s.waves
    assert prices[0] > 0 and prices[lead] == 0.0


def test_slow_link_avoids_leaving_linear2_bursts_without_gaps():
    # the pages' remote path (R = 717 GB/s, t_iss0 = 0.76 us, Q = 4.25 MiB): 256 aligned
    # 128 KiB Yd bursts (32 MiB) take 47 us to drain against a ~60 us Linear-2 main loop on
    # dsv3_share, beyond the capacity. With every Linear-1 tile first (lead = waves) the
    # Linear-2 tiles run back to back with no Linear-1 work between their bursts, so the rule
    # must price that lead above a shorter one and pick a lead below the wave count
    s, counts = counts_of("dsv3_share")
    calib = calibration(0.76, 717.0, 4.25)
    sched, lead, prices = auto_choice(counts, s.experts_per_wave, s.H, s.I, 256, 16, 28, GRID, calib)
    assert sched == 1 and lead < s.waves
    assert prices[s.waves] > prices[lead] and prices[0] > prices[lead]


def test_burst_issue_time_is_the_oracle_max_law():
    # one wave, one burst of 256 tiles: the price is the oracle's issue overhead (the drain
    # backlog beyond the gap) plus the capacity branch, nothing else (dependency stall of a
    # single wave aside)
    T0, Rr, Q = calibration(0.76, 717.0, 4.25)
    counts = [256 * 256]  # one expert, 256 m-blocks of 256 rows
    H, I = 1024, 1024
    sched, lead, prices = auto_choice(counts, 1, H, I, 256, 8, 4, 256, (T0, Rr, Q))
    t2 = 256 * max(2.0 * 256 * 256 * I / 1.2e15, 512.0 * I / 5.0e12)
    t1 = 256 * max(2.0 * 256 * 256 * H / 1.2e15, 512.0 * H / 5.0e12)
    V = 256 * 256 * 256 * 2.0
    T = max(float(BG.issue_time(V, Rr, T0, t2)), float(BG.isolated_issue_time(V, Rr, T0, Q)))
    assert prices[0] == pytest.approx((4 * 256 / 256) * (T - T0) + t1 / 2.0, rel=1e-12)
