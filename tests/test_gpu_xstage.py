"""The Burst-Gap microbenchmark on the GPU (X-Stage paper, Section 3, as its local-memory
control): invariants of the recorded times, and a calibration whose max law predicts the
measured periods. The fitted values themselves are hardware properties, so only their ranges
are checked (values are reported by `python -m mixture_experts_ffn_dispatch_amd.xstage`)."""
import numpy as np
import pytest
import torch

import mixture_experts_ffn_dispatch_amd as moe
from mixture_experts_ffn_dispatch_amd import xstage as X
from oracle import burst_gap as BG
from tests.gpu_util import note

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def bench():
    return X.Bench(buf_bytes=512 << 20)


def test_times_are_ordered_and_gaps_respected(bench):
    note("burst-gap invariants")
    k, b, p, gap = min(64, bench.cus), 64 * 1024, 12, 5e-6
    issue, period = bench.run(k, b, p, gap)
    assert issue.shape == (k, p) and period.shape == (k, p - 1)
    assert np.all(issue >= 0)
    # a period holds its issue and at least the requested gap (counter resolution aside)
    tick = 1.0 / bench.hz
    assert np.all(period >= issue[:, :-1] + gap - 2 * tick)


def test_counter_clock_matches_events(bench):
    note("burst-gap clock vs events")
    times = torch.empty(16 * 20 * 2, dtype=torch.int64, device="cuda")
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    moe.moe_burst_gap(16, 4096, 20, int(20e-6 * bench.hz), bench.buf, times)
    e1.record()
    torch.cuda.synchronize()
    t = times.cpu().numpy().reshape(16, 20, 2)
    span = (t[:, -1, 1].max() - t[:, 0, 0].min()) / bench.hz
    assert span >= 19 * 20e-6
    assert span <= e0.elapsed_time(e1) * 1e-3 * 1.05 + 5e-6


def test_invalid_configurations_rejected(bench):
    times = torch.empty(64, dtype=torch.int64, device="cuda")
    for k, b, p, g in ((0, 4096, 1, 0), (bench.cus + 1, 4096, 1, 0), (1, 4000, 1, 0), (1, 4096, 0, 0),
                       (1, 4096, 1, -1), (1, 4096, 1, 10 ** 7), (2, 1 << 30, 1, 0)):
        with pytest.raises(moe.MoeError):
            moe.moe_burst_gap(k, b, p, g, bench.buf, times)


def test_periodic_max_law_on_this_gpu(bench):
    # Section 3's periodic steady state against the oracle's equations (oracle/burst_gap.py,
    # pinned to the paper's worked numbers). The drain rate comes from the mean period of the
    # three gaps on the drain branch, t_iss0 from the two on the issue plateau; every period,
    # the corner included, must follow max(V / R, t_iss0 + G) within 10% (the whole-sweep
    # calibration fits it within 4%: profiles/xstage_local_memory_calibration.txt)
    note("burst-gap gap sweep")
    k, b = bench.cus, 128 * 1024
    v = k * b
    _, per_0gap = bench.periodic(k, b, 0.0)
    fracs = np.array([0.0, 0.25, 0.5, 1.0, 2.0, 4.0])
    gaps = fracs * per_0gap
    meas = [bench.periodic(k, b, float(g)) for g in gaps]
    r = v / np.mean([per for (_, per) in meas[:3]])
    assert 0.5e12 < r < 20e12  # bytes per second to this GPU's memory
    t_iss0 = float(np.mean([t for (t, _) in meas[-2:]]))
    for g, (t_iss, per) in zip(gaps, meas):
        pred_per = float(BG.period(v, r, t_iss0, g))
        pred_iss = float(BG.issue_time(v, r, t_iss0, g))
        note(f"  gap {g * 1e6:.3f} us: period {per * 1e6:.3f} us (model {pred_per * 1e6:.3f}), "
             f"issue {t_iss * 1e6:.3f} us (model {pred_iss * 1e6:.3f})")
        assert per == pytest.approx(pred_per, rel=0.10), (g, per, pred_per)
    # on the drain branch the issue time falls one for one with the gap (issue + gap = V / R),
    # and beyond the recovery gap it sits on its plateau
    for g, (t_iss, _) in zip(gaps[:3], meas[:3]):
        assert t_iss + g == pytest.approx(v / r, rel=0.10)
    assert meas[-1][0] == pytest.approx(meas[-2][0], rel=0.15)
