"""The Burst-Gap microbenchmark on the GPU (X-Stage paper, Section 3, as its local-memory
control): invariants of the recorded times, and a calibration whose max law predicts the
measured periods. The fitted values themselves are hardware properties, so only their ranges
are checked (values are reported by `python -m mixture_experts_ffn_dispatch_amd.xstage`)."""
import numpy as np
import pytest
import torch

import mixture_experts_ffn_dispatch_amd as moe
from mixture_experts_ffn_dispatch_amd import xstage as X
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
    note("burst-gap gap sweep")
    k, b = bench.cus, 128 * 1024
    pts = [bench.periodic(k, b, 0.0)]
    t_iss_0gap, per_0gap = pts[0]
    r = k * b / per_0gap
    assert 0.5e12 < r < 20e12  # bytes per second to this GPU's memory
    gaps = np.array([0.5, 1.0, 2.0, 4.0]) * per_0gap
    meas = [bench.periodic(k, b, float(g)) for g in gaps]
    t_iss0 = meas[-1][0]
    for g, (t_iss, per) in zip(gaps, meas):
        pred = X.predict_period(k * b, r, t_iss0, g)
        assert per == pytest.approx(float(pred), rel=0.35), (g, per, pred)
