"""Phase accounting of a per-tile trace (mixture_experts_ffn_dispatch_amd.tracing) on a
hand-built trace whose phases are known."""
import numpy as np
import pytest

from mixture_experts_ffn_dispatch_amd import _lib, tracing


def rec(task, wg, t):
    r = np.zeros(1, _lib.TRACE_DTYPE)
    r["task"], r["workgroup"] = task, wg
    for name, v in zip(("t_claim", "t_claimed", "t_start", "t_epilogue", "t_end", "t_release"), t):
        r[name] = v
    return r


def test_phases_of_a_hand_built_trace():
    l2 = np.int32(-(1 << 31) | (3 << 12))  # Linear-2, m-block 3, n-tile 0
    tr = np.concatenate([
        # workgroup 0: a Linear-1 tile 0..100 (claim 10, main 80, epilogue 10), then 20 between,
        # then a Linear-2 tile 120..200 (claim 5, wait 15, main 50, epilogue 10)
        rec(0, 0, (0, 10, 10, 90, 100, 110)),
        rec(l2, 0, (120, 125, 140, 190, 200, 0)),
        # workgroup 1: idle 50, a Linear-1 tile 50..150, idle 50 to the span's end at 200
        rec(1, 1, (50, 60, 60, 140, 150, 160)),
        np.full(2, -1, np.int32).view(np.uint8).repeat(32).view(_lib.TRACE_DTYPE)[:2],  # untouched slots
    ])
    tr["task"][-2:] = -1
    ph = tracing.tile_phases(tr, clock_hz=1e6)  # one tick = 1 us
    assert ph["span_us"] == 200 and ph["workgroups"] == 2 and ph["tiles"] == 3
    f = ph["fractions"]
    whole = 400.0
    assert f["claim"] == pytest.approx(25 / whole)
    assert f["wait"] == pytest.approx(15 / whole)
    assert f["mainloop"] == pytest.approx((80 + 50 + 80) / whole)
    assert f["epilogue"] == pytest.approx(30 / whole)
    assert f["between"] == pytest.approx(20 / whole)
    assert f["idle"] == pytest.approx(100 / whole)
    assert sum(f.values()) == pytest.approx(1.0)
    assert ph["linear2_us"]["wait"] == pytest.approx(15)
    assert "Linear-2" in tracing.format_phases("t", ph)
