"""Progress of the persistent GEMM without every locality group resident: with
MOE_FLAG_TEST_ABSENT_GROUP the workgroups of group 0 take no tile (as if a kernel running
concurrently kept their XCD busy). The other groups must run every tile, group 0's list
included, through the deferral of Linear-2 tiles that wait too long and the compare-and-swap
claims of runnable records; the bytes equal a normal run's and no wait expires. The trace shows
that no workgroup of group 0 ran a tile."""
import numpy as np
import pytest
import torch

import moe_workloads as W
from tests.gpu_util import Device, make_cfg, note, run
from tests.test_gpu_trace import NOP, plan_records

import mixture_experts_ffn_dispatch_amd as moe
from mixture_experts_ffn_dispatch_amd import _lib

pytestmark = pytest.mark.gpu

OUTPUTS = ("act", "yd", "out")


def bits(t):
    return t.view(torch.int16)


@pytest.mark.parametrize("name,schedule", [
    ("dsv3_share", moe.MOE_SCHED_AUTO),
    ("dsv3_share", moe.MOE_SCHED_EXPERT_WAVE),
    ("qwen3_30b_a3b", moe.MOE_SCHED_AUTO),
    ("small_m_zipf", moe.MOE_SCHED_INTERLEAVED),
    ("tiny", moe.MOE_SCHED_AUTO),
])
def test_absent_group_still_runs_every_tile(name, schedule):
    s = W.shape(name)
    dev = Device(W.generate(s))
    ref = run(make_cfg(s, schedule=schedule), dev, gather=True)
    cfg = make_cfg(s, schedule=schedule, flags=moe.MOE_FLAG_TEST_ABSENT_GROUP)
    note(f"absent group 0: {name} schedule {schedule}")
    L = moe.moe_workspace_layout(cfg)
    trace = torch.full((L["max_slots"] * 64,), 0xFF, dtype=torch.uint8, device="cuda")
    cfg.trace = trace
    b = run(cfg, dev, gather=True)  # asserts MOE_OK: no wait expired
    cfg.trace = None
    for key in OUTPUTS:
        assert torch.equal(bits(b[key]), bits(ref[key])), key
    tr = trace.cpu().numpy().view(_lib.TRACE_DTYPE)
    recs, goff, hdr = plan_records(b, L)
    runs = recs[:, 0] != NOP
    ran = tr[:len(recs)]
    assert np.array_equal(ran["task"][runs], recs[runs, 0]), "a tile did not run exactly once"
    assert np.all(ran["workgroup"][runs] % 8 != 0), "a workgroup of the absent group ran a tile"
    g0 = np.zeros(len(recs), bool)
    g0[goff[0]:goff[1]] = True
    assert np.any(runs & g0), "group 0's list is empty"
    # and a normal run afterwards on the same buffers is clean
    b2 = run(make_cfg(s, schedule=schedule), dev, bufs=b, gather=True)
    for key in OUTPUTS:
        assert torch.equal(bits(b2[key]), bits(ref[key])), key


def test_absent_group_single_launch():
    s = W.shape("qwen3_30b_a3b")
    dev = Device(W.generate(s))
    ref = run(make_cfg(s, schedule=moe.MOE_SCHED_AUTO), dev, gather=True)
    cfg = make_cfg(s, schedule=moe.MOE_SCHED_AUTO, flags=moe.MOE_FLAG_TEST_ABSENT_GROUP)
    b = moe.alloc_buffers(cfg, xd=False)
    moe.run_layer(cfg, b, dev.x, dev.logits, dev.w1, dev.w2, gather=True, fused=True)
    torch.cuda.synchronize()
    assert moe.moe_status_read(b["ws"]) == moe.MOE_OK
    for key in OUTPUTS:
        assert torch.equal(bits(b[key]), bits(ref[key])), key
