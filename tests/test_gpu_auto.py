"""MOE_SCHED_AUTO on the GPU: the order and lead moe_plan records equal the host model of the
rule (tests/auto_rule.py, from the oracle's routed counts and the plan's grid) for the named
workloads under three calibrations, and the outputs equal both fixed orders' bytes."""
import numpy as np
import pytest
import torch

import moe_workloads as W
from oracle import moe_ref as R
from tests.auto_rule import auto_choice, calibration
from tests.gpu_util import Device, make_cfg, note, run

import mixture_experts_ffn_dispatch_amd as moe

pytestmark = pytest.mark.gpu

CALIBRATIONS = [(0.0, 0.0, 0.0), (0.76, 717.0, 4.25), (0.93, 150.0, 4.0)]


def plan_header(b):
    return b["ws"][:256].cpu().numpy().view(np.int32)


@pytest.mark.parametrize("name", ["tiny", "dsv3_share", "qwen3_30b_a3b", "small_m_zipf", "dit_batch"])
def test_auto_choice_matches_the_host_model(name):
    s = W.shape(name)
    d = W.generate(s)
    dev = Device(d)
    ids, _ = R.route(d["logits"], s.k)
    counts = R.plan(ids, s.E)[0]
    for cal in CALIBRATIONS:
        cfg = make_cfg(s, schedule=moe.MOE_SCHED_AUTO, xs_issue_us=cal[0], xs_drain_gbps=cal[1],
                       xs_capacity_mib=cal[2])
        b = moe.alloc_buffers(cfg, xd=False)
        moe.moe_plan(cfg, dev.logits, b, b["ws"])
        torch.cuda.synchronize()
        hdr = plan_header(b)
        L = moe.moe_workspace_layout(cfg)
        sched, lead, prices = auto_choice(counts, s.experts_per_wave, s.H, s.I, L["tile_m"], L["n1_tiles"],
                                          L["n2_tiles"], int(hdr[27]), calibration(*cal))
        note(f"{name} calibration {cal}: device order {hdr[28]} lead {hdr[26]}, model {sched} lead {lead}")
        assert int(hdr[28]) == (moe.MOE_SCHED_INTERLEAVED if sched else moe.MOE_SCHED_EXPERT_WAVE)
        assert int(hdr[26]) == lead


@pytest.mark.parametrize("cal", CALIBRATIONS[:2])
def test_auto_outputs_equal_both_fixed_orders(cal):
    # a mid-size shape with several waves, so the orders differ; the bytes may not
    s = W.shape(T=2048, H=1024, I=512, E=16, k=4, experts_per_wave=2, seed=77)
    dev = Device(W.generate(s))
    auto = run(make_cfg(s, schedule=moe.MOE_SCHED_AUTO, xs_issue_us=cal[0], xs_drain_gbps=cal[1],
                        xs_capacity_mib=cal[2]), dev, gather=True)
    for sched in (moe.MOE_SCHED_EXPERT_WAVE, moe.MOE_SCHED_INTERLEAVED):
        ref = run(make_cfg(s, schedule=sched), dev, gather=True)
        for key in ("topk_ids", "perm", "act", "yd", "out"):
            assert torch.equal(auto[key].view(torch.int16) if auto[key].dtype == torch.bfloat16 else auto[key],
                               ref[key].view(torch.int16) if ref[key].dtype == torch.bfloat16 else ref[key]), key
    # the plan's tile list is dependency-safe for the order it chose
    hdr = plan_header(auto)
    assert int(hdr[28]) in (moe.MOE_SCHED_EXPERT_WAVE, moe.MOE_SCHED_INTERLEAVED)


@pytest.mark.parametrize("E,W_", [(31, 1), (62, 2), (40, 1), (80, 1)])
def test_auto_choice_at_many_waves(E, W_):
    # 31 waves: every (lead, wave) term on a lane of its own; 40 waves: one lane per lead on
    # wavefront 0; 80 waves: the whole workgroup. With these sizes the remote calibrations
    # choose leads well below the number of waves, so the prices decide.
    s = W.shape(T=75 * E, H=4096, I=2048, E=E, k=8, experts_per_wave=W_, seed=90 + E)
    d = W.generate(s, parts=("logits",))
    logits = torch.from_numpy(d["logits"]).cuda()
    ids, _ = R.route(d["logits"], s.k)
    counts = R.plan(ids, s.E)[0]
    for cal in CALIBRATIONS:
        cfg = make_cfg(s, schedule=moe.MOE_SCHED_AUTO, xs_issue_us=cal[0], xs_drain_gbps=cal[1],
                       xs_capacity_mib=cal[2])
        b = moe.alloc_buffers(cfg, xd=False)
        moe.moe_plan(cfg, logits, b, b["ws"])
        torch.cuda.synchronize()
        hdr = plan_header(b)
        L = moe.moe_workspace_layout(cfg)
        sched, lead, _ = auto_choice(counts, W_, s.H, s.I, L["tile_m"], L["n1_tiles"], L["n2_tiles"],
                                     int(hdr[27]), calibration(*cal))
        note(f"E={E} W={W_} calibration {cal}: device order {hdr[28]} lead {hdr[26]}, model {sched} lead {lead}")
        assert int(hdr[28]) == (moe.MOE_SCHED_INTERLEAVED if sched else moe.MOE_SCHED_EXPERT_WAVE)
        assert int(hdr[26]) == lead
