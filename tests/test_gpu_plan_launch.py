"""moe_plan in one launch (MOE_FLAG_PLAN_ONE_LAUNCH: route, scan and schedule, scatter with a
grid barrier) against the same steps as three launches (the default): the routing arrays and
the whole workspace are byte-identical, repeated plans on one workspace give the same bytes
(the barrier counters are back at zero after every launch), and the routing equals the
oracle's."""
import numpy as np
import pytest
import torch

import moe_workloads as W
from oracle import moe_ref as R
from tests.gpu_util import make_cfg, note

import mixture_experts_ffn_dispatch_amd as moe

pytestmark = pytest.mark.gpu

ROUTING = ("topk_ids", "topk_w", "counts", "offsets", "perm", "pos")

SHAPES = [
    ("tiny", {}),
    ("small_m_zipf", {}),
    ("qwen3_30b_a3b", {}),
    ("dsv3_share", {}),
    ("dit_batch", {}),
    ("T1", dict(T=1, H=256, I=256, E=8, k=2, experts_per_wave=1, seed=5)),
    ("T513", dict(T=513, H=256, I=256, E=12, k=3, experts_per_wave=4, seed=6)),
    ("E1024k32", dict(T=300, H=256, I=256, E=1024, k=32, experts_per_wave=16, seed=7)),
    ("E100w1", dict(T=2000, H=256, I=256, E=100, k=4, experts_per_wave=1, seed=8)),
]


def plan_bytes(cfg, logits):
    b = moe.alloc_buffers(cfg, xd=False)
    moe.moe_plan(cfg, logits, b, b["ws"])
    torch.cuda.synchronize()
    assert moe.moe_status_read(b["ws"]) == moe.MOE_OK
    return b


@pytest.mark.parametrize("name,kw", SHAPES, ids=[s[0] for s in SHAPES])
@pytest.mark.parametrize("schedule", [moe.MOE_SCHED_AUTO, moe.MOE_SCHED_EXPERT_WAVE])
def test_one_launch_equals_three_launches(name, kw, schedule):
    s = W.shape(name) if not kw else W.shape(**kw)
    d = W.generate(s, parts=("logits",))
    logits = torch.from_numpy(np.ascontiguousarray(d["logits"])).cuda()
    note(f"plan one launch vs three: {name} T={s.T} E={s.E} k={s.k} schedule={schedule}")
    one = plan_bytes(make_cfg(s, schedule=schedule, flags=moe.MOE_FLAG_PLAN_ONE_LAUNCH), logits)
    three = plan_bytes(make_cfg(s, schedule=schedule), logits)
    for key in ROUTING:
        assert torch.equal(one[key], three[key]), key
    if not torch.equal(one["ws"], three["ws"]):
        L = moe.moe_workspace_layout(make_cfg(s, schedule=schedule))
        regions = sorted((v, k) for k, v in L.items() if k in (
            "header", "layer_sync", "chunk_counts", "mblk_expert", "mblk_row0", "mblk_rows", "mblk_ready",
            "tasks", "unit_start", "group_units", "group_tasks", "wave_table"))
        diff = torch.nonzero(one["ws"] != three["ws"]).flatten().cpu().numpy()
        names = sorted({[k for v, k in regions if v <= o][-1] for o in diff})
        first = int(diff[0])
        a = one["ws"][first & ~3:(first & ~3) + 64].cpu().numpy().view(np.int32)
        b = three["ws"][first & ~3:(first & ~3) + 64].cpu().numpy().view(np.int32)
        raise AssertionError(f"workspace differs in {names} ({diff.size} bytes, first at {first}): {a} vs {b}")
    # the routing is the oracle's
    ids, w = R.route(d["logits"], s.k)
    assert np.array_equal(one["topk_ids"].cpu().numpy(), ids)
    _, _, perm, pos = R.plan(ids, s.E)
    assert np.array_equal(one["perm"].cpu().numpy(), perm)
    assert np.array_equal(one["pos"].cpu().numpy(), pos)


def test_repeated_plans_on_one_workspace():
    s = W.shape("qwen3_30b_a3b")
    d = W.generate(s, parts=("logits",))
    logits = torch.from_numpy(np.ascontiguousarray(d["logits"])).cuda()
    cfg = make_cfg(s, schedule=moe.MOE_SCHED_AUTO, flags=moe.MOE_FLAG_PLAN_ONE_LAUNCH)
    b = plan_bytes(cfg, logits)
    first = b["ws"].clone()
    L = moe.moe_workspace_layout(cfg)
    sync = b["ws"][L["layer_sync"]:L["layer_sync"] + 4096]
    assert not sync.any(), "barrier counters left non-zero"
    for _ in range(3):
        moe.moe_plan(cfg, logits, b, b["ws"])
    torch.cuda.synchronize()
    assert torch.equal(b["ws"], first)
    # a smaller config on the same workspace, then the first again
    s2 = W.shape(T=700, H=s.H, I=s.I, E=s.E, k=s.k, experts_per_wave=s.experts_per_wave, seed=11)
    d2 = W.generate(s2, parts=("logits",))
    cfg2 = make_cfg(s2, schedule=moe.MOE_SCHED_AUTO, flags=moe.MOE_FLAG_PLAN_ONE_LAUNCH)
    logits2 = torch.from_numpy(d2["logits"]).cuda()
    ref2 = plan_bytes(cfg2, logits2)
    b2 = {key: torch.empty_like(ref2[key]) for key in ROUTING}
    moe.moe_plan(cfg2, logits2, b2, b["ws"])
    torch.cuda.synchronize()
    assert moe.moe_status_read(b["ws"]) == moe.MOE_OK
    for key in ROUTING:
        assert torch.equal(b2[key], ref2[key]), key
    assert not sync.any()
    moe.moe_plan(cfg, logits, b, b["ws"])
    torch.cuda.synchronize()
    assert moe.moe_status_read(b["ws"]) == moe.MOE_OK
    # the header (list bounds, counts, the chosen order) and the counters are as after the
    # first plan; the other regions may keep the smaller plan's bytes past what this one uses
    assert torch.equal(b["ws"][:256], first[:256])
    assert not sync.any()
