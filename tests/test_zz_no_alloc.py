"""moe_layer_noalloc: the layer with the library's static workspace array (for callers that
cannot allocate) against the existing entry points (moe_plan, moe_forward_gather,
moe_combine on a caller workspace), which run the same kernels: routing, A, Yd and the output
must be byte-identical, on two calls in a row, the second with a smaller input (the array keeps
the first call's contents). The first input is also checked against the oracle."""
import numpy as np
import pytest
import torch

import moe_workloads as W
from oracle import moe_ref as R
from tests.gpu_util import Device, assert_close_rel, fetch, make_cfg, note, run

import mixture_experts_ffn_dispatch_amd as moe

pytestmark = pytest.mark.gpu

KEYS = ("topk_ids", "topk_w", "counts", "offsets", "perm", "pos", "act", "yd", "out")


def noalloc(cfg, dev):
    b = moe.alloc_buffers(cfg, xd=False)
    for key in ("act", "yd", "out"):
        b[key].fill_(float("nan"))
    status = torch.full((1,), 12345, dtype=torch.int32, device="cuda")
    moe.moe_layer_noalloc(cfg, dev.logits, b, dev.x, dev.w1, dev.w2, b["act"], b["yd"], b["out"], status)
    torch.cuda.synchronize()
    assert int(status.item()) == moe.MOE_OK
    return b


@pytest.mark.parametrize("schedule", [moe.MOE_SCHED_INTERLEAVED, moe.MOE_SCHED_EXPERT_WAVE])
def test_noalloc_matches_the_caller_workspace_path(schedule):
    shapes = [W.shape(T=700, H=512, I=384, E=12, k=3, experts_per_wave=4, seed=31),
              W.shape(T=130, H=256, I=192, E=6, k=2, experts_per_wave=2, seed=32)]
    for i, s in enumerate(shapes):
        note(f"no-alloc call {i}: {W.describe(s)}")
        d = W.generate(s)
        dev = Device(d)
        cfg = make_cfg(s, schedule=schedule)
        got = fetch(noalloc(cfg, dev), KEYS)
        ref = fetch(run(cfg, dev, gather=True), KEYS)
        for key in KEYS:
            assert np.array_equal(got[key], ref[key]), f"call {i}: {key} differs from the caller-workspace path"
        if i == 0:
            o = R.moe_layer(d["x"], d["logits"], d["w1"], d["w2"], s.k)
            np.testing.assert_array_equal(got["perm"], o["perm"])
            assert_close_rel(got["out"], o["out"], what="out vs oracle")


def test_noalloc_rejects_a_workspace_above_the_array():
    # 2^23 dispatched rows in 32-row tiles need about 20 MiB of workspace, above the static
    # array: refused on the host before anything is launched
    cfg = moe.MoeConfig(T=1 << 20, H=64, I=64, E=256, k=8, experts_per_wave=8, tile_m=32)
    assert moe.moe_workspace_size(cfg) > moe.MOE_STATIC_WORKSPACE_BYTES
    dummy = torch.empty(16, dtype=torch.int32, device="cuda")
    rt = {k: dummy for k in ("topk_ids", "topk_w", "counts", "offsets", "perm", "pos")}
    with pytest.raises(moe.MoeError) as ei:
        moe.moe_layer_noalloc(cfg, dummy, rt, dummy, dummy, dummy, dummy, dummy, dummy)
    assert ei.value.status == moe.MOE_ERR_WORKSPACE
