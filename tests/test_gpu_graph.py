"""The layer captured into a HIP graph and replayed: plan + forward (gather) + combine on a
caller workspace, and moe_layer_noalloc (the entry point for callers that cannot allocate,
such as code under graph capture). New inputs are copied into the captured buffers between
replays, with eager work and synchronisation in between; every replay must give the bytes of
an eager run on the same inputs (the kernels reset their own counters, so nothing has to be
cleared between replays)."""
import numpy as np
import pytest
import torch

import moe_workloads as W
from tests.gpu_util import Device, make_cfg, note, run

import mixture_experts_ffn_dispatch_amd as moe

pytestmark = pytest.mark.gpu

OUT = ("topk_ids", "perm", "act", "yd", "out")


def bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t


def shapes():
    return [W.shape(T=700, H=512, I=384, E=12, k=3, experts_per_wave=4, seed=51),
            W.shape("tiny")]


@pytest.mark.parametrize("noalloc", [False, True])
@pytest.mark.parametrize("si", [0, 1])
def test_graph_replays_match_eager_runs(noalloc, si):
    s = shapes()[si]
    cfg = make_cfg(s, schedule=moe.MOE_SCHED_AUTO)
    inputs = [Device(W.generate(W.shape(T=s.T, H=s.H, I=s.I, E=s.E, k=s.k, experts_per_wave=s.experts_per_wave,
                                        seed=s.seed + 100 * r))) for r in range(3)]
    dev = Device(W.generate(s))  # the captured buffers (inputs are copied in before each replay)
    b = moe.alloc_buffers(cfg, xd=False)
    status = torch.zeros((1,), dtype=torch.int32, device="cuda")

    def layer():
        if noalloc:
            moe.moe_layer_noalloc(cfg, dev.logits, b, dev.x, dev.w1, dev.w2, b["act"], b["yd"], b["out"], status)
        else:
            moe.run_layer(cfg, b, dev.x, dev.logits, dev.w1, dev.w2, gather=True)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        layer()  # warm-up outside the capture (the no-alloc array's address is looked up here)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        layer()
    torch.cuda.synchronize()
    for r, src in enumerate(inputs):
        note(f"graph replay {r}: noalloc={noalloc} {W.describe(s)}")
        for name in ("x", "logits", "w1", "w2"):
            getattr(dev, name).copy_(getattr(src, name))
        for key in ("act", "yd", "out"):
            b[key].fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        if noalloc:
            assert int(status.item()) == moe.MOE_OK
        else:
            assert moe.moe_status_read(b["ws"]) == moe.MOE_OK
        ref = run(cfg, src, gather=True)  # eager, on buffers of its own
        for key in OUT:
            assert torch.equal(bits(b[key]), bits(ref[key])), (r, key)
