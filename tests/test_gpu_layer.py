"""moe_layer, the whole layer in one kernel launch: routing, plan, A, Yd and the output are
byte-identical to moe_plan + moe_forward_gather + moe_combine (the same arithmetic), over tile
heights, expert counts, ragged token counts, repeated launches on one workspace and the five
named workloads at full size; a bounded wait that expires (forced from the host) is reported
and the next launch is clean."""
import numpy as np
import pytest
import torch

import moe_workloads as W
from oracle import moe_ref as R
from tests.gpu_util import Device, assert_close_rel, fetch, make_cfg, note, run

import mixture_experts_ffn_dispatch_amd as moe

pytestmark = pytest.mark.gpu

KEYS = ("topk_ids", "topk_w", "counts", "offsets", "perm", "pos", "act", "yd", "out")


def fused(cfg, dev, bufs=None, check=True):
    b = bufs or moe.alloc_buffers(cfg, xd=False)
    moe.run_layer(cfg, b, dev.x, dev.logits, dev.w1, dev.w2, fused=True)
    if check:
        st = moe.moe_status_read(b["ws"])
        assert st == moe.MOE_OK, moe.strerror(st)
    torch.cuda.synchronize()
    return b


def same(got, ref, what=""):
    g, r = fetch(got, KEYS), fetch(ref, KEYS)
    for key in KEYS:
        assert np.array_equal(g[key], r[key]), f"{what}: {key} differs from the separate calls"


SHAPES = [
    # (T, H, I, E, k, W, tile_m, flags)
    (300, 512, 384, 8, 2, 2, 0, 0),          # 128-row tiles? (auto), E <= 8 routing
    (513, 256, 192, 16, 4, 4, 32, 0),        # 32-row tiles, ragged T
    (700, 512, 320, 12, 3, 3, 64, 0),        # 64-row tiles, N tail
    (1000, 384, 256, 24, 6, 4, 128, 0),      # 128-row tiles
    (2048, 512, 256, 16, 4, 2, 256, 0),      # 256-row tiles
    (1024, 256, 128, 8, 2, 2, 256, moe.MOE_FLAG_WIDE_TAILS),  # wide last m-blocks
    (64, 128, 64, 1, 1, 1, 0, 0),            # one expert
    (200, 256, 128, 72, 5, 8, 0, 0),         # E in (64, 128]: 2 logits per lane
    (256, 128, 64, 1024, 32, 16, 0, 0),      # the largest E and k, 64 expert waves
    (1, 128, 64, 4, 2, 1, 0, 0),             # one token
]


@pytest.mark.parametrize("shape", SHAPES)
@pytest.mark.parametrize("schedule", [moe.MOE_SCHED_AUTO, moe.MOE_SCHED_EXPERT_WAVE])
def test_single_launch_equals_separate_calls(shape, schedule):
    T, H, I, E, k, Wv, tile_m, flags = shape
    s = W.shape(T=T, H=H, I=I, E=E, k=k, experts_per_wave=Wv, seed=500 + T + E)
    note(f"single launch: {W.describe(s)} tile_m {tile_m} flags {flags} schedule {schedule}")
    dev = Device(W.generate(s))
    cfg = make_cfg(s, schedule=schedule, tile_m=tile_m, flags=flags)
    got = fused(cfg, dev)
    ref = run(make_cfg(s, schedule=schedule, tile_m=tile_m, flags=flags), dev, gather=True)
    same(got, ref, str(shape))
    # again on the same workspace: the phase counters were left at zero
    got2 = fused(cfg, dev, bufs=got)
    same(got2, ref, f"{shape}, second launch")


def test_single_launch_against_the_oracle():
    s = W.shape(T=777, H=512, I=384, E=10, k=3, experts_per_wave=2, seed=99)
    d = W.generate(s)
    got = fetch(fused(make_cfg(s, schedule=moe.MOE_SCHED_AUTO), Device(d)), KEYS)
    o = R.moe_layer(d["x"], d["logits"], d["w1"], d["w2"], s.k)
    np.testing.assert_array_equal(got["topk_ids"], o["ids"])
    np.testing.assert_array_equal(got["perm"], o["perm"])
    assert_close_rel(got["act"], o["a"], what="A")
    assert_close_rel(got["yd"], o["yd"], what="Yd")
    assert_close_rel(got["out"], o["out"], what="out")


@pytest.mark.parametrize("name", ["tiny", "dsv3_share", "qwen3_30b_a3b", "small_m_zipf", "dit_batch"])
def test_single_launch_full_size(name):
    s = W.shape(name)
    note(f"single launch, full size {W.describe(s)}")
    dev = Device(W.generate(s))
    got = fused(make_cfg(s, schedule=moe.MOE_SCHED_AUTO), dev)
    ref = run(make_cfg(s, schedule=moe.MOE_SCHED_AUTO), dev, gather=True)
    same(got, ref, name)


def test_expired_wait_is_reported_and_the_next_launch_is_clean():
    # every Linear-2 tile waits for a Linear-1 completion that never comes (forced from the
    # host) with a small spin limit: the kernel exits with MOE_ERR_TIMEOUT, and a normal launch
    # on the same workspace afterwards gives the separate calls' bytes
    s = W.shape(T=512, H=256, I=128, E=8, k=2, experts_per_wave=2, seed=5)
    dev = Device(W.generate(s))
    cfg_t = make_cfg(s, schedule=moe.MOE_SCHED_AUTO, flags=moe.MOE_FLAG_FORCE_WAIT_TIMEOUT, spin_limit=2000)
    b = fused(cfg_t, dev, check=False)
    assert moe.moe_status_read(b["ws"]) == moe.MOE_ERR_TIMEOUT
    cfg = make_cfg(s, schedule=moe.MOE_SCHED_AUTO)
    got = fused(cfg, dev, bufs=b)
    same(got, run(make_cfg(s, schedule=moe.MOE_SCHED_AUTO), dev, gather=True), "after a timeout")
