"""GPU parity against the CPU oracle through the C ABI (MI355X).

Bars: routing ids, counts, offsets, perm, pos and the dispatched rows bit-exact; router
weights within 2^-20; A, Yd (per expert) and the layer output within
max|gpu - ref| <= 1e-2 * max|ref|; the exact-integer case bit-exact end to end.
"""
import numpy as np
import pytest
import torch

import moe_workloads as W
from oracle import invariants as V, moe_ref as R
from tests.gpu_util import Device, assert_close_rel, dev_bf16, fetch, host_bits, make_cfg, note, run

import mixture_experts_ffn_dispatch_amd as moe

pytestmark = pytest.mark.gpu


def check_routing(g, o):
    np.testing.assert_array_equal(g["topk_ids"], o["ids"])
    np.testing.assert_allclose(g["topk_w"], o["w"], rtol=0, atol=2.0 ** -20)
    np.testing.assert_array_equal(g["counts"], o["counts"])
    np.testing.assert_array_equal(g["offsets"], o["offsets"])
    np.testing.assert_array_equal(g["perm"], o["perm"])
    np.testing.assert_array_equal(g["pos"], o["pos"])


def check_full(g, o, xd_bits, E):
    check_routing(g, o)
    np.testing.assert_array_equal(xd_bits, o["xd"])
    assert_close_rel(g["act"], o["a"], what="A")
    for e in range(E):
        lo, hi = o["offsets"][e], o["offsets"][e + 1]
        if hi > lo:
            assert_close_rel(g["yd"][lo:hi], o["yd"][lo:hi], what=f"Yd expert {e}")
    assert_close_rel(g["out"], o["out"], what="out")


@pytest.mark.parametrize("k", [1, 2])
@pytest.mark.parametrize("tile_m", [32, 64, 128, 256])
@pytest.mark.parametrize("schedule", [moe.MOE_SCHED_EXPERT_WAVE, moe.MOE_SCHED_INTERLEAVED])
@pytest.mark.parametrize("gather", [False, True])
def test_exact_integer_case_bit_exact(k, tile_m, schedule, gather):
    note(f"exact-integer k={k} tile_m={tile_m} schedule={schedule} gather={gather}")
    c = V.exact_integer_case(T=100, H=256, I=192, E=4, k=k, seed=3)
    cfg = moe.MoeConfig(T=100, H=256, I=192, E=4, k=k, experts_per_wave=1, schedule=schedule, tile_m=tile_m)
    dev = Device(c)
    b = run(cfg, dev, gather=gather)
    g = fetch(b)
    ex = c["expected"]
    np.testing.assert_array_equal(g["topk_ids"], ex["ids"])
    np.testing.assert_array_equal(g["topk_w"], ex["w"])
    T = 100
    np.testing.assert_array_equal(g["act"][g["pos"]].reshape(T, k, -1), ex["a_tok"])
    np.testing.assert_array_equal(g["yd"][g["pos"]].reshape(T, k, -1), ex["y_tok"])
    np.testing.assert_array_equal(g["out"], ex["out"])


def test_tiny_workload_full_parity():
    s = W.shape("tiny")
    note(f"full parity {W.describe(s)}")
    d = W.generate(s)
    o = R.moe_layer(d["x"], d["logits"], d["w1"], d["w2"], s.k)
    b = run(make_cfg(s), Device(d))
    check_full(fetch(b), o, host_bits(b["xd"]), s.E)


SWEEP = [
    # T, H, I, E, k, W, tile_m   (ragged T, one expert, k = E, empty experts, N tails, small dims)
    (1, 64, 64, 1, 1, 1, 0),
    (37, 64, 64, 1, 1, 1, 32),
    (130, 192, 320, 5, 2, 2, 0),
    (257, 128, 64, 4, 4, 1, 64),
    (65, 320, 192, 16, 3, 3, 32),
    (300, 256, 384, 12, 1, 5, 128),
    (96, 64, 128, 64, 8, 8, 32),
    (200, 512, 256, 33, 5, 4, 256),
    (513, 128, 192, 3, 3, 1, 0),
    (150, 768, 320, 6, 2, 2, 256),  # 256-row tiles: wide last m-blocks, odd and partial n-tiles
    (300, 192, 384, 3, 1, 1, 256),
    (300, 64, 64, 1024, 32, 128, 0),  # the largest E and k the ABI accepts
    (129, 128, 64, 1000, 17, 125, 32),
    (300, 64, 64, 1024, 32, 1, 0),  # 1024 expert waves: the planner's workgroup-wide wave table
    (129, 128, 64, 100, 6, 1, 32),  # 100 expert waves
]


@pytest.mark.parametrize("T,H,I,E,k,Wv,tile_m", SWEEP)
@pytest.mark.parametrize("schedule", [moe.MOE_SCHED_EXPERT_WAVE, moe.MOE_SCHED_INTERLEAVED])
def test_shape_sweep_full_parity(T, H, I, E, k, Wv, tile_m, schedule):
    s = W.shape(T=T, H=H, I=I, E=E, k=k, experts_per_wave=Wv, seed=T * 31 + E, x_std=1.0, w_std=0.05)
    note(f"sweep {W.describe(s)} tile_m={tile_m} schedule={schedule}")
    d = W.generate(s)
    if E >= 16:  # leave some experts without rows
        d["logits"][:, E // 2:] -= 30.0
    o = R.moe_layer(d["x"], d["logits"], d["w1"], d["w2"], k)
    cfg = make_cfg(s, tile_m=tile_m, schedule=schedule)
    dev = Device(d)
    b = run(cfg, dev)
    check_full(fetch(b), o, host_bits(b["xd"]), E)
    if E >= 16:
        assert (o["counts"] == 0).any()
    # the dispatch folded into the Linear-1 loads gives the same bytes
    note("  gather path")
    bg = run(cfg, dev, gather=True)
    for key in ("act", "yd", "out"):
        assert torch.equal(b[key].view(torch.int16), bg[key].view(torch.int16)), key


# Odd numbers of 64-wide K steps, down to one, on the instances that three-buffer their weight
# rows (regular 256-row tiles, wide tails off, and 128-row tiles): the tail step after the
# loop's pairs, a step whose next two K steps lie past the end, and a single K step.
K_TAIL = [
    # T, H, I, E, k, tile_m  (K steps: H / 64 for Linear-1, I / 64 for Linear-2)
    (700, 64, 192, 3, 2, 256),    # 1 and 3
    (520, 320, 64, 2, 1, 256),    # 5 and 1
    (900, 192, 320, 4, 2, 256),   # 3 and 5, several m-blocks per expert
    (300, 64, 320, 4, 2, 128),    # 1 and 5
    (400, 448, 192, 6, 3, 128),   # 7 and 3
    (200, 192, 64, 4, 1, 256),    # 3 and 1; every expert one m-block (non-temporal weight rows)
    (120, 320, 192, 4, 2, 128),   # 5 and 3; every expert one m-block
]


@pytest.mark.parametrize("T,H,I,E,k,tile_m", K_TAIL)
def test_odd_k_steps_full_parity(T, H, I, E, k, tile_m):
    s = W.shape(T=T, H=H, I=I, E=E, k=k, experts_per_wave=1, seed=T + H + I, x_std=1.0, w_std=0.05)
    note(f"odd K steps {W.describe(s)} tile_m={tile_m}")
    d = W.generate(s)
    o = R.moe_layer(d["x"], d["logits"], d["w1"], d["w2"], k)
    cfg = make_cfg(s, tile_m=tile_m, schedule=moe.MOE_SCHED_INTERLEAVED, flags=moe.MOE_FLAG_NO_WIDE_TAILS)
    dev = Device(d)
    b = run(cfg, dev)
    check_full(fetch(b), o, host_bits(b["xd"]), E)
    bg = run(cfg, dev, gather=True)
    for key in ("act", "yd", "out"):
        assert torch.equal(b[key].view(torch.int16), bg[key].view(torch.int16)), key


def test_identical_experts_match_dense_ffn():
    s = W.shape(T=160, H=256, I=128, E=6, k=3, seed=21, x_std=1.0, w_std=0.05)
    note(f"identical experts {W.describe(s)}")
    d = W.generate(s)
    d["w1"], d["w2"] = V.identical_experts(d["x"], d["w1"][0], d["w2"][0], s.E)
    dense = V.dense_ffn(d["x"], d["w1"][0], d["w2"][0])
    b = run(make_cfg(s), Device(d))
    out = fetch(b, keys=("out",))["out"]
    ref = R.f64_to_bf16_bits(dense["y"])
    assert_close_rel(out, ref, what="identical experts vs dense FFN")


def test_top1_single_expert_matches_dense_ffn():
    s = W.shape(T=150, H=128, I=256, E=1, k=1, seed=22, x_std=1.0, w_std=0.05)
    note(f"top-1 E=1 {W.describe(s)}")
    d = W.generate(s)
    dense = V.dense_ffn(d["x"], d["w1"][0], d["w2"][0])
    b = run(make_cfg(s), Device(d))
    g = fetch(b, keys=("topk_w", "out"))
    assert np.all(g["topk_w"] == 1.0)
    assert_close_rel(g["out"], R.f64_to_bf16_bits(dense["y"]), what="E=1 top-1 vs dense FFN")


def tie_logits(T, E, k):
    """Logits full of ties: equal values, -0 against +0, ties between experts e and e + 16,
    e + 32 and e + 64 (one lane's logits in the 16-, 32- and 64-lane layouts), and rows where
    fewer than k logits are finite so that -inf logits are kept (lower ids first, weight 0)."""
    lg = np.zeros((T, E), np.float32)
    lg[1::2] = -0.0
    lg[::3, 5 % E] = 1.0
    lg[::5, 2 % E] = -0.0
    lg[::7] = np.float32(0.5)
    if E > 64:
        lg[::4, 3] = 2.0
        lg[::4, 67] = 2.0
        lg[1::4, E - 1] = 3.0
        lg[1::4, E - 65] = 3.0
        lg[3::8, 64:] = 4.0  # the lower block's ids lose to the higher block's larger logits
        lg[5::6, [20, 36, 52]] = 2.5
    lg[2::9] = -np.inf
    lg[2::9, : max(1, k // 2)] = np.float32(-1.0)
    return lg


@pytest.mark.parametrize("E,k", [(8, 3), (16, 5), (32, 8), (48, 7), (64, 6), (100, 8), (128, 8), (128, 16),
                                 (72, 32), (112, 17), (130, 5), (300, 12), (1024, 32)])
def test_routing_ties_and_signed_zero(E, k):
    # equal logits and -0/+0 must pick the lower expert id first, exactly like the oracle; the
    # shapes cover every route kernel (8- to 64-lane segments, 2 to 16 experts per lane) and
    # k up to 32 with 2 experts per lane
    T = 128
    lg = tie_logits(T, E, k)
    s = W.shape(T=T, H=64, I=64, E=E, k=k, seed=23)
    note(f"routing ties E={E} k={k}")
    d = W.generate(s, parts=("x", "w1", "w2"))
    d["logits"] = lg
    o = R.moe_layer(d["x"], lg, d["w1"], d["w2"], k)
    b = run(make_cfg(s), Device(d))
    check_routing(fetch(b), o)
