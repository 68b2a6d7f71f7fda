"""Pins of the CPU oracle against things other than itself: hand-worked golden cases, closed
forms, library routines (numpy / torch CPU), brute force on micro shapes and invariants."""
import math

import numpy as np
import pytest
import torch

import moe_workloads as W
from oracle import brute, invariants as V, moe_ref as R
from tests.conftest import golden_rows

# ------------------------------------------------------------------ bfloat16 rounding

def test_bf16_golden():
    for row in golden_rows("bf16_cases.txt"):
        src, exp_bits = row[0].split()[:2]
        x = float.fromhex(src)
        got = int(R.f64_to_bf16_bits(R.bf16_round(np.array([x])))[0])
        assert got == int(exp_bits, 16), (src, hex(got), exp_bits)


def test_bf16_matches_exact_rational_rounding():
    rng = np.random.default_rng(5)
    xs = np.concatenate([
        rng.standard_normal(2000) * 10.0 ** rng.integers(-40, 39, 2000),
        # exact ties between neighbouring bfloat16 values
        (np.arange(1, 400) * 2 + 1) * 2.0 ** -9,
        rng.standard_normal(200) * 2.0 ** -130,  # subnormal range
    ])
    ours = R.bf16_round(xs)
    for x, o in zip(xs, ours):
        assert brute.bf16_nearest(float(x)) == o, x


def test_bf16_matches_torch_on_float32_inputs():
    # torch's float32 -> bfloat16 cast is round-to-nearest-even; on float32 inputs the
    # float64 rounding must agree with it exactly
    rng = np.random.default_rng(6)
    f = (rng.standard_normal(50000) * 10.0 ** rng.integers(-30, 30, 50000)).astype(np.float32)
    t = torch.from_numpy(f).to(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(R.bf16_round(f.astype(np.float64)), t)


def test_bf16_codec_roundtrip():
    bits = np.arange(0, 1 << 16, dtype=np.uint32).astype(np.uint16)
    vals = R.bf16_to_f64(bits)
    fin = np.isfinite(vals)
    np.testing.assert_array_equal(R.f64_to_bf16_bits(vals[fin]), bits[fin])
    # decoding agrees with torch's bit reinterpretation
    tv = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(vals[fin], tv[fin])


# ------------------------------------------------------------------ SwiGLU

def test_silu_closed_forms():
    for row in golden_rows("silu_cases.txt"):
        z, expect = [float(v) for v in row[0].split()[:2]]
        got = float(R.silu(np.array([z]))[0])
        assert got == pytest.approx(expect, rel=1e-15, abs=1e-300), z


def test_silu_odd_part_identity():
    # silu(z) - silu(-z) = z * (sigmoid(z) + sigmoid(-z)) = z
    z = np.linspace(-30, 30, 1201)
    np.testing.assert_allclose(R.silu(z) - R.silu(-z), z, rtol=1e-14, atol=1e-14)
    # and silu(z)/z -> 0 as z -> -inf
    assert abs(float(R.silu(np.array([-60.0]))[0])) < 1e-24


# ------------------------------------------------------------------ routing

def test_route_golden():
    for k, logits, ids, ws in golden_rows("route_cases.txt"):
        k = int(k)
        lg = np.array([[float(v) for v in logits.split()]], np.float32)
        gi, gw = R.route(lg, k)
        assert gi[0].tolist() == [int(v) for v in ids.split()], logits
        np.testing.assert_allclose(gw[0], [float(v) for v in ws.split()], rtol=0, atol=2.0 ** -20)


def test_route_matches_brute_and_sort_routine():
    rng = np.random.default_rng(7)
    for E, k in [(1, 1), (4, 2), (8, 8), (16, 3), (33, 5)]:
        lg = rng.standard_normal((40, E)).astype(np.float32)
        lg[::7, : min(E, 3)] = 0.25  # plant ties
        ids, w = R.route(lg, k)
        bi, bw = brute.route(lg.tolist(), k)
        np.testing.assert_array_equal(ids, np.array(bi))
        np.testing.assert_allclose(w, np.array(bw, np.float32), rtol=0, atol=2.0 ** -22)
        # independent library check: torch.topk on (logit, -id) via a stable descending sort
        order = torch.sort(torch.from_numpy(lg), dim=1, descending=True, stable=True).indices
        np.testing.assert_array_equal(ids, order[:, :k].numpy())
        # weights: torch softmax of the kept logits (the full denominator cancels)
        kept = torch.gather(torch.from_numpy(lg).double(), 1, torch.from_numpy(ids).long())
        np.testing.assert_allclose(w, torch.softmax(kept, dim=1).numpy(), rtol=0, atol=2.0 ** -22)
        np.testing.assert_allclose(w.astype(np.float64).sum(1), 1.0, atol=1e-6)


# ------------------------------------------------------------------ plan

def test_plan_golden():
    for E, ids, counts, offsets, perm, pos in golden_rows("plan_cases.txt"):
        E = int(E)
        arr = np.array([[int(v) for v in tok.split()] for tok in ids.split(";")], np.int32)
        c, o, p, q = R.plan(arr, E)
        assert c.tolist() == [int(v) for v in counts.split()]
        assert o.tolist() == [int(v) for v in offsets.split()]
        assert p.tolist() == [int(v) for v in perm.split()]
        assert q.tolist() == [int(v) for v in pos.split()]


def test_plan_invariants_and_brute():
    rng = np.random.default_rng(8)
    for T, E, k in [(1, 1, 1), (13, 4, 2), (50, 16, 4), (64, 8, 8)]:
        lg = rng.standard_normal((T, E)).astype(np.float32)
        ids, _ = R.route(lg, k)
        c, o, p, q = R.plan(ids, E)
        assert c.sum() == T * k
        assert np.all(np.diff(o) >= 0) and o[0] == 0 and o[-1] == T * k
        np.testing.assert_array_equal(q[p], np.arange(T * k))
        ef = ids.reshape(-1)
        # every row of expert e's block holds a slot routed to e, in increasing slot order
        for e in range(E):
            blk = p[o[e]:o[e + 1]]
            assert np.all(ef[blk] == e) and np.all(np.diff(blk) > 0)
        bc, bo, bp, bq = brute.plan(ids.tolist(), E)
        assert (c.tolist(), o.tolist(), p.tolist(), q.tolist()) == (bc, bo, bp, bq)


def test_dispatch_inverse_permutation_is_identity():
    s = W.shape(T=37, H=64, I=64, E=5, k=3)
    d = W.generate(s, parts=("x", "logits"))
    ids, _ = R.route(d["logits"], s.k)
    _, _, perm, pos = R.plan(ids, s.E)
    xd = R.dispatch(d["x"], perm, s.k)
    # scatter back by perm, then every k-th slot is the original token
    back = np.empty_like(xd)
    back[perm] = xd
    np.testing.assert_array_equal(back[:: s.k], d["x"])
    np.testing.assert_array_equal(xd[pos].reshape(s.T, s.k, s.H)[:, 1], d["x"])


# ------------------------------------------------------------------ whole layer

@pytest.mark.parametrize("T,H,I,E,k", [(6, 8, 4, 3, 2), (9, 16, 8, 5, 3), (4, 8, 8, 1, 1), (5, 8, 4, 4, 4)])
def test_layer_matches_brute(T, H, I, E, k):
    s = W.shape(T=T, H=H, I=I, E=E, k=k, seed=100 + T, x_std=1.0, w_std=0.5)
    d = W.generate(s)
    o = R.moe_layer(d["x"], d["logits"], d["w1"], d["w2"], k)
    b = brute.layer(d["x"].tolist(), d["logits"].tolist(), d["w1"].tolist(), d["w2"].tolist(), k)
    np.testing.assert_array_equal(o["ids"], np.array(b["ids"]))
    for key in ("counts", "offsets", "perm", "pos"):
        assert o[key].tolist() == b[key], key

    def ulps(x, y):
        xi = np.asarray(x, np.uint16).astype(np.int32)
        yi = np.asarray(y, np.uint16).astype(np.int32)
        # sign-magnitude to ordered integers
        xi = np.where(xi & 0x8000, -(xi & 0x7FFF), xi)
        yi = np.where(yi & 0x8000, -(yi & 0x7FFF), yi)
        return np.abs(xi - yi)

    for key in ("a", "yd", "out"):
        u = ulps(o[key], np.array(b[key], np.uint16))
        assert u.max() <= 1, key
        assert (u == 0).mean() > 0.97, key


def _dense_vs_layer(s, w1e, w2e, d, E):
    w1, w2 = V.identical_experts(d["x"], w1e, w2e, E)
    o = R.moe_layer(d["x"], d["logits"], w1, w2, s.k)
    dense = V.dense_ffn(d["x"], w1e, w2e)
    return o, dense


def test_identical_experts_equal_dense_ffn():
    s = W.shape(T=48, H=64, I=32, E=6, k=3, seed=11, x_std=1.0, w_std=0.1)
    d = W.generate(s)
    o, dense = _dense_vs_layer(s, d["w1"][0], d["w2"][0], d, s.E)
    np.testing.assert_array_equal(R.bf16_to_f64(o["out"]), dense["y"])


def test_single_expert_top1_equals_dense_ffn():
    s = W.shape(T=40, H=64, I=64, E=1, k=1, seed=12, x_std=1.0, w_std=0.1)
    d = W.generate(s)
    o = R.moe_layer(d["x"], d["logits"], d["w1"], d["w2"], 1)
    assert np.all(o["w"] == 1.0)
    dense = V.dense_ffn(d["x"], d["w1"][0], d["w2"][0])
    np.testing.assert_array_equal(R.bf16_to_f64(o["out"]), dense["y"])


def test_dense_ffn_matches_torch():
    # the dense reduction itself against torch CPU float64 (matmul + silu library routines)
    s = W.shape(T=32, H=64, I=48, E=1, k=1, seed=13, x_std=1.0, w_std=0.1)
    d = W.generate(s)
    dense = V.dense_ffn(d["x"], d["w1"][0], d["w2"][0])
    x = torch.from_numpy(R.bf16_to_f64(d["x"]))
    w1 = torch.from_numpy(R.bf16_to_f64(d["w1"][0]))
    w2 = torch.from_numpy(R.bf16_to_f64(d["w2"][0]))
    h = x @ w1.T
    a = torch.nn.functional.silu(h[:, :48]) * h[:, 48:]
    a_b = a.float().to(torch.bfloat16).double()  # a is exact enough in f32 for this size
    np.testing.assert_allclose(dense["a"], a_b.numpy(), rtol=2.0 ** -7, atol=0)
    y = (torch.from_numpy(dense["a"]) @ w2.T).float().to(torch.bfloat16).double().numpy()
    np.testing.assert_allclose(dense["y"], y, rtol=2.0 ** -7, atol=0)


@pytest.mark.parametrize("k", [1, 2])
def test_exact_integer_case(k):
    c = V.exact_integer_case(T=64, H=256, I=256, E=4, k=k)
    o = R.moe_layer(c["x"], c["logits"], c["w1"], c["w2"], k)
    ex = c["expected"]
    np.testing.assert_array_equal(o["ids"], ex["ids"])
    np.testing.assert_array_equal(o["w"], ex["w"])
    T = c["x"].shape[0]
    np.testing.assert_array_equal(o["a"][o["pos"]].reshape(T, k, -1), ex["a_tok"])
    np.testing.assert_array_equal(o["yd"][o["pos"]].reshape(T, k, -1), ex["y_tok"])
    np.testing.assert_array_equal(o["out"], ex["out"])
    assert np.all(o["counts"] > 0)
