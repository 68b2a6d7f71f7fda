"""Plant plausible mistakes in the CPU oracle (on the CPU only) and check that the pins
catch every one: a pin set that a wrong oracle also passes would prove nothing."""
import numpy as np
import pytest

import moe_workloads as W
from oracle import brute, invariants as V, moe_ref as R
from tests.conftest import golden_rows


def _pins():
    """A compact run of the pins; raises AssertionError on the first violated one."""
    # golden routing
    for k, logits, ids, ws in golden_rows("route_cases.txt"):
        lg = np.array([[float(v) for v in logits.split()]], np.float32)
        gi, gw = R.route(lg, int(k))
        assert gi[0].tolist() == [int(v) for v in ids.split()]
        assert np.allclose(gw[0], [float(v) for v in ws.split()], rtol=0, atol=2.0 ** -20)
    # golden plan
    for E, ids, counts, offsets, perm, pos in golden_rows("plan_cases.txt"):
        arr = np.array([[int(v) for v in t.split()] for t in ids.split(";")], np.int32)
        c, o, p, q = R.plan(arr, int(E))
        assert p.tolist() == [int(v) for v in perm.split()]
        assert q.tolist() == [int(v) for v in pos.split()]
    # golden bf16 rounding
    for row in golden_rows("bf16_cases.txt"):
        src, exp_bits = row[0].split()[:2]
        got = int(R.f64_to_bf16_bits(R.bf16_round(np.array([float.fromhex(src)])))[0])
        assert got == int(exp_bits, 16)
    # exact-integer layer
    for k in (1, 2):
        c = V.exact_integer_case(T=32, H=64, I=32, E=4, k=k)
        o = R.moe_layer(c["x"], c["logits"], c["w1"], c["w2"], k)
        assert np.array_equal(o["out"], c["expected"]["out"])
    # brute force on a micro shape
    s = W.shape(T=6, H=8, I=4, E=3, k=2, seed=106, x_std=1.0, w_std=0.5)
    d = W.generate(s)
    o = R.moe_layer(d["x"], d["logits"], d["w1"], d["w2"], 2)
    b = brute.layer(d["x"].tolist(), d["logits"].tolist(), d["w1"].tolist(), d["w2"].tolist(), 2)
    for key in ("a", "yd", "out"):
        diff = np.abs(R.bf16_to_f64(o[key]) - R.bf16_to_f64(np.array(b[key], np.uint16)))
        assert diff.max() <= 2.0 ** -6 * max(1e-30, np.abs(R.bf16_to_f64(np.array(b[key], np.uint16))).max())


def test_unmutated_oracle_passes_pins():
    _pins()


def _swap_gate_up(xd_rows, w1e, w2e):
    I = w1e.shape[0] // 2
    return ORIG["expert_ffn"](xd_rows, np.concatenate([w1e[I:], w1e[:I]]), w2e)


def _silu_sign(z):
    z = np.asarray(z, dtype=np.float64)
    with np.errstate(over="ignore"):
        return z / (1.0 + np.exp(z))


def _no_renorm(logits, k):
    ids, _ = ORIG["route"](logits, k)
    l64 = np.asarray(logits, np.float64)
    p = np.exp(l64 - l64.max(1, keepdims=True))
    p /= p.sum(1, keepdims=True)
    return ids, np.take_along_axis(p, ids.astype(np.int64), 1).astype(np.float32)


def _ties_high(logits, k):
    lg = np.asarray(logits, np.float32)
    T, E = lg.shape
    ids = np.empty((T, k), np.int32)
    for t in range(T):
        ids[t] = np.lexsort((-np.arange(E), -lg[t].astype(np.float64)))[:k]
    _, w = ORIG["route"](logits, k)
    return ids, w


def _unstable_plan(ids, E):
    c, o, _, _ = ORIG["plan"](ids, E)
    ef = np.asarray(ids).reshape(-1)
    perm = np.argsort(-np.arange(ef.size))[np.argsort(ef[::-1], kind="stable")].astype(np.int32)
    pos = np.empty_like(perm)
    pos[perm] = np.arange(perm.size, dtype=np.int32)
    return c, o, perm, pos


def _combine_by_perm(yd_bits, w, pos, T, k):
    # uses the row -> slot map where the slot -> row map is needed
    inv = np.empty_like(pos)
    inv[pos] = np.arange(pos.size, dtype=pos.dtype)
    return ORIG["combine"](yd_bits, w, inv, T, k)


def _round_half_up(x):
    x = np.asarray(x, dtype=np.float64)
    _, e = np.frexp(x)
    q = np.maximum(e.astype(np.int64) - 8, -133)
    return np.ldexp(np.floor(np.ldexp(x, -q) + 0.5), q)


def _dispatch_mod(x_bits, perm, k):
    return np.asarray(x_bits)[np.asarray(perm, np.int64) % np.asarray(x_bits).shape[0]]


ORIG = {n: getattr(R, n) for n in ("expert_ffn", "route", "plan", "combine", "bf16_round", "dispatch", "silu")}

MUTANTS = {
    "swap_gate_up": ("expert_ffn", _swap_gate_up),
    "silu_sign": ("silu", _silu_sign),
    "no_renormalisation": ("route", _no_renorm),
    "ties_to_higher_id": ("route", _ties_high),
    "unstable_plan": ("plan", _unstable_plan),
    "combine_wrong_map": ("combine", _combine_by_perm),
    "round_half_up": ("bf16_round", _round_half_up),
    "dispatch_wrong_token": ("dispatch", _dispatch_mod),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_mutant(name, monkeypatch):
    attr, fn = MUTANTS[name]
    monkeypatch.setattr(R, attr, fn)
    with pytest.raises(AssertionError):
        _pins()
