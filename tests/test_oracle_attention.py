"""Pins of the attention oracle (oracle/attention_ref.py) against what fixes its result
without it: closed forms (uniform scores give the mean of V; one dominant key gives its V row;
one key gives V[0]), invariance under a joint permutation of the keys, scalar brute force on
tiny inputs, and torch's float64 scaled_dot_product_attention; three planted mistakes (no
1/sqrt(d) scale, softmax over the query axis, swapped operands) must each be caught."""
import math

import numpy as np
import pytest
import torch

import moe_workloads as W
from oracle import attention_ref as A
from oracle.moe_ref import bf16_round, bf16_to_f64, f64_to_bf16_bits


def bits(x):
    return f64_to_bf16_bits(bf16_round(np.asarray(x, np.float64)))


def rand_qkv(B, H, M, d, seed):
    s = W.attn_shape(B=B, heads=H, M=M, d=d, seed=seed)
    g = W.generate_attention(s)
    return g["q"], g["k"], g["v"]


def ulp_close(a_bits, b_bits, max_ulps=1):
    a = np.asarray(a_bits, np.int64)
    b = np.asarray(b_bits, np.int64)
    # bf16 bits of same-sign finite values: integer distance is the ulp distance
    return np.abs(a - b).max() <= max_ulps


def test_uniform_scores_give_the_mean_of_v():
    q, _, v = rand_qkv(1, 2, 37, 64, 1)
    k = np.zeros_like(q)  # every score is 0
    o, lse = A.attention(q, k, v)
    assert np.array_equal(o, bits(bf16_to_f64(v).mean(axis=2, keepdims=True).repeat(37, axis=2)))
    np.testing.assert_allclose(lse, math.log(37), rtol=0, atol=1e-12)


def test_one_dominant_key_gives_its_value_row():
    M, d = 20, 32
    q = np.zeros((1, 1, M, d))
    q[..., 0] = 64.0
    k = np.zeros((1, 1, M, d))
    k[0, 0, 7, 0] = 64.0  # scores 64*64/sqrt(32) ~ 724 for key 7, 0 for the others
    _, _, v = rand_qkv(1, 1, M, d, 2)
    o, _ = A.attention(bits(q), bits(k), v)
    assert np.array_equal(o, np.repeat(v[:, :, 7:8], M, axis=2))


def test_a_single_key_gives_v0():
    q, k, v = rand_qkv(2, 3, 1, 128, 3)
    o, lse = A.attention(q, k, v)
    assert np.array_equal(o, v)
    s = (bf16_to_f64(q) * bf16_to_f64(k)).sum(-1) / math.sqrt(128)
    np.testing.assert_allclose(lse, s, rtol=0, atol=1e-12)


def test_joint_permutation_of_the_keys_changes_nothing():
    q, k, v = rand_qkv(1, 2, 50, 64, 4)
    perm = np.random.default_rng(0).permutation(50)
    o1, l1 = A.attention(q, k, v)
    o2, l2 = A.attention(q, k[:, :, perm], v[:, :, perm])
    assert ulp_close(o1, o2) and np.mean(o1 == o2) > 0.999
    np.testing.assert_allclose(l1, l2, rtol=0, atol=1e-12)


def brute(q_bits, k_bits, v_bits):
    """Scalar loops: per query, scores by fsum, softmax by math.exp, weighted fsum of V."""
    q, k, v = bf16_to_f64(q_bits), bf16_to_f64(k_bits), bf16_to_f64(v_bits)
    B, H, M, d = q.shape
    out = np.zeros((B, H, M, d))
    lse = np.zeros((B, H, M))
    for b in range(B):
        for h in range(H):
            for i in range(M):
                s = [math.fsum(q[b, h, i, t] * k[b, h, j, t] for t in range(d)) / math.sqrt(d) for j in range(M)]
                mx = max(s)
                e = [math.exp(x - mx) for x in s]
                z = math.fsum(e)
                lse[b, h, i] = mx + math.log(z)
                for t in range(d):
                    out[b, h, i, t] = math.fsum(e[j] * v[b, h, j, t] for j in range(M)) / z
    return bits(out), lse


def test_brute_force_on_tiny_inputs():
    for seed, (B, H, M, d) in enumerate([(1, 1, 5, 8), (2, 2, 7, 16), (1, 3, 3, 4)]):
        q, k, v = rand_qkv(B, H, M, d, 10 + seed)
        o, lse = A.attention(q, k, v)
        ob, lb = brute(q, k, v)
        assert ulp_close(o, ob) and np.mean(o == ob) > 0.97
        np.testing.assert_allclose(lse, lb, rtol=0, atol=1e-12)


def torch_attention(q_bits, k_bits, v_bits):
    t = [torch.from_numpy(bf16_to_f64(x)) for x in (q_bits, k_bits, v_bits)]
    o = torch.nn.functional.scaled_dot_product_attention(*t)  # scale 1/sqrt(d), float64, CPU
    return bits(o.numpy())


def test_library_routine():
    q, k, v = rand_qkv(1, 2, 200, 128, 20)
    o, _ = A.attention(q, k, v)
    ot = torch_attention(q, k, v)
    assert ulp_close(o, ot) and np.mean(o == ot) > 0.999


def test_selected_rows_equal_the_full_result():
    q, k, v = rand_qkv(1, 2, 90, 64, 21)
    o, lse = A.attention(q, k, v)
    rows = np.array([0, 5, 89])
    o2, l2 = A.attention(q, k, v, rows=rows)
    assert np.array_equal(o2, o[:, :, rows])
    np.testing.assert_allclose(l2, lse[:, :, rows], rtol=0, atol=1e-12)


def _mutant(kind):
    def f(q_bits, k_bits, v_bits):
        q, k, v = bf16_to_f64(q_bits), bf16_to_f64(k_bits), bf16_to_f64(v_bits)
        d = q.shape[-1]
        s = np.matmul(q, np.swapaxes(k, -1, -2))
        if kind == "scale_by_d":
            s = s / d
        elif kind != "no_scale":
            s = s / np.sqrt(d)
        ax = -2 if kind == "softmax_over_queries" else -1
        e = np.exp(s - s.max(axis=ax, keepdims=True))
        p = e / e.sum(axis=ax, keepdims=True)
        o = np.matmul(p, v) if kind != "swapped_operands" else np.matmul(p, q)
        return bits(o)
    return f


@pytest.mark.parametrize("kind", ["no_scale", "scale_by_d", "softmax_over_queries", "swapped_operands"])
def test_planted_mistakes_are_caught(kind):
    q, k, v = rand_qkv(1, 2, 40, 32, 30)
    bad = _mutant(kind)(q, k, v)
    good = torch_attention(q, k, v)
    assert not ulp_close(bad, good, max_ulps=4)
