"""Plain float64 definition of the attention forward that the X-Stage paper fuses with the
Ulysses all-to-all (CPU oracle; test infrastructure only).

Section 4.3 of "X-Stage: An Overlooked Pipeline Stage for Communication-Computation Overlap
in DiT Inference": after the first Ulysses all-to-all each GPU holds the whole sequence of M
tokens for its share of the heads, and runs full, non-causal attention (the DiT setting) with
head dimension d; FlashAttention computes it tile by tile, writing one b_m x d output tile at
each tile boundary. The result is the plain definition, per (batch, head):

    O = softmax(Q K^T / sqrt(d)) V        softmax over the key axis, every key visible

Readings: Q, K, V and O are [B, heads, M, d] row-major, bfloat16 in and out; the scale is
1/sqrt(d) (the standard one; the page prints no formula); O is rounded to bfloat16 once, by
round-to-nearest-even, and everything before is float64 here. The log-sum-exp of each query's
scaled scores, lse = log(sum_j exp(s_j)), is also returned (float64).
"""
from __future__ import annotations

import numpy as np

from oracle.moe_ref import bf16_round, bf16_to_f64, f64_to_bf16_bits


def attention(q_bits, k_bits, v_bits, rows=None):
    """Attention of every head (or, per head, only the query rows `rows`).

    q_bits, k_bits, v_bits: uint16 [B, H, M, d] bfloat16 bits. rows: optional int array of
    query indices (the same for every head). Returns (O bits [B, H, len(rows) or M, d],
    lse float64 [B, H, len(rows) or M]).
    """
    q = bf16_to_f64(q_bits)
    k = bf16_to_f64(k_bits)
    v = bf16_to_f64(v_bits)
    if rows is not None:
        q = q[:, :, np.asarray(rows, np.int64)]
    d = q.shape[-1]
    s = np.matmul(q, np.swapaxes(k, -1, -2)) / np.sqrt(d)  # [B, H, Mq, M]
    m = s.max(axis=-1, keepdims=True)
    e = np.exp(s - m)
    den = e.sum(axis=-1, keepdims=True)
    o = np.matmul(e / den, v)
    lse = (m + np.log(den))[..., 0]
    return f64_to_bf16_bits(bf16_round(o)), lse


def flops(B: int, H: int, M: int, d: int) -> int:
    """Multiply-add work of the two products per head: 2 M^2 d each."""
    return 4 * B * H * M * M * d
