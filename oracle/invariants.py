"""Special cases with a known answer, for pinning the CPU oracle (test infrastructure only).

Each builder returns inputs (bfloat16 bit patterns as uint16, float32 logits) whose layer
output is fixed by something other than the oracle itself:

  * ``dense_ffn``: the plain SwiGLU feed-forward network of one expert applied to every
    token, written with numpy matmul (the textbook routine the MoE layer reduces to);
  * ``identical_experts``: every expert holds the same weights, so the router-weighted sum of
    k identical rows is that row times sum(w) = 1 (the renormalised weights), and the layer
    equals ``dense_ffn``;
  * ``single_expert``: E = 1 and k = 1, the weight is exp(0)/exp(0) = 1 exactly;
  * ``exact_integer_case``: small integers everywhere, so every value before a rounding point
    is exact in float32 and every rounded intermediate is exactly representable; any correct
    implementation must then produce the same bits.
"""
from __future__ import annotations

import numpy as np


def _bits(a: np.ndarray) -> np.ndarray:
    """bfloat16 bits of float32 values that are exactly representable (checked)."""
    f = np.asarray(a, dtype=np.float32)
    b = f.view(np.uint32)
    if np.any(b & np.uint32(0xFFFF)):
        raise ValueError("value not exactly representable in bfloat16")
    return (b >> np.uint32(16)).astype(np.uint16)


def _decode(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32).astype(
        np.float64)


def _nearest_bf16(x: np.ndarray) -> np.ndarray:
    """Round-to-nearest-even to bfloat16 for float64 values, via float32 bit arithmetic on
    values that are exactly float32 (used only where the pre-rounding value is exact)."""
    f = np.asarray(x, dtype=np.float64).astype(np.float32)
    if not np.array_equal(f.astype(np.float64), np.asarray(x, np.float64)):
        raise ValueError("pre-rounding value is not exact in float32")
    b = f.view(np.uint32)
    r = (b + np.uint32(0x7FFF) + ((b >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def dense_ffn(x_bits, w1e_bits, w2e_bits) -> dict:
    """Dense SwiGLU FFN for all tokens with one weight set: A = bf16(silu(x Wg^T) * (x Wu^T)),
    Y = bf16(A W2^T), in float64 via numpy matmul. Returns A and Y as float64 values."""
    from oracle.moe_ref import bf16_round  # rounding is the oracle's own; pinned separately

    x = _decode(x_bits)
    w1 = _decode(w1e_bits)
    w2 = _decode(w2e_bits)
    I = w1.shape[0] // 2
    g = x @ w1[:I].T
    u = x @ w1[I:].T
    a = bf16_round(g / (1.0 + np.exp(-g)) * u)
    y = bf16_round(a @ w2.T)
    return dict(a=a, y=y)


def identical_experts(x_bits, w1e_bits, w2e_bits, E: int):
    """Stack one expert's weights E times."""
    w1 = np.broadcast_to(w1e_bits, (E,) + w1e_bits.shape).copy()
    w2 = np.broadcast_to(w2e_bits, (E,) + w2e_bits.shape).copy()
    return w1, w2


def exact_integer_case(T: int = 64, H: int = 256, I: int = 256, E: int = 4, k: int = 2,
                       seed: int = 0):
    """Inputs whose layer output is exact at every step (see the module docstring).

    X in {0, 1} with X[:, 0] = 1. Gate rows of W1 hold 32*c_e (c_e in {1, 2}) on column 0
    only, so every gate value is 32 or 64 and silu(g) equals g in float32 (1 + e^-32 rounds
    to 1) and rounds back to g in bfloat16. Up rows hold {-1, 0, 1} with column 0 zero, so
    |up| <= H - 1 < 256 and A = g * up has at most 8 significant bits. W2 has one 1 per row,
    so each Yd entry is a copy of an A entry. Logits give each token either one clear winner
    (k = 1) or an exact tie between its two picks (k = 2, weights 1/2 each) with every other
    logit strictly lower; the tied pair varies with t so that every expert receives rows.
    Every value before a rounding point is an integer or half-integer below 2^24.

    Returns dict(x, logits, w1, w2, expected) where ``expected`` holds ids, w, a, yd, out
    derived directly from the construction above (not from the oracle).
    """
    if k not in (1, 2) or E < 2 or H < 2 or I < 1 or H > 256:
        raise ValueError("exact case needs k in {1,2}, E >= 2, 2 <= H <= 256")
    rng = np.random.Generator(np.random.PCG64(seed))
    x = (rng.random((T, H)) < 0.5).astype(np.float32)
    x[:, 0] = 1.0
    c = 1 + (np.arange(E) % 2)  # per-expert gate scale 1 or 2
    w1 = np.zeros((E, 2 * I, H), np.float32)
    w1[:, :I, 0] = (32.0 * c)[:, None]
    up = rng.integers(-1, 2, size=(E, I, H)).astype(np.float32)
    up[:, :, 0] = 0.0
    w1[:, I:, :] = up
    w2 = np.zeros((E, H, I), np.float32)
    src = rng.integers(0, I, size=(E, H))
    for e in range(E):
        w2[e, np.arange(H), src[e]] = 1.0
    logits = np.full((T, E), -4.0, np.float32)
    ids = np.zeros((T, k), np.int32)
    for t in range(T):
        a = t % E
        b = (a + 1 + (t // E) % (E - 1)) % E
        if k == 1:
            logits[t, a] = 1.0
            ids[t, 0] = a
        else:
            logits[t, a] = logits[t, b] = 0.5
            ids[t] = (min(a, b), max(a, b))
        # give non-picked experts distinct strictly lower logits
        others = [e for e in range(E) if e not in ids[t]]
        for r, e in enumerate(others):
            logits[t, e] = -1.0 - 0.25 * r
    wts = np.full((T, k), 1.0 / k, np.float32)
    # expected values straight from the construction
    a_tok = np.zeros((T, k, I), np.float64)
    y_tok = np.zeros((T, k, H), np.float64)
    for t in range(T):
        for j in range(k):
            e = ids[t, j]
            g = 32.0 * c[e]
            u = up[e] @ x[t]
            a_tok[t, j] = g * u
            y_tok[t, j] = a_tok[t, j][src[e]]
    out = (y_tok * (1.0 / k)).sum(axis=1)
    expected = dict(ids=ids, w=wts, a_tok=_nearest_bf16(a_tok), y_tok=_nearest_bf16(y_tok),
                    out=_nearest_bf16(out))
    return dict(x=_bits(x), logits=logits, w1=_bits(w1), w2=_bits(w2), expected=expected)
