"""Plain float64 definition of the MoE FFN layer (CPU oracle; test infrastructure only).

Follows the MoE-layer paragraph of the Introduction of "X-Stage: An Overlooked Pipeline Stage
for Communication-Computation Overlap in DiT Inference": route -> Dispatch -> Linear-1 ->
SwiGLU -> Linear-2 -> Combine with the router weights. Steps the page leaves open are fixed
by these readings:

  routing   softmax over all E router logits, keep the k largest logits (descending; equal
            logits -> lower expert id first), renormalise the kept probabilities to sum to 1;
            weights are handed on as float32.
  plan      rows of the dispatched buffer are grouped by expert and, inside one expert,
            ordered by the flat slot index f = t*k + j (a stable counting sort).
  Linear-1  W1[e] is [2I, H]: rows [0, I) are the gate projection, rows [I, 2I) the up
            projection; SwiGLU(x) = silu(x W_gate^T) * (x W_up^T), silu(z) = z / (1 + e^-z)
            (the definition of Shazeer, "GLU Variants Improve Transformer", which the page
            cites for SwiGLU).
  Linear-2  W2[e] is [H, I].
  rounding  bfloat16 round-to-nearest-even at exactly three points: the activation A, the
            expert output rows Yd and the layer output; everything else is float64 here.
  combine   out[t] = sum over j = 0..k-1 (ascending) of w[t, j] * Yd[row of (t, j)].
"""
from __future__ import annotations

import numpy as np

# ---------------------------------------------------------------- bfloat16 helpers

_BF16_MAX = float.fromhex("0x1.fep127")  # largest finite bfloat16


def bf16_round(x) -> np.ndarray:
    """Round float64 values to the nearest bfloat16 value, ties to even (result in float64).

    bfloat16 has 8 significant bits and float32's exponent range; subnormals step by 2^-133.
    The value is scaled by a power of two so its last kept bit is the units place, rounded
    with ``np.rint`` (ties to even) and scaled back. Magnitudes that round above the largest
    finite bfloat16 become infinities; NaN stays NaN.
    """
    x = np.asarray(x, dtype=np.float64)
    with np.errstate(invalid="ignore", over="ignore"):
        _, e = np.frexp(x)  # x = m * 2^e with 0.5 <= |m| < 1
        q = np.maximum(e.astype(np.int64) - 8, -133)  # exponent of the last kept bit
        y = np.ldexp(np.rint(np.ldexp(x, -q)), q)
        y = np.where(np.abs(y) > _BF16_MAX, np.copysign(np.inf, x), y)
    return np.where(np.isfinite(x), y, x)


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """Decode bfloat16 bit patterns (uint16) to float64."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    with np.errstate(invalid="ignore"):
        return b.view(np.float32).astype(np.float64)


def f64_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Encode float64 values that are already bfloat16-representable as bit patterns."""
    f = np.asarray(x, dtype=np.float64).astype(np.float32)
    return (f.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


# ---------------------------------------------------------------- routing and plan

def route(logits: np.ndarray, k: int):
    """Top-k routing of each token (Introduction, MoE-layer paragraph: the router selects
    one or more experts per token; Combine weights by the router weights).

    logits: float32 [T, E]. Returns ids int32 [T, k] (descending logit, ties -> lower id) and
    weights float32 [T, k] = softmax(logits)[ids] renormalised over the k kept experts,
    computed in float64 and rounded once to float32.
    """
    lg = np.asarray(logits, dtype=np.float32)
    T, E = lg.shape
    if not 1 <= k <= E:
        raise ValueError("need 1 <= k <= E")
    l64 = lg.astype(np.float64)
    ids = np.empty((T, k), np.int32)
    expert = np.arange(E)
    for t in range(T):
        # lexsort sorts by the last key first: primary -logit ascending, then expert id
        order = np.lexsort((expert, -l64[t]))
        ids[t] = order[:k]
    p = np.exp(l64 - l64.max(axis=1, keepdims=True))
    p /= p.sum(axis=1, keepdims=True)
    kept = np.take_along_axis(p, ids.astype(np.int64), axis=1)
    w = (kept / kept.sum(axis=1, keepdims=True)).astype(np.float32)
    return ids, w


def plan(ids: np.ndarray, E: int):
    """Expert-contiguous row plan (Dispatch groups each expert's tokens together).

    Flat slot f = t*k + j goes to expert e_f = ids[t, j]. Returns
      counts  int32 [E]     rows per expert
      offsets int32 [E+1]   first row of each expert; offsets[E] = T*k
      perm    int32 [T*k]   perm[r] = slot stored in row r (stable by f inside an expert)
      pos     int32 [T*k]   pos[f] = row holding slot f (inverse of perm)
    """
    ef = np.asarray(ids, dtype=np.int64).reshape(-1)
    counts = np.bincount(ef, minlength=E).astype(np.int32)
    offsets = np.zeros(E + 1, np.int32)
    offsets[1:] = np.cumsum(counts)
    perm = np.argsort(ef, kind="stable").astype(np.int32)
    pos = np.empty_like(perm)
    pos[perm] = np.arange(perm.size, dtype=np.int32)
    return counts, offsets, perm, pos


def dispatch(x_bits: np.ndarray, perm: np.ndarray, k: int) -> np.ndarray:
    """Dispatched rows: Xd[r] = X[perm[r] // k] (a bit copy of bfloat16 rows)."""
    return np.asarray(x_bits)[np.asarray(perm, dtype=np.int64) // k]


# ---------------------------------------------------------------- expert FFN

def silu(z: np.ndarray) -> np.ndarray:
    """silu(z) = z * sigmoid(z) = z / (1 + exp(-z)), float64."""
    z = np.asarray(z, dtype=np.float64)
    with np.errstate(over="ignore"):
        return z / (1.0 + np.exp(-z))


def expert_ffn(xd_rows: np.ndarray, w1e: np.ndarray, w2e: np.ndarray):
    """One expert's two-layer FFN on its dispatched rows (bfloat16 bits in and out).

    Linear-1: h = x W1^T in float64, h = [gate | up]; A = bf16(silu(gate) * up);
    Linear-2: Yd = bf16(A W2^T). Returns (A bits [n, I], Yd bits [n, H]).
    """
    I = w1e.shape[0] // 2
    x = bf16_to_f64(xd_rows)
    h = x @ bf16_to_f64(w1e).T
    a = bf16_round(silu(h[:, :I]) * h[:, I:])
    y = bf16_round(a @ bf16_to_f64(w2e).T)
    return f64_to_bf16_bits(a), f64_to_bf16_bits(y)


def forward(xd_bits: np.ndarray, offsets: np.ndarray, w1: np.ndarray, w2: np.ndarray):
    """Linear-1 + SwiGLU + Linear-2 for every expert with rows (experts with none are skipped).

    Returns A bits [T*k, I] and Yd bits [T*k, H].
    """
    R = xd_bits.shape[0]
    E, twoI, H = w1.shape
    a = np.zeros((R, twoI // 2), np.uint16)
    yd = np.zeros((R, H), np.uint16)
    for e in range(E):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if hi > lo:
            a[lo:hi], yd[lo:hi] = expert_ffn(xd_bits[lo:hi], w1[e], w2[e])
    return a, yd


def combine(yd_bits: np.ndarray, w: np.ndarray, pos: np.ndarray, T: int, k: int) -> np.ndarray:
    """out[t] = bf16(sum_{j=0..k-1} w[t,j] * Yd[pos[t*k+j]]), float64 sum in ascending j."""
    y = bf16_to_f64(yd_bits)
    w64 = np.asarray(w, dtype=np.float64).reshape(T, k)
    p = np.asarray(pos, dtype=np.int64).reshape(T, k)
    acc = np.zeros((T, yd_bits.shape[1]), np.float64)
    for j in range(k):
        acc += w64[:, j:j + 1] * y[p[:, j]]
    return f64_to_bf16_bits(bf16_round(acc))


def moe_layer(x_bits, logits, w1, w2, k: int) -> dict:
    """The whole layer on all tokens. Returns every intermediate by name."""
    E = w1.shape[0]
    T = x_bits.shape[0]
    ids, w = route(logits, k)
    counts, offsets, perm, pos = plan(ids, E)
    xd = dispatch(x_bits, perm, k)
    a, yd = forward(xd, offsets, w1, w2)
    out = combine(yd, w, pos, T, k)
    return dict(ids=ids, w=w, counts=counts, offsets=offsets, perm=perm, pos=pos,
                xd=xd, a=a, yd=yd, out=out)
