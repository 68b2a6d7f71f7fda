"""Seeded synthetic workloads for one GPU's share of an expert-parallel MoE FFN layer.

This module only draws inputs. It holds none of the layer's arithmetic: no routing, no
GEMM, no activation, no combine. The GPU library's tests and benchmark and the CPU oracle
both take their inputs from here, so the two sides see the same bytes.

Recipe (per named workload):
  * one root seed per workload; every tensor t and fixed-size block b of it is drawn from
    ``numpy.random.Generator(PCG64(SeedSequence(seed, spawn_key=(t, b))))``, so the bytes do
    not depend on how many threads draw them;
  * activations X and expert weights W1, W2 are drawn as float32 normals and rounded to
    bfloat16 by round-to-nearest-even (stored as uint16 bit patterns);
  * router logits are float32 N(0, 1), plus an optional per-expert bias added in float64
    and rounded once to float32 (the bias shapes expert popularity; it is part of the input,
    not of the layer).
"""
from __future__ import annotations

import concurrent.futures as _cf
import os
from dataclasses import dataclass, replace

import numpy as np

__all__ = ["MoeShape", "SHAPES", "SHAPE_ORDER", "shape", "generate", "flops", "nthreads",
           "AttnShape", "ATTN_SHAPES", "attn_shape", "generate_attention"]

_BLOCK = 1 << 22  # elements per independently seeded block

# tensor ids inside one workload's seed space
_T_X, _T_LOGITS, _T_BIAS, _T_W1, _T_W2 = 0, 1, 2, 3, 4


@dataclass(frozen=True)
class MoeShape:
    """Shape and value recipe of one synthetic MoE layer workload."""

    name: str
    T: int  # tokens
    H: int  # hidden size
    I: int  # expert intermediate size (Linear-1 produces 2*I: gate and up)
    E: int  # local experts
    k: int  # experts per token
    experts_per_wave: int
    seed: int
    x_std: float = 1.0
    w_std: float = 0.02
    bias: str = "none"  # "none" | "normal0.5" | "zipf1.2"

    @property
    def rows(self) -> int:
        return self.T * self.k

    @property
    def waves(self) -> int:
        return -(-self.E // self.experts_per_wave)


# The five named workloads. Seeds are 1000 + workload number.
SHAPES = {
    "tiny": MoeShape("tiny", 256, 512, 1024, 8, 2, 1, 1001, x_std=0.02),
    "dsv3_share": MoeShape("dsv3_share", 4096, 7168, 2048, 32, 8, 4, 1002),
    "qwen3_30b_a3b": MoeShape("qwen3_30b_a3b", 8192, 2048, 768, 128, 8, 16, 1003, bias="normal0.5"),
    "small_m_zipf": MoeShape("small_m_zipf", 512, 4096, 1536, 64, 6, 8, 1004, bias="zipf1.2"),
    "dit_batch": MoeShape("dit_batch", 65536, 4096, 8192, 16, 2, 2, 1005),
}
SHAPE_ORDER = ["tiny", "dsv3_share", "qwen3_30b_a3b", "small_m_zipf", "dit_batch"]


def shape(name: str | None = None, **kw) -> MoeShape:
    """A named workload, or a custom one (``shape(T=.., H=.., ..., seed=..)``)."""
    if name is not None:
        s = SHAPES[name]
        return replace(s, **kw) if kw else s
    kw.setdefault("name", "custom")
    kw.setdefault("experts_per_wave", 1)
    kw.setdefault("seed", 7)
    return MoeShape(**kw)


def flops(s: MoeShape) -> int:
    """Multiply-add work of the two expert GEMMs: 2*rows*H*(2I) + 2*rows*I*H."""
    return 6 * s.T * s.k * s.H * s.I


def nthreads() -> int:
    n = os.environ.get("MOE_GEN_THREADS")
    if n:
        return max(1, int(n))
    try:
        return max(1, min(16, len(os.sched_getaffinity(0))))
    except AttributeError:  # pragma: no cover
        return max(1, min(16, os.cpu_count() or 1))


def _f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 bit patterns, nearest-even (inputs are finite normals)."""
    b = a.view(np.uint32)
    lsb = (b >> np.uint32(16)) & np.uint32(1)
    return ((b + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)


def _draw_normal_bf16(seed: int, tensor: int, n: int, std: float, pool) -> np.ndarray:
    out = np.empty(n, np.uint16)
    nblk = -(-n // _BLOCK)

    def one(b: int) -> None:
        lo, hi = b * _BLOCK, min(n, (b + 1) * _BLOCK)
        g = np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed, spawn_key=(tensor, b))))
        buf = g.standard_normal(hi - lo, dtype=np.float32)
        if std != 1.0:
            buf *= np.float32(std)
        out[lo:hi] = _f32_to_bf16_bits(buf)

    list(pool.map(one, range(nblk)))
    return out


def _draw_normal_f32(seed: int, tensor: int, n: int) -> np.ndarray:
    out = np.empty(n, np.float32)
    for b in range(-(-n // _BLOCK)):
        lo, hi = b * _BLOCK, min(n, (b + 1) * _BLOCK)
        g = np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed, spawn_key=(tensor, b))))
        out[lo:hi] = g.standard_normal(hi - lo, dtype=np.float32)
    return out


def expert_bias(s: MoeShape) -> np.ndarray | None:
    """Per-expert logit bias of the workload (float64), or None."""
    if s.bias == "none":
        return None
    if s.bias == "normal0.5":
        return _draw_normal_f32(s.seed, _T_BIAS, s.E).astype(np.float64) * 0.5
    if s.bias == "zipf1.2":
        # softmax over this bias is exactly Zipf(1.2) over expert ranks e+1
        return -1.2 * np.log(np.arange(1, s.E + 1, dtype=np.float64))
    raise ValueError(f"unknown bias recipe {s.bias!r}")


def generate(s: MoeShape, parts=("x", "logits", "w1", "w2"), threads: int | None = None) -> dict:
    """Draw the workload's tensors.

    Returns a dict with (as requested):
      x      uint16 [T, H]      bf16 bits
      logits float32 [T, E]
      w1     uint16 [E, 2I, H]  bf16 bits; rows [0, I) gate, rows [I, 2I) up
      w2     uint16 [E, H, I]   bf16 bits
    """
    res = {}
    with _cf.ThreadPoolExecutor(threads or nthreads()) as pool:
        if "x" in parts:
            res["x"] = _draw_normal_bf16(s.seed, _T_X, s.T * s.H, s.x_std, pool).reshape(s.T, s.H)
        if "logits" in parts:
            lg = _draw_normal_f32(s.seed, _T_LOGITS, s.T * s.E).reshape(s.T, s.E)
            bias = expert_bias(s)
            if bias is not None:
                lg = (lg.astype(np.float64) + bias[None, :]).astype(np.float32)
            res["logits"] = lg
        if "w1" in parts:
            res["w1"] = _draw_normal_bf16(s.seed, _T_W1, s.E * 2 * s.I * s.H, s.w_std, pool).reshape(
                s.E, 2 * s.I, s.H)
        if "w2" in parts:
            res["w2"] = _draw_normal_bf16(s.seed, _T_W2, s.E * s.H * s.I, s.w_std, pool).reshape(
                s.E, s.H, s.I)
    return res


def describe(s: MoeShape) -> str:
    return (f"{s.name}: T={s.T} H={s.H} I={s.I} E={s.E} k={s.k} W={s.experts_per_wave} "
            f"seed={s.seed} x~N(0,{s.x_std}) w~N(0,{s.w_std}) bias={s.bias}")


def gflop(s: MoeShape) -> float:
    return flops(s) / 1e9



# ---------------------------------------------------------------- attention inputs
# The paper's second workload (Section 4.3): full, non-causal attention of a DiT after the
# Ulysses all-to-all, one GPU holding every token of its share of the heads, head dimension
# 128. Q, K and V are float32 N(0, 1) draws rounded to bfloat16 (stored [B, heads, M, d]).

_T_Q, _T_K, _T_V = 10, 11, 12


@dataclass(frozen=True)
class AttnShape:
    """Shape and seed of one synthetic attention workload."""

    name: str
    B: int
    heads: int  # heads on this GPU
    M: int      # sequence length (every token of the sequence)
    d: int      # head dimension
    seed: int

    @property
    def flops(self) -> int:
        return 4 * self.B * self.heads * self.M * self.M * self.d


ATTN_SHAPES = {
    # a ragged sequence the oracle finishes at once
    "attn_tiny": AttnShape("attn_tiny", 1, 2, 300, 128, 2001),
    # one GPU's share of a 40-head, d = 128 video DiT under 8-way Ulysses: 5 heads, 32K tokens
    "attn_dit_share": AttnShape("attn_dit_share", 1, 5, 32768, 128, 2002),
}


def attn_shape(name: str | None = None, **kw) -> AttnShape:
    if name is not None:
        s = ATTN_SHAPES[name]
        return replace(s, **kw) if kw else s
    kw.setdefault("name", "custom_attn")
    kw.setdefault("seed", 9)
    return AttnShape(**kw)


def generate_attention(s: AttnShape, threads: int | None = None) -> dict:
    """q, k, v: uint16 [B, heads, M, d] bfloat16 bits of N(0, 1) draws."""
    n = s.B * s.heads * s.M * s.d
    shape4 = (s.B, s.heads, s.M, s.d)
    with _cf.ThreadPoolExecutor(threads or nthreads()) as pool:
        return {name: _draw_normal_bf16(s.seed, t, n, 1.0, pool).reshape(shape4)
                for name, t in (("q", _T_Q), ("k", _T_K), ("v", _T_V))}
