"""One GPU's share of an expert-parallel MoE FFN layer on MI355X (gfx950).

The compute lives in ``libmoe.so`` (hand-written HIP kernels behind the C ABI of
``include/moe.h``). This package is the thin Python side: ``_lib`` marshals arguments to the
four calls, and ``alloc_buffers`` / ``run_layer`` allocate device memory with torch and chain
the calls on one stream. Nothing here computes any part of the layer.
"""
from __future__ import annotations

from ._lib import (  # noqa: F401
    MOE_ERR_HIP, MOE_ERR_INVALID_ARG, MOE_ERR_TIMEOUT, MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE,
    MOE_FLAG_FORCE_WAIT_TIMEOUT, MOE_FLAG_NO_WIDE_TAILS, MOE_FLAG_WIDE_TAILS, MOE_FLAG_PLAN_ONE_LAUNCH, MOE_FLAG_TEST_ABSENT_GROUP, MOE_OK, MOE_SCHED_EXPERT_WAVE, MOE_SCHED_INTERLEAVED, MOE_SCHED_AUTO, LIB_PATH,
    MoeConfig, MoeError, abi_version, attn_forward, load, moe_burst_clock_hz, moe_burst_gap, moe_combine, moe_dispatch, moe_forward,
    moe_forward_gather, moe_layer, moe_layer_noalloc, moe_plan, MOE_STATIC_WORKSPACE_BYTES,
    moe_status_read, moe_workspace_layout, moe_workspace_size, strerror,
)


def alloc_routing(cfg: MoeConfig, device="cuda") -> dict:
    """Device buffers for ``moe_routing`` (torch tensors)."""
    import torch

    R = cfg.T * cfg.k
    i32 = dict(dtype=torch.int32, device=device)
    return dict(
        topk_ids=torch.empty((cfg.T, cfg.k), **i32),
        topk_w=torch.empty((cfg.T, cfg.k), dtype=torch.float32, device=device),
        counts=torch.empty(cfg.E, **i32),
        offsets=torch.empty(cfg.E + 1, **i32),
        perm=torch.empty(R, **i32),
        pos=torch.empty(R, **i32),
    )


def alloc_buffers(cfg: MoeConfig, device="cuda", xd=True) -> dict:
    """Routing buffers, workspace and the row buffers (xd unless ``xd=False``, act, yd) plus
    the output."""
    import torch

    R = cfg.T * cfg.k
    bf = dict(dtype=torch.bfloat16, device=device)
    b = alloc_routing(cfg, device)
    b["ws"] = torch.zeros(moe_workspace_size(cfg), dtype=torch.uint8, device=device)
    b["xd"] = torch.empty((R, cfg.H), **bf) if xd else None
    b["act"] = torch.empty((R, cfg.I), **bf)
    b["yd"] = torch.empty((R, cfg.H), **bf)
    b["out"] = torch.empty((cfg.T, cfg.H), **bf)
    return b


def run_layer(cfg: MoeConfig, bufs: dict, x, logits, w1, w2, stream=None, gather=False, fused=False) -> None:
    """plan -> dispatch -> forward -> combine on one stream (asynchronous); with ``gather``,
    plan -> forward_gather (dispatch folded into the Linear-1 loads) -> combine; with
    ``fused``, the single launch of moe_layer."""
    if fused:
        moe_layer(cfg, logits, bufs, x, w1, w2, bufs["act"], bufs["yd"], bufs["out"], bufs["ws"], stream)
        return
    moe_plan(cfg, logits, bufs, bufs["ws"], stream)
    if gather:
        moe_forward_gather(cfg, bufs, x, w1, w2, bufs["act"], bufs["yd"], bufs["ws"], stream)
    else:
        moe_dispatch(cfg, bufs, x, bufs["xd"], stream)
        moe_forward(cfg, bufs["xd"], w1, w2, bufs["act"], bufs["yd"], bufs["ws"], stream)
    moe_combine(cfg, bufs, bufs["yd"], bufs["out"], stream)
