"""Helpers for the GPU tests: move seeded inputs to the device, run the four C-ABI calls, and
bring results back as numpy bit patterns. No arithmetic of the layer lives here."""
from __future__ import annotations

import sys

import numpy as np
import torch

import mixture_experts_ffn_dispatch_amd as moe


def note(msg: str) -> None:
    print(msg, file=sys.stderr, flush=True)


def dev_bf16(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()


def host_bits(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def make_cfg(s, **kw) -> moe.MoeConfig:
    base = dict(T=s.T, H=s.H, I=s.I, E=s.E, k=s.k, experts_per_wave=s.experts_per_wave)
    base.update(kw)
    return moe.MoeConfig(**base)


class Device:
    """Inputs of one workload resident on the GPU."""

    def __init__(self, data: dict):
        self.x = dev_bf16(data["x"])
        self.logits = torch.from_numpy(np.ascontiguousarray(data["logits"])).cuda()
        self.w1 = dev_bf16(data["w1"])
        self.w2 = dev_bf16(data["w2"])


def run(cfg: moe.MoeConfig, dev: Device, bufs: dict | None = None, check_status: bool = True,
        gather: bool = False) -> dict:
    """The layer through the C ABI: plan, dispatch, forward, combine; with ``gather`` the
    dispatch is folded into the forward (moe_forward_gather) and no xd buffer exists."""
    bufs = bufs or moe.alloc_buffers(cfg, xd=not gather)
    moe.run_layer(cfg, bufs, dev.x, dev.logits, dev.w1, dev.w2, gather=gather)
    if check_status:
        st = moe.moe_status_read(bufs["ws"])
        assert st == moe.MOE_OK, moe.strerror(st)
    torch.cuda.synchronize()
    return bufs


def fetch(bufs: dict, keys=("topk_ids", "topk_w", "counts", "offsets", "perm", "pos", "act", "yd", "out")) -> dict:
    res = {}
    for k in keys:
        t = bufs[k]
        res[k] = host_bits(t) if t.dtype == torch.bfloat16 else t.cpu().numpy()
    return res


def bf16_f64(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def assert_close_rel(got_bits, ref_bits, rel=1e-2, what=""):
    """max|got - ref| <= rel * max|ref| (the acceptance bound for bf16 outputs)."""
    g, r = bf16_f64(got_bits), bf16_f64(ref_bits)
    assert np.all(np.isfinite(g)), f"{what}: non-finite output"
    scale = np.abs(r).max()
    err = np.abs(g - r).max()
    assert err <= rel * scale, f"{what}: max|err| {err:.3e} > {rel} * {scale:.3e}"
    return err / scale if scale > 0 else 0.0
