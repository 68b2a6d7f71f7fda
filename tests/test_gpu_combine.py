"""moe_combine on its own, through the C ABI (MI355X).

The router-weighted combine of the X-Stage paper's MoE-layer paragraph: out[t] =
bf16(sum over j ascending of w[t, j] * Yd[pos[t*k + j]]). The routing comes from moe_plan on
random logits, Yd is random bf16, and every output element is compared with a float64
reference: the kernel accumulates in fp32, so the two agree to within one bf16 unit and are
equal almost everywhere. The shapes put 1, 2, 3 (uneven) and 4 column segments per token row
through the kernel, which cuts rows when there are few tokens.
"""
import numpy as np
import pytest
import torch

import moe_workloads as W
from tests.gpu_util import bf16_f64, fetch, make_cfg, note

import mixture_experts_ffn_dispatch_amd as moe

pytestmark = pytest.mark.gpu


def segments(T, H):
    """Column segments per token row, as the library chooses them."""
    cpr = H // 8
    segs = min(4, max(1, -(-4096 // T)))
    while segs > 1 and cpr // segs < 128:
        segs -= 1
    return segs


@pytest.mark.parametrize("T,H,E,k,segs", [
    (100, 4096, 16, 4, 4),
    (100, 3200, 8, 3, 3),   # 400 chunks per row: segments of 134, 134 and 132
    (1500, 2048, 32, 8, 2),
    (1, 8192, 4, 2, 4),
    (5000, 1024, 64, 6, 1),
])
def test_combine_matches_float64_reference(T, H, E, k, segs):
    assert segments(T, H) == segs
    s = W.shape(T=T, H=H, I=64, E=E, k=k, seed=T + H)
    note(f"combine T={T} H={H} E={E} k={k} segments={segs}")
    cfg = make_cfg(s)
    logits = torch.from_numpy(W.generate(s, parts=("logits",))["logits"]).cuda()
    b = moe.alloc_buffers(cfg, xd=False)
    moe.moe_plan(cfg, logits, b, b["ws"])
    gen = torch.Generator(device="cuda").manual_seed(T * 7 + H)
    b["yd"].copy_(torch.randn(b["yd"].shape, generator=gen, device="cuda").to(torch.bfloat16))
    b["out"].fill_(float("nan"))  # every element must be written
    moe.moe_combine(cfg, b, b["yd"], b["out"])
    torch.cuda.synchronize()
    assert moe.moe_status_read(b["ws"]) == moe.MOE_OK
    g = fetch(b, keys=("pos", "topk_w", "yd", "out"))
    yd = bf16_f64(g["yd"])
    w = g["topk_w"].astype(np.float64).reshape(T, k)
    rows = g["pos"].reshape(T, k)
    ref = np.einsum("tj,tjh->th", w, yd[rows])
    out = bf16_f64(g["out"])
    assert np.all(np.isfinite(out))
    # one bf16 unit at |ref|, plus the error bound of a k-term fp32 sum (which matters only
    # where the terms cancel)
    ulp = np.exp2(np.floor(np.log2(np.maximum(np.abs(ref), 1e-30))) - 7)
    acc = np.einsum("tj,tjh->th", np.abs(w), np.abs(yd[rows])) * k * 2.0 ** -23
    err = np.abs(out - ref)
    bad = err > ulp + acc
    if bad.any():
        t, h = np.argwhere(bad)[0]
        raise AssertionError(f"{bad.sum()} elements off, e.g. out[{t},{h}] = {out[t, h]!r} "
                             f"against {ref[t, h]!r} (bound {ulp[t, h] + acc[t, h]:.3e})")
    # RNE of the fp32 sum: the float64 sum rounds to the same bf16 value almost everywhere
    ref_bf16 = torch.from_numpy(ref.astype(np.float32)).to(torch.bfloat16).float().numpy()
    assert np.mean(out == ref_bf16) > 0.99
