"""Parity at the five named workloads' full sizes, in the launch configuration the benchmark
times (automatic tile height and grid, both schedules). Routing and the dispatched rows are
checked in full; A, Yd and the output on sampled tokens that the oracle computes one by one
(rows of a GEMM are independent, so a token's rows need only its own inputs)."""
import numpy as np
import pytest
import torch

import moe_workloads as W
from oracle import moe_ref as R
from tests.gpu_util import Device, assert_close_rel, bf16_f64, fetch, make_cfg, note, run

import mixture_experts_ffn_dispatch_amd as moe

pytestmark = pytest.mark.gpu

SAMPLED_TOKENS = 12


@pytest.mark.parametrize("name", ["tiny", "dsv3_share", "qwen3_30b_a3b", "small_m_zipf", "dit_batch"])
def test_full_size_sampled_parity(name):
    s = W.shape(name)
    note(f"full size {W.describe(s)}: generating")
    d = W.generate(s)
    dev = Device(d)
    note("  gpu run (expert-wave order)")
    cfg = make_cfg(s, schedule=moe.MOE_SCHED_EXPERT_WAVE)
    b = run(cfg, dev)
    note("  gpu run (interleaved order)")
    b2 = run(make_cfg(s, schedule=moe.MOE_SCHED_INTERLEAVED), dev)
    for key in ("act", "yd", "out"):
        assert torch.equal(b[key].view(torch.int16), b2[key].view(torch.int16)), key
    note("  gpu run (interleaved order, dispatch folded into the Linear-1 loads)")
    b3 = run(make_cfg(s, schedule=moe.MOE_SCHED_INTERLEAVED), dev, gather=True)
    for key in ("act", "yd", "out"):
        assert torch.equal(b2[key].view(torch.int16), b3[key].view(torch.int16)), key
    del b3

    note("  oracle routing")
    ids, w = R.route(d["logits"], s.k)
    counts, offsets, perm, pos = R.plan(ids, s.E)
    g = fetch(b, keys=("topk_ids", "topk_w", "counts", "offsets", "perm", "pos"))
    np.testing.assert_array_equal(g["topk_ids"], ids)
    np.testing.assert_allclose(g["topk_w"], w, rtol=0, atol=2.0 ** -20)
    np.testing.assert_array_equal(g["counts"], counts)
    np.testing.assert_array_equal(g["offsets"], offsets)
    np.testing.assert_array_equal(g["perm"], perm)
    np.testing.assert_array_equal(g["pos"], pos)
    # dispatched rows: every row is the bit copy of its token (gathered by torch from the
    # oracle's permutation)
    src = torch.from_numpy(perm.astype(np.int64) // s.k).cuda()
    assert torch.equal(b["xd"].view(torch.int16), dev.x.view(torch.int16).index_select(0, src))

    note("  oracle on sampled tokens")
    rng = np.random.default_rng(s.seed)
    toks = np.sort(rng.choice(s.T, size=min(SAMPLED_TOKENS, s.T), replace=False))
    a_ref = np.zeros((len(toks), s.k, s.I), np.uint16)
    y_ref = np.zeros((len(toks), s.k, s.H), np.uint16)
    for e in np.unique(ids[toks]):
        sel = [(i, j) for i, t in enumerate(toks) for j in range(s.k) if ids[t, j] == e]
        rows = d["x"][[toks[i] for i, _ in sel]]
        a, y = R.expert_ffn(rows, d["w1"][e], d["w2"][e])
        for r, (i, j) in enumerate(sel):
            a_ref[i, j], y_ref[i, j] = a[r], y[r]
    out_ref = np.zeros((len(toks), s.H), np.uint16)
    for i, t in enumerate(toks):
        acc = np.zeros(s.H, np.float64)
        for j in range(s.k):
            acc += float(w[t, j]) * bf16_f64(y_ref[i, j])
        out_ref[i] = R.f64_to_bf16_bits(R.bf16_round(acc))
    rows = pos.reshape(s.T, s.k)[toks]
    act = b["act"].view(torch.int16).cpu().numpy().view(np.uint16)
    yd = b["yd"].view(torch.int16).cpu().numpy().view(np.uint16)
    out = b["out"].view(torch.int16).cpu().numpy().view(np.uint16)
    assert_close_rel(act[rows.reshape(-1)], a_ref.reshape(-1, s.I), what="A (sampled)")
    for i in range(len(toks)):
        for j in range(s.k):
            assert_close_rel(yd[rows[i, j]], y_ref[i, j], what=f"Yd token {toks[i]} slot {j}")
    assert_close_rel(out[toks], out_ref, what="out (sampled)")
    note("  ok")


@pytest.mark.parametrize("name", ["dsv3_share", "qwen3_30b_a3b"])
def test_full_size_wide_blocks_byte_identical(name):
    # wide last m-blocks (forced on, and off) at full size, in the benchmark's launch
    # configuration: the long K loops and the many tiles give the same bytes either way
    s = W.shape(name)
    note(f"wide last m-blocks, full size {W.describe(s)}")
    dev = Device(W.generate(s))
    outs = []
    for flags in (moe.MOE_FLAG_WIDE_TAILS, moe.MOE_FLAG_NO_WIDE_TAILS):
        b = run(make_cfg(s, schedule=moe.MOE_SCHED_INTERLEAVED, flags=flags), dev, gather=True)
        outs.append({k: b[k] for k in ("act", "yd", "out")})
    for key in ("act", "yd", "out"):
        assert torch.equal(outs[0][key].view(torch.int16), outs[1][key].view(torch.int16)), key
