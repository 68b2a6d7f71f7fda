"""Parity at the five named workloads' full sizes, in the launch configuration the benchmark
times (automatic tile height, grid, order and lead, dispatch folded into the Linear-1 loads),
with the interleaved order, the Expert-Wave order and the separate dispatch byte-identical to
it.

Routing, the plan and the dispatched rows are checked in full. A, Yd and the output are
compared with the oracle element by element: on every row for four workloads, and for the
largest (dit_batch, 131072 dispatched rows of H = 4096, I = 8192) on the first and last row of
every m-block, every row of each expert's last m-block, and all k rows of every token owning
one of those rows, so that the oracle's own combine gives those tokens' outputs."""
import numpy as np
import pytest
import torch

import moe_workloads as W
from oracle import moe_ref as R
from tests.gpu_util import Device, assert_close_rel, fetch, make_cfg, note, run

import mixture_experts_ffn_dispatch_amd as moe

pytestmark = pytest.mark.gpu

NOP, WIDE = 0x7FFFFFFE, 1 << 30


def run_filled(cfg, dev, gather=False):
    """The layer on buffers whose A, Yd and output start as NaN, so an element no tile wrote
    shows up."""
    b = moe.alloc_buffers(cfg, xd=not gather)
    for key in ("act", "yd", "out"):
        b[key].fill_(float("nan"))
    run(cfg, dev, b, gather=gather)
    for key in ("act", "yd", "out"):
        assert not torch.isnan(b[key]).any(), f"{key}: elements never written"
    return b


def check_plan(cfg, b):
    """The plan at full size: the tile list holds every (phase, m-block, n-tile) once, each
    Linear-2 tile after the Linear-1 tiles of its m-block; the group record lists hold every
    tile the kernel runs exactly once (the odd n-tiles of wide m-blocks are no-ops), each with
    its m-block's expert, first row and rows."""
    L = moe.moe_workspace_layout(cfg)
    ws = b["ws"].cpu().numpy()
    hdr = ws[:256].view(np.int32)
    n, nmb, n1, n2 = (int(hdr[i]) for i in (2, 3, 5, 6))
    assert n == nmb * (n1 + n2) and n1 == L["n1_tiles"] and n2 == L["n2_tiles"]

    def decode(words):
        w = words.astype(np.int64) & 0xFFFFFFFF
        return w >> 31, (w >> 12) & 0x7FFFF, w & 0xFFF

    ph, mb, nt = decode(ws[L["tasks"]:L["tasks"] + 4 * n].view(np.int32))
    assert np.all(mb < nmb) and np.all(nt < np.where(ph == 1, n2, n1))
    key = (ph * nmb + mb) * max(n1, n2) + nt
    assert len(np.unique(key)) == n and np.sum(ph == 0) == nmb * n1
    pos = np.arange(n)
    last_l1, first_l2 = np.full(nmb, -1), np.full(nmb, n)
    np.maximum.at(last_l1, mb[ph == 0], pos[ph == 0])
    np.minimum.at(first_l2, mb[ph == 1], pos[ph == 1])
    assert np.all(last_l1 < first_l2), "a Linear-2 tile precedes a Linear-1 tile of its m-block"

    table = {k: ws[L[k]:L[k] + 4 * nmb].view(np.int32) for k in ("mblk_expert", "mblk_row0", "mblk_rows")}
    recs = ws[L["group_tasks"]:L["group_tasks"] + 16 * int(hdr[40])].view(np.int32).reshape(-1, 4)
    real = recs[recs[:, 0] != NOP]
    rph, rmb, rnt = decode(real[:, 0])
    wide = (table["mblk_rows"] & WIDE) != 0
    runs = ~(wide[mb] & (nt % 2 == 1))  # tiles the kernel runs: all but odd n-tiles of wide blocks
    assert len(real) == np.sum(runs)
    assert np.array_equal(np.sort((rph * nmb + rmb) * max(n1, n2) + rnt), np.sort(key[runs]))
    assert np.array_equal(real[:, 1], table["mblk_expert"][rmb])
    assert np.array_equal(real[:, 2], table["mblk_row0"][rmb])
    assert np.array_equal(real[:, 3], table["mblk_rows"][rmb])


FULL_ROWS = ["tiny", "dsv3_share", "qwen3_30b_a3b", "small_m_zipf"]
SAMPLED_ROWS = ["dit_batch"]


def mblock_rows(offsets, tile_m):
    """Dispatched rows that cover every m-block of every expert: its first and last row, and
    all rows of an expert's last m-block when it is partial."""
    rows = []
    for e in range(len(offsets) - 1):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        for m in range(lo, hi, tile_m):
            rows += [m, min(m + tile_m, hi) - 1]
        if (hi - lo) % tile_m:
            rows += range(lo + (hi - lo) // tile_m * tile_m, hi)
    return np.unique(np.asarray(rows, np.int64))


def oracle_rows(d, s, perm, offsets, rows):
    """A and Yd of the given (sorted) dispatched rows from the oracle's per-expert FFN."""
    xd = R.dispatch(d["x"], perm[rows], s.k)
    experts = np.searchsorted(offsets, rows, side="right") - 1
    a = np.empty((len(rows), s.I), np.uint16)
    y = np.empty((len(rows), s.H), np.uint16)
    for e in np.unique(experts):
        sel = experts == e
        a[sel], y[sel] = R.expert_ffn(xd[sel], d["w1"][e], d["w2"][e])
    return a, y, experts


def compare_per_expert(got, ref, experts, what):
    """max|gpu - ref| <= 1e-2 max|ref| over each expert's rows; returns the worst ratio."""
    worst = 0.0
    for e in np.unique(experts):
        sel = experts == e
        worst = max(worst, assert_close_rel(got[sel], ref[sel], what=f"{what} expert {e}"))
    return worst


@pytest.mark.parametrize("name", FULL_ROWS + SAMPLED_ROWS)
def test_full_size_parity(name):
    s = W.shape(name)
    note(f"full size {W.describe(s)}: generating")
    d = W.generate(s)
    dev = Device(d)
    note("  gpu run (automatic order, dispatch folded into the Linear-1 loads: the benchmark's launch)")
    cfg = make_cfg(s, schedule=moe.MOE_SCHED_AUTO)
    b = run_filled(cfg, dev, gather=True)
    check_plan(cfg, b)
    note("  gpu run (interleaved order with the D_knee lead, separate dispatch)")
    b2 = run_filled(make_cfg(s, schedule=moe.MOE_SCHED_INTERLEAVED), dev)
    for key in ("act", "yd", "out"):
        assert torch.equal(b[key].view(torch.int16), b2[key].view(torch.int16)), key
    # dispatched rows: every row is the bit copy of its token (gathered by torch from the
    # oracle's permutation, below)
    xd_gpu = b2["xd"]
    del b2
    note("  gpu run (expert-wave order, separate dispatch)")
    cfg_ew = make_cfg(s, schedule=moe.MOE_SCHED_EXPERT_WAVE)
    b3 = run_filled(cfg_ew, dev)
    check_plan(cfg_ew, b3)
    for key in ("act", "yd", "out"):
        assert torch.equal(b[key].view(torch.int16), b3[key].view(torch.int16)), key
    del b3

    note("  oracle routing and plan")
    ids, w = R.route(d["logits"], s.k)
    counts, offsets, perm, pos = R.plan(ids, s.E)
    g = fetch(b)
    np.testing.assert_array_equal(g["topk_ids"], ids)
    np.testing.assert_allclose(g["topk_w"], w, rtol=0, atol=2.0 ** -20)
    np.testing.assert_array_equal(g["counts"], counts)
    np.testing.assert_array_equal(g["offsets"], offsets)
    np.testing.assert_array_equal(g["perm"], perm)
    np.testing.assert_array_equal(g["pos"], pos)
    src = torch.from_numpy(perm.astype(np.int64) // s.k).cuda()
    assert torch.equal(xd_gpu.view(torch.int16), dev.x.view(torch.int16).index_select(0, src))
    del xd_gpu, src

    if name in FULL_ROWS:
        note("  oracle: the whole layer")
        o = R.moe_layer(d["x"], d["logits"], d["w1"], d["w2"], s.k)
        experts = np.searchsorted(offsets, np.arange(s.T * s.k), side="right") - 1
        ea = compare_per_expert(g["act"], o["a"], experts, "A")
        ey = compare_per_expert(g["yd"], o["yd"], experts, "Yd")
        eo = assert_close_rel(g["out"], o["out"], what="out")
        note(f"  every row: A {ea:.2e}, Yd {ey:.2e}, out {eo:.2e} of max|ref|")
        return

    tile_m = moe.moe_workspace_layout(cfg)["tile_m"]
    rows = mblock_rows(offsets, tile_m)
    tokens = np.unique(perm[rows] // s.k)
    slot_rows = pos.reshape(s.T, s.k)[tokens]  # [tokens, k]
    rows = np.unique(np.concatenate([rows, slot_rows.reshape(-1)]))
    note(f"  oracle: {len(rows)} of {s.T * s.k} dispatched rows ({len(tokens)} tokens)")
    a_ref, y_ref, experts = oracle_rows(d, s, perm, offsets, rows)
    ea = compare_per_expert(g["act"][rows], a_ref, experts, "A")
    ey = compare_per_expert(g["yd"][rows], y_ref, experts, "Yd")
    # the oracle's combine over these tokens: their k Yd rows in slot order
    y_tok = y_ref[np.searchsorted(rows, slot_rows.reshape(-1))]
    out_ref = R.combine(y_tok, w[tokens], np.arange(len(tokens) * s.k), len(tokens), s.k)
    eo = assert_close_rel(g["out"][tokens], out_ref, what="out")
    note(f"  sampled rows: A {ea:.2e}, Yd {ey:.2e}, out {eo:.2e} of max|ref|")


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
