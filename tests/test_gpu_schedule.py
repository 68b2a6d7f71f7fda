"""The expert-wave schedules on the GPU: the tile list moe_plan writes matches a sequential
model of both orders (X-Stage paper, Introduction, expert-wave paragraph: the Expert-Wave
order; Section 4.2: Linear-1 tiles of a later wave placed between the Linear-2 tiles of the
current one), every order is dependency-safe, and all orders, grid sizes, leads and tile
heights give byte-identical results. Also the bounded-wait error path."""
import numpy as np
import pytest
import torch

import moe_workloads as W
from oracle import moe_ref as R
from tests.gpu_util import Device, assert_close_rel, fetch, make_cfg, note, run

import mixture_experts_ffn_dispatch_amd as moe

pytestmark = pytest.mark.gpu

SHAPE = W.shape(T=700, H=256, I=384, E=12, k=3, experts_per_wave=2, seed=41, x_std=1.0, w_std=0.05)


@pytest.fixture(scope="module")
def workload():
    d = W.generate(SHAPE)
    d["logits"][:, 7] -= 40.0  # one expert without rows, so one wave has a gap
    return d, Device(d)


BLOCK_M, BLOCK_N, UNIT = 4, 8, 32  # tile blocks of one expert; units of consecutive tiles


def run_tiles(phase, wave_experts, mb_of, n):
    """One run's tiles in emission order: per expert, blocks of up to BLOCK_M m-blocks x
    BLOCK_N n-tiles, n-tile major inside a block."""
    out = []
    for e in wave_experts:
        mbs = mb_of[e]
        for m0 in range(0, len(mbs), BLOCK_M):
            for n0 in range(0, n, BLOCK_N):
                for nt in range(n0, min(n, n0 + BLOCK_N)):
                    for mb in mbs[m0:m0 + BLOCK_M]:
                        out.append((phase, mb, nt))
    return out


def model_order(counts, tile_m, n1, n2, W_, schedule, lead):
    """Sequential model: cut every run into units of UNIT tiles and walk the waves, emitting
    one unit at a time. Returns the units in list order (lists of (phase, m-block, n-tile))."""
    E = len(counts)
    mb_of = []  # m-block ids per expert, in expert order
    nxt = 0
    for e in range(E):
        nb = -(-int(counts[e]) // tile_m)
        mb_of.append(list(range(nxt, nxt + nb)))
        nxt += nb
    nw = -(-E // W_)

    def units(run):
        return [run[i:i + UNIT] for i in range(0, len(run), UNIT)]

    L1 = [units(run_tiles(0, range(w * W_, min(E, (w + 1) * W_)), mb_of, n1)) for w in range(nw)]
    L2 = [units(run_tiles(1, range(w * W_, min(E, (w + 1) * W_)), mb_of, n2)) for w in range(nw)]
    if schedule == moe.MOE_SCHED_EXPERT_WAVE:
        return [u for w in range(nw) for u in L1[w] + L2[w]]
    D = max(1, lead)
    seq = [u for w in range(min(D, nw)) for u in L1[w]]
    for i in range(nw):
        l2 = L2[i]
        l1 = L1[i + D] if i + D < nw else []
        done = 0
        for j, u in enumerate(l2, 1):
            seq.append(u)
            target = j * len(l1) // len(l2)
            while done < target:
                seq.append(l1[done])
                done += 1
        seq.extend(l1[done:])
    return seq


def decode(raw):
    raw = raw.astype(np.int64) & 0xFFFFFFFF
    return [(int(t >> 31), int((t >> 12) & 0x7FFFF), int(t & 0xFFF)) for t in raw]


def read_tasks(cfg, bufs):
    L = moe.moe_workspace_layout(cfg)
    ws = bufs["ws"].cpu().numpy()
    hdr = ws[:128].view(np.int32)
    n, nunits = int(hdr[2]), int(hdr[16])
    tasks = decode(ws[L["tasks"]:L["tasks"] + 4 * n].view(np.int32))
    starts = ws[L["unit_start"]:L["unit_start"] + 4 * (nunits + 1)].view(np.int32).tolist()
    gunits = ws[L["group_units"]:L["group_units"] + 4 * nunits].view(np.int32).tolist()
    goff = hdr[17:26].tolist()
    return tasks, starts, gunits, goff, L


def model_groups(units, groups=8):
    """Units of each phase dealt round-robin to the groups in list order."""
    seen = [0, 0]
    lists = [[] for _ in range(groups)]
    for u, tiles in enumerate(units):
        ph = tiles[0][0]
        lists[seen[ph] % groups].append(u)
        seen[ph] += 1
    return lists


# long runs: several full units per run, so the unit-level merge is exercised
LONG = W.shape(T=2048, H=256, I=512, E=8, k=4, experts_per_wave=2, seed=43, x_std=1.0, w_std=0.05)


@pytest.fixture(scope="module")
def long_workload():
    return Device(W.generate(LONG))


# Many expert waves: the planner builds its per-wave table on one wavefront up to 64 waves and
# with the whole workgroup above that; EDGE sits at the limit, MANY above it (some waves empty).
EDGE = W.shape(T=600, H=128, I=128, E=128, k=4, experts_per_wave=2, seed=46, x_std=1.0, w_std=0.05)
MANY = W.shape(T=600, H=128, I=128, E=136, k=4, experts_per_wave=2, seed=45, x_std=1.0, w_std=0.05)


@pytest.fixture(scope="module")
def wave_workloads():
    many = W.generate(MANY)
    many["logits"][:, 100:102] -= 40.0  # experts 100 and 101 get no rows: wave 50 is empty
    return {"edge": Device(W.generate(EDGE)), "many": Device(many)}


def auto_lead(counts, tile_m, n1, n2, W_, H, I, grid):
    """The lead moe_plan picks for lead_waves = 0: the smallest D at which, for every wave i
    with Linear-2 tiles, the tiles between the last Linear-1 tile of wave i and its first
    Linear-2 tile (in the interleaved list) cover G * t1 / t_mean positions (durations
    proportional to K = H, I), else nw. Counted directly on the model's list."""
    E = len(counts)
    nw = -(-E // W_)
    mb = [-(-int(c) // tile_m) for c in counts]
    a = [sum(mb[w * W_:(w + 1) * W_]) * n1 for w in range(nw)]
    b = [sum(mb[w * W_:(w + 1) * W_]) * n2 for w in range(nw)]
    A, B = sum(a), sum(b)
    need = grid * H * (A + B)
    den = A * H + B * I
    for D in range(1, nw + 1):
        seq = []  # (phase, wave) per tile in the interleaved list, tiles merged as whole runs
        seq += [(0, w) for w in range(min(D, nw)) for _ in range(a[w])]
        for i in range(nw):
            seq += [(1, i)] * b[i]
            if i + D < nw:
                seq += [(0, i + D)] * a[i + D]
        ok = True
        for i in range(nw):
            if b[i] == 0:
                continue
            last_l1 = max(p for p, t in enumerate(seq) if t == (0, i)) if a[i] else -1
            first_l2 = min(p for p, t in enumerate(seq) if t == (1, i))
            if (first_l2 - last_l1 - 1) * den < need:
                ok = False
                break
        if ok:
            return D
    return max(nw, 1)


@pytest.mark.parametrize("schedule,lead", [(0, 0), (1, 1), (1, 2), (1, 3), (1, 9), (1, 0)])
@pytest.mark.parametrize("tile_m", [32, 128, 256])
@pytest.mark.parametrize("which", ["short", "long", "edge", "many"])
def test_task_list_matches_model(workload, long_workload, wave_workloads, which, schedule, lead, tile_m):
    shape, dev = {"short": (SHAPE, workload[1]), "long": (LONG, long_workload), "edge": (EDGE, None),
                  "many": (MANY, None)}[which]
    dev = dev or wave_workloads[which]
    # with 256-row tiles, force wide last m-blocks (the long shape would not choose them)
    flags = moe.MOE_FLAG_WIDE_TAILS if tile_m == 256 else 0
    cfg = make_cfg(shape, schedule=schedule, lead_waves=lead, tile_m=tile_m, flags=flags)
    note(f"task list {which} schedule={schedule} lead={lead} tile_m={tile_m} flags={flags}")
    b = run(cfg, dev)
    tasks, starts, gunits, goff, L = read_tasks(cfg, b)
    counts = b["counts"].cpu().numpy()
    hdr = b["ws"][:256].cpu().numpy().view(np.int32)
    used_lead, grid = int(hdr[26]), int(hdr[27])
    if schedule == moe.MOE_SCHED_EXPERT_WAVE:
        assert used_lead == 0
    elif lead > 0:
        nw = -(-shape.E // shape.experts_per_wave)
        assert used_lead == min(lead, nw)
    else:
        assert grid >= 1
        assert used_lead == auto_lead(counts, L["tile_m"], L["n1_tiles"], L["n2_tiles"], shape.experts_per_wave,
                                      shape.H, shape.I, grid)
        lead = used_lead
    units = model_order(counts, L["tile_m"], L["n1_tiles"], L["n2_tiles"], shape.experts_per_wave, schedule, lead)
    assert tasks == [t for u in units for t in u]
    # the unit table marks where each unit starts, the last entry is the list length
    expect_starts = [0]
    for u in units:
        expect_starts.append(expect_starts[-1] + len(u))
    assert starts == expect_starts
    # each locality group's unit list, groups one after another
    lists = model_groups(units)
    assert goff == [sum(len(x) for x in lists[:g]) for g in range(9)]
    assert gunits == [u for x in lists for u in x]
    # each group's tile records: its units in its order, UNIT slots per unit holding the unit's
    # tiles with the m-block's expert, first dispatched row and row count; spare slots no-op
    ws = b["ws"].cpu().numpy()
    gtoff = hdr[32:41].tolist()
    assert gtoff == [UNIT * g for g in goff]
    recs = ws[L["group_tasks"]:L["group_tasks"] + 16 * UNIT * len(gunits)].view(np.int32).reshape(-1, 4)
    assert len(gunits) * UNIT <= L["max_slots"]
    offsets = b["offsets"].cpu().numpy()
    first_mb, nxt = [], 0
    for e in range(shape.E):
        first_mb.append(nxt)
        nxt += -(-int(counts[e]) // L["tile_m"])
    NOP, WIDE, ONCE = 0x7FFFFFFE, 1 << 30, 1 << 29
    tm = L["tile_m"]
    mb_expert = [e for e in range(shape.E) for _ in range(-(-int(counts[e]) // tm))]
    n_wide = 0
    for slot, u in enumerate(gunits):
        block = recs[slot * UNIT:(slot + 1) * UNIT]
        tiles = units[u]
        assert all(int(r[0]) == NOP for r in block[len(tiles):])
        for (ph, mb, nt), rec in zip(tiles, block[:len(tiles)].tolist()):
            e = mb_expert[mb]
            i = mb - first_mb[e]
            expect_rows = min(tm, int(counts[e]) - i * tm)
            # with 256-row tiles an m-block of at most 128 rows is wide: its even n-tiles cover
            # two, its odd ones hold no-op records
            wide = tm == 256 and 2 * expect_rows <= tm
            if wide and nt % 2:
                assert rec[0] == NOP
                continue
            n_wide += wide
            assert tuple(decode(np.array([rec[0]]))[0]) == (ph, mb, nt)
            assert rec[1] == e and rec[2] == offsets[e] + i * tm
            # an expert's only m-block is marked: its weight rows are read by its tiles alone
            once = -(-int(counts[e]) // tm) == 1
            assert rec[3] == expect_rows | (WIDE if wide else 0) | (ONCE if once else 0)
    if tm == 256 and which == "long":
        assert n_wide > 0  # five of its experts end in a block of at most 128 rows
    # dependency safety: every Linear-2 tile comes after all Linear-1 tiles of its m-block
    seen = {}
    for ph, mb, _ in tasks:
        if ph == 0:
            seen[mb] = seen.get(mb, 0) + 1
        else:
            assert seen.get(mb, 0) == L["n1_tiles"]


def test_all_orders_grids_and_tiles_byte_identical(workload):
    d, dev = workload
    o = R.moe_layer(d["x"], d["logits"], d["w1"], d["w2"], SHAPE.k)
    ref = None
    variants = [dict(schedule=0), dict(schedule=1), dict(schedule=1, lead_waves=2),
                dict(schedule=1, lead_waves=6), dict(schedule=0, num_workgroups=1),
                dict(schedule=1, num_workgroups=3), dict(schedule=1, num_workgroups=1000),
                dict(tile_m=32), dict(tile_m=64), dict(tile_m=128), dict(tile_m=256, schedule=1)]
    for v in variants:
        note(f"invariance variant {v}")
        g = fetch(run(make_cfg(SHAPE, **v), dev), keys=("act", "yd", "out", "perm"))
        np.testing.assert_array_equal(g["perm"], o["perm"])
        if ref is None:
            ref = g
            continue
        for key in ("act", "yd", "out"):
            assert np.array_equal(g[key], ref[key]), (v, key)


# Wide last m-blocks: with 256-row tiles an m-block of at most 128 rows runs as tiles of 512
# weight rows by 128 token rows. Shapes with some experts ending in such a block and others
# not, even and odd (and partial) n-tile counts.
WIDE_SHAPES = [
    # counts about 1024: five experts end in a block of at most 128 rows; n1 = 4, n2 = 1; the
    # default would not choose wide blocks here (T k > 768 E)
    LONG,
    # counts about 400: two experts end in a block of at most 128 rows; n1 = 3, n2 = 2; chosen
    # by default (T k <= 768 E)
    W.shape(T=1200, H=384, I=320, E=6, k=2, experts_per_wave=2, seed=44, x_std=1.0, w_std=0.05),
]


def wide_records(cfg, bufs):
    """Number of tile records the plan marked wide (bit 30 of the row count)."""
    L = moe.moe_workspace_layout(cfg)
    hdr = bufs["ws"][:256].cpu().numpy().view(np.int32)
    n = int(hdr[40])  # end of the last group's record list
    recs = bufs["ws"][L["group_tasks"]:L["group_tasks"] + 16 * n].cpu().numpy().view(np.int32).reshape(-1, 4)
    return int(((recs[:, 0] != 0x7FFFFFFE) & ((recs[:, 3] & (1 << 30)) != 0)).sum())


@pytest.mark.parametrize("which", [0, 1])
def test_wide_tail_tiles_byte_identical(which):
    shape = WIDE_SHAPES[which]
    d = W.generate(shape)
    dev = Device(d)
    o = R.moe_layer(d["x"], d["logits"], d["w1"], d["w2"], shape.k)
    tails = o["counts"] % 256
    assert ((tails > 0) & (tails <= 128)).any() and ((tails == 0) | (tails > 128)).any()
    # regular tiles everywhere first, then wide ones on the shared cursor (grid 1) and on the
    # group lists, in both orders, with rows from xd and gathered from x
    NO, ON = moe.MOE_FLAG_NO_WIDE_TAILS, moe.MOE_FLAG_WIDE_TAILS
    variants = [dict(flags=NO, schedule=1), dict(flags=ON, schedule=1), dict(flags=ON, schedule=0),
                dict(flags=ON, schedule=0, num_workgroups=1), dict(flags=ON, schedule=1, num_workgroups=3),
                dict(flags=ON, schedule=1, lead_waves=2, gather=True), dict(flags=ON, schedule=0, gather=True),
                dict(flags=NO, schedule=0, num_workgroups=1, gather=True), dict(schedule=1)]
    ref = None
    for v in variants:
        v = dict(v)
        gather = v.pop("gather", False)
        note(f"wide tails {shape.T}x{shape.E} variant {v} gather={gather}")
        cfg = make_cfg(shape, tile_m=256, **v)
        bufs = run(cfg, dev, gather=gather)
        flags = v.get("flags", 0)
        if flags == ON:  # off by default
            assert wide_records(cfg, bufs) > 0
        else:
            assert wide_records(cfg, bufs) == 0
        g = fetch(bufs, keys=("act", "yd", "out", "perm"))
        np.testing.assert_array_equal(g["perm"], o["perm"])
        if ref is None:
            ref = g
            for key, what in (("act", "a"), ("yd", "yd"), ("out", "out")):
                assert_close_rel(g[key], o[what], what=key)
            continue
        for key in ("act", "yd", "out"):
            assert np.array_equal(g[key], ref[key]), (v, key)


def test_repeated_calls_reuse_buffers(workload):
    d, dev = workload
    cfg = make_cfg(SHAPE, schedule=1)
    bufs = moe.alloc_buffers(cfg)
    first = fetch(run(cfg, dev, bufs), keys=("yd", "out"))
    # forward alone again on the same plan, then the whole layer again
    moe.moe_forward(cfg, bufs["xd"], dev.w1, dev.w2, bufs["act"], bufs["yd"], bufs["ws"])
    assert moe.moe_status_read(bufs["ws"]) == moe.MOE_OK
    again = fetch(run(cfg, dev, bufs), keys=("yd", "out"))
    for key in first:
        assert np.array_equal(first[key], again[key])


@pytest.mark.parametrize("wide", [False, True])
def test_bounded_wait_reports_timeout_and_recovers(workload, wide):
    d, dev = workload
    small = W.shape(T=64, H=128, I=128, E=4, k=2, experts_per_wave=2, seed=42)
    ds = W.generate(small)
    dv = Device(ds)
    # wide: 256-row tiles with every (short) m-block wide, on the kernel instance that runs them
    extra = dict(tile_m=256) if wide else {}
    flags = moe.MOE_FLAG_WIDE_TAILS if wide else 0
    cfg = make_cfg(small, flags=flags | moe.MOE_FLAG_FORCE_WAIT_TIMEOUT, spin_limit=20, **extra)
    bufs = moe.alloc_buffers(cfg)
    note(f"forced bounded-wait timeout wide={wide}")
    run(cfg, dv, bufs, check_status=False)
    assert moe.moe_status_read(bufs["ws"]) == moe.MOE_ERR_TIMEOUT
    cfg_ok = make_cfg(small, flags=flags, **extra)
    run(cfg_ok, dv, bufs)  # asserts MOE_OK
    o = R.moe_layer(ds["x"], ds["logits"], ds["w1"], ds["w2"], small.k)
    g = fetch(bufs, keys=("out",))
    from tests.gpu_util import assert_close_rel
    assert_close_rel(g["out"], o["out"], what="after recovery")


def test_repeated_calls_reuse_buffers_wide():
    # the wide-capable instance resets its counters and cursors for the next call as well
    shape = WIDE_SHAPES[1]
    d = W.generate(shape)
    dev = Device(d)
    cfg = make_cfg(shape, schedule=1, tile_m=256, flags=moe.MOE_FLAG_WIDE_TAILS)
    bufs = moe.alloc_buffers(cfg)
    note("repeated calls, wide last m-blocks")
    first = fetch(run(cfg, dev, bufs), keys=("yd", "out"))
    assert wide_records(cfg, bufs) > 0
    for _ in range(2):
        moe.moe_forward(cfg, bufs["xd"], dev.w1, dev.w2, bufs["act"], bufs["yd"], bufs["ws"])
        assert moe.moe_status_read(bufs["ws"]) == moe.MOE_OK
    again = fetch(run(cfg, dev, bufs), keys=("yd", "out"))
    for key in first:
        assert np.array_equal(first[key], again[key])


def test_dispatch_on_side_stream_orders_with_plan(workload):
    d, dev = workload
    cfg = make_cfg(SHAPE)
    s = torch.cuda.Stream()
    bufs = moe.alloc_buffers(cfg)
    with torch.cuda.stream(s):
        moe.run_layer(cfg, bufs, dev.x, dev.logits, dev.w1, dev.w2, stream=s)
    assert moe.moe_status_read(bufs["ws"], stream=s) == moe.MOE_OK
    g = fetch(bufs, keys=("out",))
    ref = fetch(run(cfg, dev), keys=("out",))
    assert np.array_equal(g["out"], ref["out"])
