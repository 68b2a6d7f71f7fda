"""Host model of moe_plan's MOE_SCHED_AUTO rule (the rule is stated in include/moe.h), for the
tests: from the routed counts and the X-Stage calibration it prices the Expert-Wave order and
the interleaved order at every lead and returns the choice. Burst issue times come from the
Burst-Gap oracle (oracle/burst_gap.py: the max law and the isolated-burst capacity branch).
The arithmetic follows the rule's statement step by step in float64, so it reproduces the
device's choice exactly."""
from __future__ import annotations

import numpy as np

from oracle import burst_gap as BG

MFMA_FLOPS = 1.2e15
STREAM_BYTES = 5.0e12
CACHE_BYTES = 256.0 * 1024 * 1024
LOCAL = (0.927, 6646.0, 31.2)  # t_iss0 us, R GB/s, Q MiB: this GPU's own memory


def calibration(issue_us=0.0, drain_gbps=0.0, capacity_mib=0.0):
    """Seconds, bytes/s, bytes; zeros take the local calibration (as the library does, which
    holds the values as float32 in moe_config)."""
    f = np.float32
    iu = float(f(issue_us)) if issue_us > 0 else LOCAL[0]
    dg = float(f(drain_gbps)) if drain_gbps > 0 else LOCAL[1]
    cm = float(f(capacity_mib)) if capacity_mib > 0 else LOCAL[2]
    return iu * 1e-6, dg * 1e9, cm * 1048576.0


def auto_choice(counts, W, H, I, tile_m, n1, n2, grid, calib):
    """Returns (schedule, lead, prices): schedule 0 = Expert-Wave, 1 = interleaved."""
    counts = np.asarray(counts, np.int64)
    E = len(counts)
    nw = -(-E // W)
    off = np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)
    mblk = -(-counts // tile_m)
    m = np.array([int(mblk[w * W:min(E, (w + 1) * W)].sum()) for w in range(nw)], np.int64)
    a, b = m * n1, m * n2
    PA = np.concatenate([[0], np.cumsum(a)]).astype(np.int64)
    PB = np.concatenate([[0], np.cumsum(b)]).astype(np.int64)
    A, B = int(PA[-1]), int(PB[-1])
    T0, R, Q = calib
    G, BM = float(grid), float(tile_m)
    t1 = G * max(2.0 * BM * 256.0 * H / MFMA_FLOPS, 512.0 * H / STREAM_BYTES)
    t2 = G * max(2.0 * BM * 256.0 * I / MFMA_FLOPS, 512.0 * I / STREAM_BYTES)
    vt = BM * 256.0 * 2.0
    den = A * H + B * I
    need = grid * H * (A + B)
    rows = int(off[E])
    active = int((counts > 0).sum())
    flops = 6.0 * rows * H * I
    nbytes = rows * H * 4.0 + active * 6.0 * H * I + rows * I * 4.0
    hbm_bound = nbytes / STREAM_BYTES > flops / MFMA_FLOPS

    def price(D):
        xs = dep = over = 0.0
        for i in range(nw):
            last = min(i + D, nw - 1) if D > 0 else i
            ws = float(off[min(E, (last + 1) * W)] - off[i * W]) * I * 2.0
            over = max(over, ws - CACHE_BYTES)
            bi = int(b[i])
            if bi == 0:
                continue
            an = int(a[i + D]) if (D > 0 and i + D < nw) else 0
            share = (bi * t2) / (bi * t2 + an * t1)
            kact = max(1.0, float(min(grid, bi)) * share)
            V = kact * vt
            g = t2
            T = max(float(BG.issue_time(V, R, T0, g)), float(BG.isolated_issue_time(V, R, T0, Q)))
            xs += (bi / kact) * (T - T0)
            reach = True
            if D > 0:
                dist = int(PB[i] - PB[max(0, i - D + 1)] + PA[min(i + D, nw)] - PA[min(i + 1, nw)])
                reach = dist * den < need
            if reach:
                dep += t1 / 2.0
        return xs + dep + (over / STREAM_BYTES if hbm_bound else 0.0)

    prices = {0: price(0)}
    best, best_d = None, 1
    for D in range(1, nw + 1):
        prices[D] = price(D)
        if best is None or prices[D] <= best:
            best, best_d = prices[D], D
    if prices[0] < best:
        return 0, 0, prices
    return 1, best_d, prices
