"""Burst-Gap calibration of this GPU's own memory path (the X-Stage paper's Section 3, run as
its local-memory control), and the design test of the paper's Section 4 applied to the
persistent GEMM's Linear-2 epilogue bursts.

The measurements run in ``libmoe`` (``moe_burst_gap``); this module drives the sweeps, turns
counter readings into times and fits the three calibrated quantities of the Burst-Gap model:

  t_iss0  backpressure-free issue time of a burst (the large-gap plateau of the issue time)
  r       effective drain rate: zero-gap periodic bursts settle at period = V / r
  q       effective outstanding capacity: isolated bursts issue in t_iss0 until
          V - r * t_iss0 exceeds q, then in (V - q) / r. Here t_iss0 of a small isolated burst
          grows with its size (the path absorbs it at an aggregate rate s), so q is fitted on
          the largest bursts and the knee is where the line V / s meets (V - q) / r.

    python -m mixture_experts_ffn_dispatch_amd.xstage [--producers K] [--json out.json]
"""
from __future__ import annotations

import argparse
import json
import sys

import numpy as np

KIB = 1024
MIB = 1024 * KIB


# ------------------------------------------------------------------ model and fitting (host)

def predict_issue(v, r, t_iss0, gap):
    """Issue time of periodic bursts: the floor t_iss0, or the drain backlog V / r - G."""
    return np.maximum(t_iss0, np.asarray(v, float) / r - np.asarray(gap, float))


def predict_period(v, r, t_iss0, gap):
    """Period of periodic bursts: drain-limited V / r, or issue-plus-gap t_iss0 + G."""
    return np.maximum(np.asarray(v, float) / r, t_iss0 + np.asarray(gap, float))


def predict_isolated(v, r, t_iss0, q):
    """Issue time of one burst into an empty path: t_iss0 up to the knee, then (V - q) / r."""
    v = np.asarray(v, float)
    return np.where(v - r * t_iss0 <= q, t_iss0, (v - q) / r)


def fit_drain_rate(volumes, periods) -> float:
    """Least-squares slope through the origin of period = V / r over drain-dominated points."""
    v = np.asarray(volumes, float)
    t = np.asarray(periods, float)
    return float(np.dot(v, v) / np.dot(v, t))


def fit_issue_floor(gaps, issue_times, frac=0.25) -> float:
    """Median issue time over the largest `frac` of the gaps (the recovered plateau)."""
    g = np.asarray(gaps, float)
    t = np.asarray(issue_times, float)
    sel = g >= np.quantile(g, 1.0 - frac)
    return float(np.median(t[sel]))


def fit_capacity(volumes, issue_times, r, n_branch=2) -> float:
    """q from the `n_branch` largest isolated bursts, taken to lie on the drain-limited branch
    t = (V - q) / r: the mean of V - r * t over them."""
    v = np.asarray(volumes, float)
    t = np.asarray(issue_times, float)
    sel = np.argsort(v)[-n_branch:]
    return float(np.mean(v[sel] - r * t[sel]))


def fit_knee(volumes, issue_times, r, q, n_small=2):
    """Knee of the isolated-burst curve: before it a burst issues at the aggregate rate s of
    the `n_small` smallest bursts (t = V / s, least squares through the origin), after it on the
    drain-limited branch (V - q) / r; the branches meet at V = q / (1 - r / s). Returns
    (s, knee volume), the knee None when s <= r (no absorption beyond the drain rate)."""
    v = np.asarray(volumes, float)
    t = np.asarray(issue_times, float)
    sel = np.argsort(v)[:n_small]
    s = float(np.dot(v[sel], v[sel]) / np.dot(v[sel], t[sel]))
    return s, (q / (1.0 - r / s) if s > r else None)


def design_test(v, r, t_iss0, q, gap) -> dict:
    """The paper's two bounds for recurring bursts of volume V separated by gap G."""
    out = {"rate_bound": bool(v / r <= t_iss0 + gap), "recovery_gap_s": v / r - t_iss0}
    out["capacity_bound"] = None if q is None else bool(v - r * t_iss0 <= q)
    return out


# ------------------------------------------------------------------ measurement (GPU)

class Bench:
    """Owns the device buffers and runs one (K, B, P, G) configuration per call."""

    def __init__(self, buf_bytes=2 << 30):
        import torch

        from . import _lib

        self.torch = torch
        self.lib = _lib
        self.buf = torch.empty(buf_bytes, dtype=torch.uint8, device="cuda")
        self.hz = _lib.moe_burst_clock_hz()
        self.cus = torch.cuda.get_device_properties(0).multi_processor_count

    def run(self, producers: int, nbytes: int, periods: int, gap_s: float):
        """Per-producer, per-period (issue time, period) in seconds; the last period has none."""
        torch = self.torch
        times = torch.empty(producers * periods * 2, dtype=torch.int64, device="cuda")
        gap_ticks = int(round(gap_s * self.hz))
        self.lib.moe_burst_gap(producers, nbytes, periods, gap_ticks, self.buf, times)
        torch.cuda.synchronize()
        t = times.cpu().numpy().reshape(producers, periods, 2).astype(np.float64) / self.hz
        issue = t[:, :, 1] - t[:, :, 0]
        period = np.diff(t[:, :, 0], axis=1)
        return issue, period

    def periodic(self, producers, nbytes, gap_s, periods=40, skip=8):
        """Steady-state mean issue time and period (first `skip` periods dropped)."""
        issue, period = self.run(producers, nbytes, periods, gap_s)
        return float(issue[:, skip:].mean()), float(period[:, skip:].mean())

    def isolated(self, producers, nbytes, repeats=5):
        """Issue time of one burst into a quiet path (median over launches of the mean over
        producers)."""
        vals = []
        for _ in range(repeats):
            issue, _ = self.run(producers, nbytes, 1, 0.0)
            vals.append(float(issue[:, 0].mean()))
        return float(np.median(vals))


def calibrate(producers: int | None = None, burst_bytes: int = 128 * KIB, log=print) -> dict:
    """The three sweeps of the paper's Section 3 on this GPU, and the fitted parameters."""
    b = Bench()
    k = producers or b.cus
    res = {"producers": k, "clock_hz": b.hz, "burst_bytes": burst_bytes}

    # 1. drain rate: zero-gap periodic bursts over producer counts and volumes
    pts = []
    for kk in sorted({max(1, k // 4), max(1, k // 2), k}):
        for bb in (64 * KIB, 256 * KIB, 1 * MIB, 4 * MIB):
            t_iss, per = b.periodic(kk, bb, 0.0)
            pts.append({"producers": kk, "bytes": bb, "volume": kk * bb, "issue_s": t_iss, "period_s": per})
            log(f"zero gap  K={kk:4d} B={bb // KIB:6d} KiB  V={kk * bb / MIB:8.2f} MiB  period {per * 1e6:9.3f} us")
    v = np.array([p["volume"] for p in pts], float)
    per = np.array([p["period_s"] for p in pts])
    big = v >= np.median(v)  # the drain-dominated end of the sweep
    r = fit_drain_rate(v[big], per[big])
    res["zero_gap"] = pts
    res["r_bytes_per_s"] = r
    log(f"drain rate r = {r / 1e9:.1f} GB/s")

    # 2. gap sweep at K producers x burst_bytes: issue floor and the max law
    vol = k * burst_bytes
    g_star_guess = vol / r
    gaps = np.unique(np.concatenate([[0.0], np.linspace(0.1, 3.0, 15) * g_star_guess]))
    sweep = []
    for g in gaps:
        t_iss, p_ = b.periodic(k, burst_bytes, float(g))
        sweep.append({"gap_s": float(g), "issue_s": t_iss, "period_s": p_})
    t_iss0 = fit_issue_floor([s["gap_s"] for s in sweep], [s["issue_s"] for s in sweep])
    for s in sweep:
        s["predicted_issue_s"] = float(predict_issue(vol, r, t_iss0, s["gap_s"]))
        s["predicted_period_s"] = float(predict_period(vol, r, t_iss0, s["gap_s"]))
        log(f"gap {s['gap_s'] * 1e6:8.3f} us  issue {s['issue_s'] * 1e6:8.3f} (model {s['predicted_issue_s'] * 1e6:8.3f})"
            f"  period {s['period_s'] * 1e6:8.3f} (model {s['predicted_period_s'] * 1e6:8.3f}) us")
    per_err = [abs(s["period_s"] - s["predicted_period_s"]) / s["period_s"] for s in sweep]
    res["gap_sweep"] = {"volume": vol, "points": sweep, "t_iss0_s": t_iss0,
                        "recovery_gap_s": vol / r - t_iss0, "max_period_rel_err": float(max(per_err))}
    log(f"t_iss0 = {t_iss0 * 1e6:.3f} us, recovery gap {(vol / r - t_iss0) * 1e6:.3f} us, "
        f"max period error {max(per_err) * 100:.1f}%")

    # 3. isolated bursts of growing volume: the knee and the capacity
    iso = []
    for bb in (16 * KIB, 64 * KIB, 128 * KIB, 256 * KIB, 512 * KIB, 1 * MIB, 2 * MIB, 4 * MIB):
        t = b.isolated(k, bb)
        iso.append({"bytes": bb, "volume": k * bb, "issue_s": t})
        log(f"isolated  B={bb // KIB:6d} KiB  V={k * bb / MIB:8.2f} MiB  issue {t * 1e6:9.3f} us")
    iv = [p["volume"] for p in iso]
    it = [p["issue_s"] for p in iso]
    q = fit_capacity(iv, it, r)
    s_abs, v_knee = fit_knee(iv, it, r, q)
    res["isolated"] = {"points": iso, "q_bytes": q, "absorb_rate_bytes_per_s": s_abs, "knee_volume": v_knee}
    for p in iso:
        p["predicted_issue_s"] = float(max(p["volume"] / s_abs, (p["volume"] - q) / r))
    log(f"capacity q = {q / MIB:.2f} MiB, bursts absorbed at {s_abs / 1e9:.0f} GB/s up to the knee at V = "
        + ("none" if v_knee is None else f"{v_knee / MIB:.2f} MiB ({v_knee / k / KIB:.0f} KiB per producer)"))
    res["model"] = {"t_iss0_s": t_iss0, "r_bytes_per_s": r, "q_bytes": q}
    return res


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--producers", type=int, default=0, help="K (default: one per CU)")
    ap.add_argument("--burst-kib", type=int, default=128, help="B of the gap sweep (KiB per producer)")
    ap.add_argument("--gemm-gap-us", type=float, default=0.0,
                    help="also apply the design test to K x B bursts separated by this gap")
    ap.add_argument("--json", default=None, help="write the full results here")
    args = ap.parse_args(argv)
    res = calibrate(args.producers or None, args.burst_kib * KIB, log=lambda m: print(m, flush=True))
    if args.gemm_gap_us > 0:
        m = res["model"]
        res["design_test"] = design_test(res["producers"] * args.burst_kib * KIB, m["r_bytes_per_s"], m["t_iss0_s"],
                                         m["q_bytes"], args.gemm_gap_us * 1e-6)
        print("design test:", res["design_test"], flush=True)
    if args.json:
        with open(args.json, "w") as f:
            json.dump(res, f, indent=1)
    return 0


if __name__ == "__main__":
    sys.exit(main())
