"""Per-tile phases of the persistent GEMM from its trace (moe_config.trace, include/moe.h).

The X-Stage paper (Section 5) instruments its persistent kernel per tile to see where the time
goes; this reads the records the traced kernel writes and splits every workgroup's share of
the kernel's span into phases:

  claim     t_claimed - t_claim      one atomic on the group cursor and the record load
  wait      t_start - t_claimed      a Linear-2 tile's dependency wait (Linear-1: setup only)
  mainloop  t_epilogue - t_start     operand loads and MFMAs over K
  epilogue  t_end - t_epilogue       SwiGLU / rounding, LDS staging, the stores
  between   next t_claim - t_end     the completion release (Linear-1) and the barrier
  idle      before the workgroup's first claim and after its last tile, within the span

The span runs from the first claim to the last t_end of any workgroup. Times are readings of
the real-time counter; the clock rate is passed in (moe_burst_clock_hz).
"""
from __future__ import annotations

import numpy as np

PHASES = ("claim", "wait", "mainloop", "epilogue", "between", "idle")


def tile_phases(trace: np.ndarray, clock_hz: float) -> dict:
    """Phase fractions of the summed workgroup time, plus mean per-tile microseconds."""
    r = trace[trace["task"] != -1]
    if len(r) == 0:
        raise ValueError("the trace holds no tile")
    us = 1e6 / float(clock_hz)
    l2 = ((r["task"].astype(np.int64) & 0xFFFFFFFF) >> 31) == 1
    t0, t1 = int(r["t_claim"].min()), int(r["t_end"].max())
    span = t1 - t0
    tot = {p: 0 for p in PHASES}
    tot["claim"] = int((r["t_claimed"] - r["t_claim"]).sum())
    tot["wait"] = int((r["t_start"] - r["t_claimed"]).sum())
    tot["mainloop"] = int((r["t_epilogue"] - r["t_start"]).sum())
    tot["epilogue"] = int((r["t_end"] - r["t_epilogue"]).sum())
    wgs = np.unique(r["workgroup"])
    for wg in wgs:
        w = r[r["workgroup"] == wg]
        w = w[np.argsort(w["t_claim"], kind="stable")]
        tot["between"] += int((w["t_claim"][1:] - w["t_end"][:-1]).sum())
        tot["idle"] += int(w["t_claim"][0] - t0) + int(t1 - w["t_end"][-1])
    whole = span * len(wgs)
    out = {"span_us": span * us, "workgroups": int(len(wgs)), "tiles": int(len(r)),
           "linear1_tiles": int((~l2).sum()), "linear2_tiles": int(l2.sum()),
           "fractions": {p: tot[p] / whole for p in PHASES}}
    for name, sel in (("linear1", ~l2), ("linear2", l2)):
        if sel.any():
            x = r[sel]
            out[name + "_us"] = {"claim": float((x["t_claimed"] - x["t_claim"]).mean() * us),
                                 "wait": float((x["t_start"] - x["t_claimed"]).mean() * us),
                                 "mainloop": float((x["t_epilogue"] - x["t_start"]).mean() * us),
                                 "epilogue": float((x["t_end"] - x["t_epilogue"]).mean() * us)}
    return out


def format_phases(title: str, ph: dict) -> str:
    lines = [f"{title}: span {ph['span_us']:.1f} us, {ph['workgroups']} workgroups, "
             f"{ph['tiles']} tiles ({ph['linear1_tiles']} Linear-1, {ph['linear2_tiles']} Linear-2)",
             "  share of workgroup time: " + ", ".join(f"{p} {100 * f:.1f}%" for p, f in ph["fractions"].items())]
    for name in ("linear1", "linear2"):
        if name + "_us" in ph:
            lines.append(f"  {name} tile mean us: " + ", ".join(f"{k} {v:.2f}" for k, v in ph[name + "_us"].items()))
    return "\n".join(lines)
