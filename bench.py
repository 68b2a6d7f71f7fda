"""Benchmark: one GPU's share of the expert-parallel MoE FFN layer on MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload dsv3_share]

A step is one pass of the whole layer over one batch already resident in HBM: moe_plan
(route, histogram, scan, scatter, tile list) -> moe_forward_gather (persistent grouped GEMM with
the dispatch gather folded into the Linear-1 loads: Linear-1 + SwiGLU, Linear-2; or, with
--dispatch separate, moe_dispatch then moe_forward) -> moe_combine. W untimed steps, then
exactly K timed steps bracketed by device synchronisation, with events only around the forward
call; the per-call breakdown comes from a separate shorter pass with events between all calls.
Prints ONE JSON line on stdout.

value = layer TFLOP/s = 6*T*k*H*I per step / seconds per step (the two expert GEMMs).
roofline = the persistent GEMM kernel (the dominant launch): its flops per launch divided by
its average duration, measured with events on the stream it runs on, against the dense bf16
MFMA peak of MI355X (2.5 PFLOP/s).
cpu_baseline = the CPU oracle (float64 NumPy) on a bounded sample of the same workload: the
first experts' rows (whole experts, in expert order) until about 10 s of work, scaled to
TFLOP/s by the sample's flops.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

MFMA_PEAK_TFLOPS = 2500.0  # MI355X dense bf16
HBM_PEAK_GBPS = 8000.0
HDR_LEAD = 26  # workspace header slot holding the interleave lead the plan used


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def algorithmic_bytes(s, counts) -> int:
    """Bytes the staged layer must move once each: X and logits in, weights of experts with
    rows, Xd / A / Yd written and read once, the output, and the routing metadata."""
    R = s.T * s.k
    active = int((counts > 0).sum())
    return (s.T * s.H * 2 + s.T * s.E * 4 + active * 3 * s.H * s.I * 2 + 2 * R * s.H * 2 + 2 * R * s.I * 2
            + 2 * R * s.H * 2 + s.T * s.H * 2 + R * 16)


def gemm_bytes(s, counts) -> int:
    """Algorithmic HBM bytes of one moe_forward launch: Xd read, active experts' W1 and W2
    read, A written and read back, Yd written."""
    R = s.T * s.k
    active = int((counts > 0).sum())
    return R * s.H * 2 + active * 3 * s.H * s.I * 2 + 2 * R * s.I * 2 + R * s.H * 2


def kernel_source_sha() -> str:
    """Hash of the code (comments and blank lines left out) of the GEMM and of the planner that
    writes the tile order it walks: the profiled traffic belongs to exactly this code."""
    h = hashlib.sha256()
    for f in ("moe_gemm.hip", "moe_internal.h", "moe_plan.hip"):
        with open(os.path.join(ROOT, "mixture_experts_ffn_dispatch_amd", "csrc", f), encoding="utf-8") as fh:
            for line in fh:
                code = line.split("//", 1)[0].rstrip()
                if code:
                    h.update(code.encode() + b"\n")
    return h.hexdigest()[:16]


def traffic_from_profiles(workload: str):
    """HBM bytes per launch of the persistent GEMM from committed rocprofv3 counter runs, or
    None when they are missing or were taken on a different kernel source."""
    p = os.path.join(ROOT, "profiles", f"gemm_persistent_{workload}_traffic.json")
    if not os.path.exists(p):
        return None
    with open(p) as f:
        t = json.load(f)
    if t.get("kernel_sha") != kernel_source_sha():
        return None
    return t.get("hbm_bytes_per_launch")


def cpu_baseline(s, data, budget_s: float = 10.0) -> dict:
    """Time the CPU oracle on whole experts (in expert order) until the budget is spent."""
    import numpy as np

    from oracle import moe_ref as R

    try:
        from threadpoolctl import threadpool_info

        cores = max([i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"] or [1])
    except Exception:  # pragma: no cover
        cores = os.cpu_count() or 1
    t0 = time.perf_counter()
    ids, w = R.route(data["logits"], s.k)
    counts, offsets, perm, pos = R.plan(ids, s.E)
    t_route = time.perf_counter() - t0
    rows = 0
    experts = 0
    t_ffn = 0.0
    for e in range(s.E):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if hi == lo:
            continue
        xd = R.dispatch(data["x"], perm[lo:hi], s.k)
        t1 = time.perf_counter()
        R.expert_ffn(xd, data["w1"][e], data["w2"][e])
        t_ffn += time.perf_counter() - t1
        rows += hi - lo
        experts += 1
        if t_ffn >= budget_s:
            break
    flops = 6.0 * rows * s.H * s.I
    # routing of the whole batch is charged in proportion to the rows sampled
    t_total = t_ffn + t_route * rows / (s.T * s.k)
    return {"value": round(flops / t_total / 1e12, 6), "unit": "TFLOP/s", "cores": int(cores), "kind": "oracle",
            "sample": f"{experts} of {s.E} experts ({rows} of {s.T * s.k} dispatched rows), float64 NumPy; "
                      f"routing of all {s.T} tokens charged pro rata; {t_total:.1f} s"}


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="dsv3_share")
    ap.add_argument("--schedule", choices=["interleaved", "expert_wave"], default="interleaved")
    ap.add_argument("--lead", type=int, default=0, help="interleave lead D (0 = chosen by the plan)")
    ap.add_argument("--tile-m", type=int, default=0)
    ap.add_argument("--dispatch", choices=["fused", "separate"], default="fused",
                    help="fused: Linear-1 gathers token rows itself (moe_forward_gather); separate: "
                         "moe_dispatch writes xd first")
    ap.add_argument("--num-workgroups", type=int, default=0)
    ap.add_argument("--wide-tails", choices=["auto", "on", "off"], default="auto",
                    help="wide last m-blocks: the library's choice, forced on, or off (comparison)")
    ap.add_argument("--no-compare", action="store_true", help="skip timing the other schedule")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=10.0)
    ap.add_argument("--lib", default=None, help="load another build of libmoe (same ABI) instead of the in-tree one")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 1 GiB device copy (reference for HBM byte counters)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        log("bench.py measures one GPU's share of the layer and runs on exactly one GPU; the "
            "expert-parallel exchange across GPUs is not implemented. Use --gpus 1.")
        return 2

    import numpy as np
    import torch

    import mixture_experts_ffn_dispatch_amd as moe
    import moe_workloads as W

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    moe.load(args.lib)
    s = W.shape(args.workload)
    log(f"workload {W.describe(s)}")
    t0 = time.perf_counter()
    data = W.generate(s)
    log(f"generated inputs in {time.perf_counter() - t0:.1f} s")

    def dev(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()

    x, w1, w2 = dev(data["x"]), dev(data["w1"]), dev(data["w2"])
    logits = torch.from_numpy(data["logits"]).cuda()
    sched = {"interleaved": moe.MOE_SCHED_INTERLEAVED, "expert_wave": moe.MOE_SCHED_EXPERT_WAVE}

    def make_cfg(name):
        return moe.MoeConfig(T=s.T, H=s.H, I=s.I, E=s.E, k=s.k, experts_per_wave=s.experts_per_wave,
                             schedule=sched[name], lead_waves=args.lead, tile_m=args.tile_m,
                             num_workgroups=args.num_workgroups,
                             flags={"auto": 0, "on": moe.MOE_FLAG_WIDE_TAILS,
                                    "off": moe.MOE_FLAG_NO_WIDE_TAILS}[args.wide_tails])

    stream = torch.cuda.current_stream()

    def timed(name, steps, warmup):
        cfg = make_cfg(name)
        fused = args.dispatch == "fused"
        b = moe.alloc_buffers(cfg, xd=not fused)

        def step(fwd_ev=None, call_ev=None):
            # fwd_ev: two events around the forward call; call_ev: five events between the calls
            def mark(i):
                if call_ev is not None:
                    call_ev[i].record(stream)

            mark(0)
            moe.moe_plan(cfg, logits, b, b["ws"])
            mark(1)
            if not fused:
                moe.moe_dispatch(cfg, b, x, b["xd"])
            mark(2)
            if fwd_ev is not None:
                fwd_ev[0].record(stream)
            if fused:
                moe.moe_forward_gather(cfg, b, x, w1, w2, b["act"], b["yd"], b["ws"])
            else:
                moe.moe_forward(cfg, b["xd"], w1, w2, b["act"], b["yd"], b["ws"])
            if fwd_ev is not None:
                fwd_ev[1].record(stream)
            mark(3)
            moe.moe_combine(cfg, b, b["yd"], b["out"])
            mark(4)

        for _ in range(warmup):
            step()
        st = moe.moe_status_read(b["ws"])
        assert st == moe.MOE_OK, moe.strerror(st)
        # Timed region: K whole layers back to back. Only the forward call is bracketed by
        # events (its mean duration is the roofline's `achieved`); events between every call
        # would add their own gaps to the step.
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(steps)]
        torch.cuda.synchronize()
        t_start = time.perf_counter()
        for i in range(steps):
            step(fwd_ev=ev[i])
        torch.cuda.synchronize()
        wall = time.perf_counter() - t_start
        st = moe.moe_status_read(b["ws"])
        assert st == moe.MOE_OK, moe.strerror(st)
        fwd = np.array([e[0].elapsed_time(e[1]) for e in ev])  # ms
        # per-call breakdown from a separate, shorter pass with events between the calls
        nb = min(steps, 10)
        evb = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(nb)]
        for i in range(nb):
            step(call_ev=evb[i])
        torch.cuda.synchronize()
        per = np.array([[e[j].elapsed_time(e[j + 1]) for j in range(4)] for e in evb])  # ms
        step_ms = np.array([e[0].elapsed_time(e[4]) for e in evb])
        counts = b["counts"].cpu().numpy()
        layout = moe.moe_workspace_layout(cfg)
        lead_used = int(b["ws"][:128].cpu().numpy().view(np.int32)[HDR_LEAD])
        return dict(wall_ms=wall * 1e3 / steps, fwd_ms=fwd, step_ms=step_ms, per=per, counts=counts,
                    layout=layout, lead_used=lead_used)

    main_res = timed(args.schedule, args.steps, args.warmup)
    other = None
    if not args.no_compare:
        oname = "expert_wave" if args.schedule == "interleaved" else "interleaved"
        other = (oname, timed(oname, args.steps, args.warmup))

    if args.copy_calibration:
        src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()

    flops = 6.0 * s.T * s.k * s.H * s.I
    ms = float(main_res["wall_ms"])
    fwd_ms = float(np.mean(main_res["fwd_ms"]))
    counts = main_res["counts"]
    traffic = traffic_from_profiles(args.workload)
    achieved = flops / (fwd_ms * 1e-3) / 1e12
    # the GEMM's bound: MFMA when its algorithmic intensity is above the MFMA/HBM ridge
    # (2.5 PFLOP/s / 8 TB/s = 312.5 flop/B), HBM below it (small M: weights dominate)
    gbytes = gemm_bytes(s, counts)
    if flops / gbytes >= MFMA_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBPS * 1e9):
        roof = {"bound": "mfma", "kernel": "gemm_persistent_kernel", "achieved": round(achieved, 3),
                "peak": MFMA_PEAK_TFLOPS, "unit": "TFLOP/s", "frac": round(achieved / MFMA_PEAK_TFLOPS, 4),
                "traffic": traffic}
    else:
        gbps = gbytes / (fwd_ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "kernel": "gemm_persistent_kernel", "achieved": round(gbps, 1),
                "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": round(gbps / HBM_PEAK_GBPS, 4), "traffic": traffic,
                "tflops": round(achieved, 3)}
    rec = {
        "metric": "MoE layer TFLOP/s (bf16) and % of MFMA peak; us/layer; HBM GB/s at small M",
        "value": round(flops / (ms * 1e-3) / 1e12, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": s.name, "T": s.T, "H": s.H, "I": s.I, "E": s.E, "k": s.k,
                   "experts_per_wave": s.experts_per_wave, "schedule": args.schedule, "dispatch": args.dispatch, "lead_waves": args.lead,
                   "wide_tails": args.wide_tails,
                   "lead_used": main_res["lead_used"],
                   "tile_m": main_res["layout"]["tile_m"], "seed": s.seed},
        "roofline": roof,
        "us_per_layer": round(ms * 1e3, 2),
        "mfma_frac_layer": round(flops / (ms * 1e-3) / 1e12 / MFMA_PEAK_TFLOPS, 4),
        "hbm_gbps_algorithmic": round(algorithmic_bytes(s, counts) / (ms * 1e-3) / 1e9, 1),
        "gemm_hbm_gbps_algorithmic": round(gemm_bytes(s, counts) / (fwd_ms * 1e-3) / 1e9, 1),
        "per_call_us": {k: round(float(np.mean(main_res["per"][:, j])) * 1e3, 2)
                        for j, k in enumerate(("plan", "dispatch", "forward", "combine"))},
        "step_us_median": round(float(np.median(main_res["step_ms"])) * 1e3, 2),
        "active_experts": int((counts > 0).sum()),
    }
    if other is not None:
        oname, o = other
        rec["other_schedule"] = {"schedule": oname, "value": round(flops / (o["wall_ms"] * 1e-3) / 1e12, 3),
                                 "us_per_layer": round(float(o["wall_ms"]) * 1e3, 2),
                                 "forward_us": round(float(np.mean(o["fwd_ms"])) * 1e3, 2)}
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on a bounded sample ...")
        rec["cpu_baseline"] = cpu_baseline(s, data, args.cpu_budget)
    print(json.dumps(rec), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
