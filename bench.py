"""Benchmark: one GPU's share of the expert-parallel MoE FFN layer on MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload dit_batch]

A step is one pass of the whole layer over one batch already resident in HBM: moe_plan
(route, histogram, scan, scatter, tile list) -> moe_forward_gather (persistent grouped GEMM with
the dispatch gather folded into the Linear-1 loads: Linear-1 + SwiGLU, Linear-2; or, with
--dispatch separate, moe_dispatch then moe_forward) -> moe_combine. The headline workload is
the largest one (dit_batch: T = 65536, H = 4096, I = 8192, E = 16, k = 2). W untimed steps,
then exactly K timed steps bracketed by device synchronisation; events on the launch stream
mark each step and its forward call. Prints ONE JSON line on stdout.

value = layer TFLOP/s = 6*T*k*H*I per step / wall-clock seconds per step (the two expert GEMMs).
roofline = the persistent GEMM kernel (the dominant launch): its flops per launch divided by
its average duration, measured with events on the stream it runs on, against the dense bf16
MFMA peak of MI355X (2.5 PFLOP/s); for an HBM-bound workload its algorithmic bytes against
8 TB/s.
schedules = both tile orders timed in alternating trials, the order of the pair rotated from
one trial to the next (X-Stage paper, Section 5, setup: warm up, repeat, report the median,
rotate the scheduler order): median, min and max microseconds per layer.
workloads = the same alternating trials for the other named workloads, with the GEMM's
event-timed duration, its fraction of the MFMA peak, and its algorithmic HBM rate.
cpu_baseline = the CPU oracle (float64 NumPy) on a bounded sample of the headline workload:
the first experts' rows (whole experts, in expert order) until about 10 s of work, scaled to
TFLOP/s by the sample's flops; with the host's CPU model and core counts.
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
HDR_SCHED = 28  # ... and the order it wrote (0 Expert-Wave, 1 interleaved)


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
    for f in ("moe_gemm.hip", "moe_internal.h", "moe_plan.hip", "moe_plan_dev.h"):
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


def attention_block(name, steps, warmup, moe, W, log) -> dict:
    """The attention forward of the X-Stage paper's Section 4.3 on one workload: event-timed
    launches, TFLOP/s against the bf16 MFMA peak, and the paper's design test for its output
    bursts (each persistent workgroup stores one b_m x d bf16 tile at a tile boundary, the next
    tile's Q-loop is the gap) against this GPU's own memory path."""
    import numpy as np
    import torch

    s = W.attn_shape(name)
    log(f"attention {s.name}: B={s.B} heads={s.heads} M={s.M} d={s.d}")
    g = W.generate_attention(s)

    def dev(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()

    q, k, v = dev(g["q"]), dev(g["k"]), dev(g["v"])
    o = torch.empty_like(q)
    lse = torch.empty((s.B, s.heads, s.M), dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()
    for _ in range(warmup):
        moe.attn_forward(s.B, s.heads, s.M, q, k, v, o, lse)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(steps)]
    torch.cuda.synchronize()
    for e in ev:
        e[0].record(stream)
        moe.attn_forward(s.B, s.heads, s.M, q, k, v, o, lse)
        e[1].record(stream)
    torch.cuda.synchronize()
    ms = np.array([e[0].elapsed_time(e[1]) for e in ev])
    t = float(np.median(ms)) * 1e-3
    tflops = s.flops / t / 1e12
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    bm = moe._lib.ATTN_TILE_QUERIES
    tiles = s.B * s.heads * -(-s.M // bm)
    grid = min(cus * moe._lib.ATTN_WORKGROUPS_PER_CU, tiles)
    rounds = -(-tiles // grid)
    qloop = t / rounds  # one tile's Q-loop: the gap between a workgroup's output bursts
    burst = bm * s.d * 2  # bytes per workgroup per tile boundary
    v_agg = grid * burst   # aligned producers, the conservative case
    r, t0, cap = 6646e9, 0.927e-6, 31.2 * 2 ** 20  # this GPU's own memory (moe_burst_gap)
    return {"workload": s.name, "B": s.B, "heads": s.heads, "M": s.M, "d": s.d, "kernel": "attn_fwd_kernel",
            "us": stats_us(ms), "tflops": round(tflops, 2), "mfma_frac": round(tflops / MFMA_PEAK_TFLOPS, 4),
            "tiles": tiles, "grid": grid, "qloop_us": round(qloop * 1e6, 2),
            "burst_bytes_per_tile": burst, "aligned_burst_bytes": v_agg,
            "design_test_local": {"rate_bound": v_agg / r <= t0 + qloop, "capacity_bound": v_agg - r * t0 <= cap,
                                  "recovery_gap_us": round((v_agg / r - t0) * 1e6, 3)}}


def host_cpu() -> dict:
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:  # pragma: no cover
        pass
    try:
        usable = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        usable = os.cpu_count() or 1
    return {"cpu_model": model, "nproc": usable, "logical_cpus": os.cpu_count()}


def stats_us(ms) -> dict:
    import numpy as np

    a = np.asarray(ms, dtype=float) * 1e3
    return {"median": round(float(np.median(a)), 2), "min": round(float(a.min()), 2),
            "max": round(float(a.max()), 2), "n": int(a.size)}


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="dit_batch")
    ap.add_argument("--schedule", choices=["auto", "interleaved", "expert_wave"], default="auto",
                    help="tile order of the headline: auto (moe_plan picks order and lead), interleaved "
                         "(lead --lead, 0 = D_knee), expert_wave")
    ap.add_argument("--lead", type=int, default=0, help="interleave lead D (0 = chosen by the plan)")
    ap.add_argument("--tile-m", type=int, default=0)
    ap.add_argument("--dispatch", choices=["fused", "separate"], default="fused",
                    help="fused: Linear-1 gathers token rows itself (moe_forward_gather); separate: "
                         "moe_dispatch writes xd first")
    ap.add_argument("--launch", choices=["single", "calls"], default="calls",
                    help="single: the whole layer in one kernel launch (moe_layer); calls: moe_plan, "
                         "moe_forward_gather, moe_combine")
    ap.add_argument("--plan-launches", type=int, choices=[1, 3], default=3,
                    help="moe_plan as three launches (the default) or one launch with a grid barrier")
    ap.add_argument("--num-workgroups", type=int, default=0)
    ap.add_argument("--wide-tails", choices=["auto", "on", "off"], default="auto",
                    help="wide last m-blocks: the library's choice, forced on, or off (comparison)")
    ap.add_argument("--trials", type=int, default=20,
                    help="alternating trials per schedule (0 or --no-compare: the headline schedule only)")
    ap.add_argument("--no-compare", action="store_true", help="skip timing the other schedule")
    ap.add_argument("--others", default="tiny,dsv3_share,qwen3_30b_a3b,small_m_zipf",
                    help="comma-separated workloads measured after the headline ('none': skip)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=10.0)
    ap.add_argument("--lib", default=None, help="load another build of libmoe (same ABI) instead of the in-tree one")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 1 GiB device copy (reference for HBM byte counters)")
    ap.add_argument("--attention", default="attn_dit_share",
                    help="also time the attention forward on this workload ('none': skip)")
    ap.add_argument("--trace-summary", default=None,
                    help="also run one traced layer per schedule of the headline workload and write "
                         "its per-tile phases to this file")
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
    stream = torch.cuda.current_stream()
    sched = {"auto": moe.MOE_SCHED_AUTO, "interleaved": moe.MOE_SCHED_INTERLEAVED,
             "expert_wave": moe.MOE_SCHED_EXPERT_WAVE}
    fused = args.dispatch == "fused"

    def dev(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()

    class Layer:
        """One workload's inputs on the GPU, with the buffers of one schedule (and launch)."""

        def __init__(self, s, inputs, name, single=False):
            self.s, self.single = s, single
            self.name = name + ("_single" if single else "")
            self.x, self.logits, self.w1, self.w2 = inputs
            self.cfg = moe.MoeConfig(T=s.T, H=s.H, I=s.I, E=s.E, k=s.k, experts_per_wave=s.experts_per_wave,
                                     schedule=sched[name], lead_waves=0 if name == "auto" else args.lead,
                                     tile_m=args.tile_m,
                                     num_workgroups=args.num_workgroups,
                                     flags={"auto": 0, "on": moe.MOE_FLAG_WIDE_TAILS,
                                            "off": moe.MOE_FLAG_NO_WIDE_TAILS}[args.wide_tails]
                                     | (moe.MOE_FLAG_PLAN_ONE_LAUNCH if args.plan_launches == 1 else 0))
            self.b = moe.alloc_buffers(self.cfg, xd=not fused)

        def step(self, ev=None):
            """One layer. ev: four events (step start, forward start, forward end, step end), or
            None; with five events, one between every two calls (breakdown)."""
            c, b = self.cfg, self.b
            five = ev is not None and len(ev) == 5

            def mark(i):
                if ev is not None:
                    ev[i].record(stream)

            if self.single:  # one launch: the forward events bracket the whole layer
                mark(0)
                if five:
                    mark(1)
                mark(2 if five else 1)
                moe.moe_layer(c, self.logits, b, self.x, self.w1, self.w2, b["act"], b["yd"], b["out"], b["ws"])
                mark(3 if five else 2)
                mark(4 if five else 3)
                return

            mark(0)
            moe.moe_plan(c, self.logits, b, b["ws"])
            if five:
                mark(1)
            if not fused:
                moe.moe_dispatch(c, b, self.x, b["xd"])
            mark(2 if five else 1)
            if fused:
                moe.moe_forward_gather(c, b, self.x, self.w1, self.w2, b["act"], b["yd"], b["ws"])
            else:
                moe.moe_forward(c, b["xd"], self.w1, self.w2, b["act"], b["yd"], b["ws"])
            mark(3 if five else 2)
            moe.moe_combine(c, b, b["yd"], b["out"])
            mark(4 if five else 3)

        def check(self):
            st = moe.moe_status_read(self.b["ws"])
            assert st == moe.MOE_OK, moe.strerror(st)

        def lead_used(self):
            return int(self.b["ws"][:128].cpu().numpy().view(np.int32)[HDR_LEAD])

        def order_used(self):
            return ["expert_wave", "interleaved"][int(self.b["ws"][:128].cpu().numpy().view(np.int32)[HDR_SCHED])]

    def events(n, m):
        return [[torch.cuda.Event(enable_timing=True) for _ in range(m)] for _ in range(n)]

    def alternate(layers, trials):
        """Alternating trials: each trial runs every schedule once, the order rotated from one
        trial to the next. Returns per schedule the layer and forward times (ms)."""
        ev = {l.name: events(trials, 4) for l in layers}
        for i in range(trials):
            for j in range(len(layers)):
                l = layers[(i + j) % len(layers)]
                l.step(ev[l.name][i])
        torch.cuda.synchronize()
        for l in layers:
            l.check()
        return {l.name: (np.array([e[0].elapsed_time(e[3]) for e in ev[l.name]]),
                         np.array([e[1].elapsed_time(e[2]) for e in ev[l.name]])) for l in layers}

    def load_inputs(name):
        s = W.shape(name)
        log(f"workload {W.describe(s)}")
        t0 = time.perf_counter()
        data = W.generate(s)
        inputs = (dev(data["x"]), torch.from_numpy(data["logits"]).cuda(), dev(data["w1"]), dev(data["w2"]))
        log(f"  inputs generated and uploaded in {time.perf_counter() - t0:.1f} s")
        return s, data, inputs

    def gemm_roofline(s, counts, fwd_ms):
        flops = 6.0 * s.T * s.k * s.H * s.I
        achieved = flops / (fwd_ms * 1e-3) / 1e12
        gbytes = gemm_bytes(s, counts)
        gbps = gbytes / (fwd_ms * 1e-3) / 1e9
        # the GEMM's bound: MFMA when its algorithmic intensity is above the MFMA/HBM ridge
        # (2.5 PFLOP/s / 8 TB/s = 312.5 flop/B), HBM below it (small M: weights dominate)
        mfma = flops / gbytes >= MFMA_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBPS * 1e9)
        return mfma, achieved, gbps

    # ---- the headline workload
    s, data, inputs = load_inputs(args.workload)
    flops = 6.0 * s.T * s.k * s.H * s.I
    main_l = Layer(s, inputs, args.schedule, single=args.launch == "single")
    for _ in range(args.warmup):
        main_l.step()
    main_l.check()
    # Timed region: K whole layers back to back, four events per step on the launch stream
    # (step start, forward start and end, step end).
    ev = events(args.steps, 4)
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for i in range(args.steps):
        main_l.step(ev[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    main_l.check()
    step_ms = np.array([e[0].elapsed_time(e[3]) for e in ev])
    fwd_ms_all = np.array([e[1].elapsed_time(e[2]) for e in ev])
    # per-call breakdown from a separate, shorter pass with events between all calls
    nb = min(args.steps, 10)
    evb = events(nb, 5)
    for i in range(nb):
        main_l.step(evb[i])
    torch.cuda.synchronize()
    per = np.array([[e[j].elapsed_time(e[j + 1]) for j in range(4)] for e in evb])  # ms
    counts = main_l.b["counts"].cpu().numpy()
    layout = moe.moe_workspace_layout(main_l.cfg)
    lead_used = main_l.lead_used()
    order_used = main_l.order_used()
    schedules = None
    if not args.no_compare and args.trials > 0:
        others_l = [Layer(s, inputs, n) for n in ("auto", "interleaved", "expert_wave") if n != main_l.name]
        if args.schedule == "auto":  # the same order in the other launch form
            others_l.append(Layer(s, inputs, "auto", single=args.launch != "single"))
        for l in others_l:
            for _ in range(args.warmup):
                l.step()
        res = alternate([main_l] + others_l, args.trials)
        schedules = {n: {"us_per_layer": stats_us(r[0]), "forward_us": stats_us(r[1])} for n, r in res.items()}
        for l in [main_l] + others_l:
            schedules[l.name]["order"] = l.order_used()
            schedules[l.name]["lead"] = l.lead_used()
        del others_l

    if args.trace_summary:
        from mixture_experts_ffn_dispatch_amd import tracing

        hz = moe.moe_burst_clock_hz()
        text = [f"# command: python3 bench.py {' '.join(sys.argv[1:])}",
                "# per-tile phases of gemm_persistent_kernel from its trace (one traced layer per schedule, "
                "after the timed runs)"]
        for name in ("auto", "interleaved", "expert_wave"):
            tl = Layer(s, inputs, name)
            tl.step()
            buf = torch.full((layout["max_slots"] * 64,), 0xFF, dtype=torch.uint8, device="cuda")
            tl.cfg.trace = buf
            tl.step()
            tl.cfg.trace = None
            torch.cuda.synchronize()
            tl.check()
            ph = tracing.tile_phases(buf.cpu().numpy().view(moe._lib.TRACE_DTYPE), hz)
            text.append(tracing.format_phases(f"{s.name} {name} ({tl.order_used()}, lead {tl.lead_used()})", ph))
            del tl, buf
        with open(args.trace_summary, "w") as f:
            f.write("\n".join(text) + "\n")
        log("\n".join(text))

    if args.copy_calibration:
        src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    ms = wall * 1e3 / args.steps
    fwd_ms = float(np.mean(fwd_ms_all))
    traffic = traffic_from_profiles(args.workload)
    mfma, achieved, gbps = gemm_roofline(s, counts, fwd_ms)
    kname = "gemm_persistent_kernel" + (" (single launch: the whole layer)" if args.launch == "single" else "")
    if mfma:
        roof = {"bound": "mfma", "kernel": kname, "achieved": round(achieved, 3),
                "peak": MFMA_PEAK_TFLOPS, "unit": "TFLOP/s", "frac": round(achieved / MFMA_PEAK_TFLOPS, 4),
                "traffic": traffic}
    else:
        roof = {"bound": "hbm", "kernel": kname, "achieved": round(gbps, 1),
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
                   "experts_per_wave": s.experts_per_wave, "schedule": args.schedule, "launch": args.launch,
                   "dispatch": args.dispatch, "plan_launches": args.plan_launches,
                   "lead_waves": args.lead, "wide_tails": args.wide_tails, "order_used": order_used,
                   "lead_used": lead_used,
                   "tile_m": layout["tile_m"], "seed": s.seed},
        "roofline": roof,
        "us_per_layer": round(ms * 1e3, 2),
        "step_us": stats_us(step_ms),
        "forward_us": stats_us(fwd_ms_all),
        "mfma_frac_layer": round(flops / (ms * 1e-3) / 1e12 / MFMA_PEAK_TFLOPS, 4),
        "hbm_gbps_algorithmic": round(algorithmic_bytes(s, counts) / (ms * 1e-3) / 1e9, 1),
        "gemm_hbm_gbps_algorithmic": round(gbps, 1),
        "per_call_us": {k: round(float(np.mean(per[:, j])) * 1e3, 2)
                        for j, k in enumerate(("plan", "dispatch", "forward", "combine"))},
        "active_experts": int((counts > 0).sum()),
    }
    if schedules is not None:
        rec["schedules"] = schedules
    cpu = None
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on a bounded sample ...")
        cpu = cpu_baseline(s, data, args.cpu_budget)
        cpu.update(host_cpu())
    del main_l, inputs, data
    torch.cuda.empty_cache()

    # ---- the other workloads: alternating trials of both schedules
    others = [n for n in args.others.split(",") if n and n != "none" and n != args.workload]
    if others:
        rec["workloads"] = {}
    for name in others:
        so, _, inp = load_inputs(name)
        names = [args.schedule] if args.no_compare else \
            [args.schedule] + [n for n in ("auto", "interleaved", "expert_wave") if n != args.schedule]
        ls = [Layer(so, inp, n, single=args.launch == "single" and i == 0) for i, n in enumerate(names)]
        if not args.no_compare and args.schedule == "auto":
            ls.append(Layer(so, inp, "auto", single=args.launch != "single"))
        for l in ls:
            for _ in range(args.warmup):
                l.step()
        res = alternate(ls, max(args.trials, 1))
        c = ls[0].b["counts"].cpu().numpy()
        lay, fw = res[ls[0].name]
        fmean = float(np.mean(fw))
        mfma_o, ach, gb = gemm_roofline(so, c, fmean)
        fl = 6.0 * so.T * so.k * so.H * so.I
        w = {"bound": "mfma" if mfma_o else "hbm", "us_per_layer": stats_us(lay),
             "tflops": round(fl / (float(np.median(lay)) * 1e-3) / 1e12, 2),
             "gemm_us": round(fmean * 1e3, 2), "gemm_tflops": round(ach, 2),
             "gemm_mfma_frac": round(ach / MFMA_PEAK_TFLOPS, 4),
             "gemm_hbm_gbps": round(gb, 1), "gemm_hbm_frac": round(gb / HBM_PEAK_GBPS, 4),
             "order_used": ls[0].order_used(), "lead_used": ls[0].lead_used(),
             "tile_m": moe.moe_workspace_layout(ls[0].cfg)["tile_m"]}
        for l in ls[1:]:
            w[f"{l.name}_us_per_layer"] = stats_us(res[l.name][0])
            w[f"{l.name}_lead"] = l.lead_used()
        rec["workloads"][name] = w
        del ls, inp
        torch.cuda.empty_cache()
    if args.attention != "none":
        rec["attention"] = attention_block(args.attention, args.steps, args.warmup, moe, W, log)
    if cpu is not None:
        rec["cpu_baseline"] = cpu
    print(json.dumps(rec), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
