"""Turn rocprofv3 CSV outputs into the short text summaries kept under profiles/.

    python -m mixture_experts_ffn_dispatch_amd.prof_summary trace  <kernel_stats.csv> <out.txt> <command...>
    python -m mixture_experts_ffn_dispatch_amd.prof_summary counters <counter_collection.csv> <out.txt> <command...>
    python -m mixture_experts_ffn_dispatch_amd.prof_summary traffic <fetch.csv> <write.csv> <workload> <out.json> <kernel_sha> <command...>

Counter values are averaged per kernel over the dispatches in the file. For the traffic
summary, FETCH_SIZE and WRITE_SIZE (KiB per dispatch) of the persistent GEMM are scaled by
what the same counters read for the plain device copy in the same run: the largest rocclr
copyBuffer dispatches, each copying 1 GiB (1 GiB read + 1 GiB written).
"""
import collections
import csv
import json
import sys

KERNELS = ("gemm_persistent_kernel", "attn_fwd_kernel", "route_hist_kernel", "scan_schedule_kernel", "scatter_kernel",
           "dispatch_kernel", "combine_kernel", "copyBuffer")


def short(name):
    for k in KERNELS:
        if k in name:
            return k
    return name[:48]


def counters(path):
    agg = collections.defaultdict(list)
    copies = collections.defaultdict(list)
    for r in csv.DictReader(open(path)):
        k = short(r["Kernel_Name"])
        if k == "copyBuffer":
            copies[r["Counter_Name"]].append((int(r["Grid_Size"]), float(r["Counter_Value"])))
        else:
            agg[(k, r["Counter_Name"])].append(float(r["Counter_Value"]))
    out = {k: sum(v) / len(v) for k, v in agg.items()}
    for name, vals in copies.items():  # only the largest copies (the 1 GiB reference)
        big = max(g for g, _ in vals)
        sel = [v for g, v in vals if g == big]
        out[("copyBuffer", name)] = sum(sel) / len(sel)
    return out


def main():
    mode = sys.argv[1]
    if mode == "trace":
        src, out, cmd = sys.argv[2], sys.argv[3], " ".join(sys.argv[4:])
        rows = list(csv.DictReader(open(src)))
        with open(out, "w") as f:
            f.write(f"# command: {cmd}\n# rocprofv3 --kernel-trace --stats: per-kernel launch statistics\n")
            f.write(f"{'kernel':60s} {'calls':>6s} {'avg_us':>10s} {'min_us':>10s} {'max_us':>10s} {'pct':>6s}\n")
            for r in rows:
                f.write(f"{r['Name'][:60]:60s} {int(r['Calls']):6d} {float(r['AverageNs'])/1e3:10.2f} "
                        f"{float(r['MinNs'])/1e3:10.2f} {float(r['MaxNs'])/1e3:10.2f} {float(r['Percentage']):6.2f}\n")
    elif mode == "counters":
        src, out, cmd = sys.argv[2], sys.argv[3], " ".join(sys.argv[4:])
        c = counters(src)
        with open(out, "w") as f:
            f.write(f"# command: {cmd}\n# mean counter value per dispatch\n")
            for (k, n), v in sorted(c.items()):
                f.write(f"{k:28s} {n:28s} {v:16.6g}\n")
    elif mode == "traffic":
        fetch, write, workload, out, sha = sys.argv[2:7]
        cmd = " ".join(sys.argv[7:])  # the profiled command; run once with each counter
        cf, cw = counters(fetch), counters(write)
        copy_bytes = 1024 * 1024 * 1024
        f_scale = copy_bytes / (cf[("copyBuffer", "FETCH_SIZE")] * 1024)
        w_scale = copy_bytes / (cw[("copyBuffer", "WRITE_SIZE")] * 1024)
        fb = cf[("gemm_persistent_kernel", "FETCH_SIZE")] * 1024 * f_scale
        wb = cw[("gemm_persistent_kernel", "WRITE_SIZE")] * 1024 * w_scale
        rec = {"kernel": "gemm_persistent_kernel", "workload": workload, "kernel_sha": sha,
               "commands": [cmd.replace("<COUNTER>", c) for c in ("FETCH_SIZE", "WRITE_SIZE")],
               "fetch_size_kib": cf[("gemm_persistent_kernel", "FETCH_SIZE")],
               "write_size_kib": cw[("gemm_persistent_kernel", "WRITE_SIZE")],
               "fetch_scale": f_scale, "write_scale": w_scale,
               "hbm_read_bytes_per_launch": fb, "hbm_write_bytes_per_launch": wb,
               "hbm_bytes_per_launch": fb + wb}
        with open(out, "w") as f:
            json.dump(rec, f, indent=1)
            f.write("\n")
    else:
        raise SystemExit(f"unknown mode {mode}")


if __name__ == "__main__":
    main()
