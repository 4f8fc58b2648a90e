"""Condense rocprofv3 output of bench.py runs into the short text summaries kept under profiles/.

  python pmc_summary.py stats   --dir D --kernel K --workload W --command "..."
      kernel-trace --stats run (D/*kernel_stats.csv) -> profiles/K_W_kernel_stats.txt
  python pmc_summary.py traffic --fetch D1 --write D2 --copy-fetch D3 --copy-write D4 --copy-bytes N
                                --kernel K --workload W --command-fetch "..." ... [--alg-bytes B]
      two --pmc runs of the workload (FETCH_SIZE, WRITE_SIZE) and the same two counters over a
      plain device copy of N bytes -> profiles/K_W_pmc.txt with the HBM bytes per launch, each
      counter scaled by what it reads for the copy (bytes counted / bytes copied)

bench.py reads `hbm_bytes_per_launch` back only while `source_hash` matches the kernel's source.
"""
import argparse
import csv
import glob
import os
import re
import statistics
import sys

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)
import bench  # noqa: E402  (KERNEL_SOURCES, source_hash)

# demangled kernel names of the bench stages
KERNEL_PATTERNS = {
    "moe_decode_fused": r"moe_decode_fused_kernel",
    "gemv_gate_up": r"gemv_gate_up_kernel",
    "gemm_gate_up_mfma": r"expert_gemm_kernel<0",
}
COPY_PATTERN = r"copy"


def _csv_rows(directory, suffix):
    files = sorted(glob.glob(os.path.join(directory, "**", f"*{suffix}"), recursive=True))
    if not files:
        raise SystemExit(f"no *{suffix} under {directory}")
    rows = []
    for fn in files:
        with open(fn, newline="") as f:
            rows.extend(csv.DictReader(f))
    return rows


def counter_per_dispatch(directory, counter, pattern):
    """Mean over the matching dispatches of the counter's value (summed over its instances)."""
    per = {}
    for r in _csv_rows(directory, "counter_collection.csv"):
        if r.get("Counter_Name") != counter or not re.search(pattern, r.get("Kernel_Name", "")):
            continue
        key = r.get("Dispatch_Id") or r.get("Correlation_Id")
        per[key] = per.get(key, 0.0) + float(r["Counter_Value"])
    if not per:
        raise SystemExit(f"{counter}: no dispatch of /{pattern}/ in {directory}")
    return statistics.mean(per.values()), len(per)


def cmd_stats(a):
    rows = _csv_rows(a.dir, "kernel_stats.csv")
    pat = KERNEL_PATTERNS[a.kernel]
    rows.sort(key=lambda r: -float(r["TotalDurationNs"]))
    mine = [r for r in rows if re.search(pat, r["Name"])]
    if not mine:
        raise SystemExit(f"no /{pat}/ kernel in {a.dir}")
    m = mine[0]
    out = os.path.join(a.out, f"{a.kernel}_{a.workload}_kernel_stats.txt")
    with open(out, "w") as f:
        f.write(f"# rocprofv3 kernel-trace summary of {a.kernel} on the {a.workload} workload\n")
        f.write(f"command: {a.command}\n")
        f.write(f"kernel: {m['Name']}\n")
        f.write(f"calls: {m['Calls']}\n")
        f.write(f"average_us: {float(m['AverageNs']) / 1e3:.2f}\n")
        f.write(f"min_us: {float(m['MinNs']) / 1e3:.2f}\n")
        f.write(f"max_us: {float(m['MaxNs']) / 1e3:.2f}\n")
        f.write(f"source_hash: {bench.source_hash(bench.KERNEL_SOURCES[a.kernel])}\n\n")
        f.write("| kernel | calls | avg us | min us | max us | % of GPU time |\n|---|---|---|---|---|---|\n")
        for r in rows[:12]:
            name = r["Name"] if len(r["Name"]) <= 90 else r["Name"][:87] + "..."
            f.write(f"| {name} | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | {float(r['MinNs']) / 1e3:.2f} | "
                    f"{float(r['MaxNs']) / 1e3:.2f} | {float(r['Percentage']):.1f} |\n")
    print(out)


def cmd_traffic(a):
    pat = KERNEL_PATTERNS[a.kernel]
    fetch, nf = counter_per_dispatch(a.fetch, "FETCH_SIZE", pat)
    write, nw = counter_per_dispatch(a.write, "WRITE_SIZE", pat)
    cfetch, _ = counter_per_dispatch(a.copy_fetch, "FETCH_SIZE", COPY_PATTERN)
    cwrite, _ = counter_per_dispatch(a.copy_write, "WRITE_SIZE", COPY_PATTERN)
    # the counters are in KiB; each scale is counted bytes / bytes the copy really moved
    sf = cfetch * 1024.0 / a.copy_bytes
    sw = cwrite * 1024.0 / a.copy_bytes
    hbm = fetch * 1024.0 / sf + write * 1024.0 / sw
    out = os.path.join(a.out, f"{a.kernel}_{a.workload}_pmc.txt")
    with open(out, "w") as f:
        f.write(f"# rocprofv3 HBM counters of {a.kernel} on the {a.workload} workload\n")
        f.write(f"command_fetch: {a.command_fetch}\n")
        f.write(f"command_write: {a.command_write}\n")
        f.write(f"command_copy_fetch: {a.command_copy_fetch}\n")
        f.write(f"command_copy_write: {a.command_copy_write}\n")
        f.write(f"fetch_kib_per_dispatch: {fetch:.1f}\n")
        f.write(f"fetch_dispatches: {nf}\n")
        f.write(f"write_kib_per_dispatch: {write:.1f}\n")
        f.write(f"write_dispatches: {nw}\n")
        f.write(f"copy_bytes: {a.copy_bytes}\n")
        f.write(f"copy_fetch_kib: {cfetch:.1f}\n")
        f.write(f"copy_write_kib: {cwrite:.1f}\n")
        f.write(f"fetch_scale: {sf:.4f}\n")
        f.write(f"write_scale: {sw:.4f}\n")
        f.write(f"hbm_bytes_per_launch: {hbm:.0f}\n")
        if a.alg_bytes:
            f.write(f"alg_bytes_per_launch: {a.alg_bytes}\n")
            f.write(f"traffic_over_alg: {hbm / a.alg_bytes:.4f}\n")
        f.write(f"source_hash: {bench.source_hash(bench.KERNEL_SOURCES[a.kernel])}\n")
    print(out)


def main():
    p = argparse.ArgumentParser()
    sub = p.add_subparsers(dest="cmd", required=True)
    s = sub.add_parser("stats")
    s.add_argument("--dir", required=True)
    s.add_argument("--kernel", required=True, choices=sorted(KERNEL_PATTERNS))
    s.add_argument("--workload", required=True)
    s.add_argument("--command", required=True)
    t = sub.add_parser("traffic")
    for name in ("fetch", "write", "copy-fetch", "copy-write"):
        t.add_argument(f"--{name}", required=True)
        t.add_argument(f"--command-{name}", required=True)
    t.add_argument("--copy-bytes", type=int, required=True)
    t.add_argument("--kernel", required=True, choices=sorted(KERNEL_PATTERNS))
    t.add_argument("--workload", required=True)
    t.add_argument("--alg-bytes", type=int, default=0)
    for q in (s, t):
        q.add_argument("--out", default=os.path.join(ROOT, "profiles"), help="directory of the summary")
    a = p.parse_args()
    os.makedirs(a.out, exist_ok=True)
    (cmd_stats if a.cmd == "stats" else cmd_traffic)(a)


if __name__ == "__main__":
    main()
