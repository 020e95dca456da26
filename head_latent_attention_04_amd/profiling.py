"""Summaries of rocprofv3 output for the committed profiles (host-side text processing only).

  python3 -m head_latent_attention_04_amd.profiling stats <run_kernel_stats.csv> --title T --command C
      prints the per-kernel duration table (microseconds) with the command that produced it.

  python3 -m head_latent_attention_04_amd.profiling counters <run_counter_collection.csv>... --kernel NAME --command C
      prints the average per-dispatch value of every collected counter for kernels named NAME.

  python3 -m head_latent_attention_04_amd.profiling traffic --fetch <fetch run_counter_collection.csv>
      --write <write run_counter_collection.csv> --kernel NAME --workload W --copy-bytes N --command C
      prints the JSON that bench.py reads as the attention kernel's measured HBM traffic: the average
      FETCH_SIZE and WRITE_SIZE per dispatch of NAME, each scaled by the factor that turns the same
      counter's reading for a plain device copy of N bytes (read N, write N) into N bytes.

  python3 -m head_latent_attention_04_amd.profiling backtoback <run_kernel_trace.csv> --kernel NAME
      prints the average duration of the dispatches of NAME in the longest run of consecutive
      dispatches of that kernel alone (a timing loop that launches it back to back), to set beside
      a benchmark's per-launch figure for the same loop.
"""
import argparse
import csv
import hashlib
import json
import os
import re
import sys
from collections import defaultdict

_ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
_KERNEL_SRC = os.path.join(_ROOT, "head_latent_attention_04_amd", "csrc", "decode_mfma.hip")


def _short(name: str) -> str:
    n = name.replace("void ", "")
    n = re.sub(r"\((?!.*<).*", "", n) if "(" in n else n
    return n[:64]


def stats(path: str, title: str, command: str) -> str:
    rows = list(csv.DictReader(open(path)))
    out = [f"# {title}", f"# command: {command}",
           "# source: rocprofv3 kernel stats (durations in microseconds; calls include set-up and warm-up launches)",
           f"{'kernel':64s} {'calls':>6s} {'avg_us':>9s} {'min_us':>9s} {'max_us':>9s} {'pct':>6s}"]
    for r in rows:
        name = re.sub(r"\(mla::.*|\(int.*|\(unsigned.*|\(char.*", "", r["Name"]).replace("void ", "")[:64]
        out.append(f"{name:64s} {int(r['Calls']):6d} {float(r['AverageNs']) / 1e3:9.2f} "
                   f"{float(r['MinNs']) / 1e3:9.2f} {float(r['MaxNs']) / 1e3:9.2f} {float(r['Percentage']):6.2f}")
    return "\n".join(out)


def _per_dispatch(path: str, counter: str):
    """{kernel name: [value per dispatch]} for one counter (rocprofv3 counter collection CSV)."""
    vals = defaultdict(list)
    for r in csv.DictReader(open(path)):
        if r["Counter_Name"] == counter:
            vals[r["Kernel_Name"]].append(float(r["Counter_Value"]))
    return vals


def _copy_reading(vals, copy_bytes: int) -> float:
    """The counter reading (KiB) of the plain copy of copy_bytes: the largest copy-kernel dispatch."""
    cands = [v for k, vs in vals.items() if "copyBuffer" in k or "copy" in k.lower() for v in vs]
    if not cands:
        raise SystemExit("no copy kernel dispatch in the counter run")
    return max(cands)


def traffic(fetch_csv: str, write_csv: str, kernel: str, workload: str, copy_bytes: int, command: str) -> dict:
    res = {"kernel": kernel, "workload": workload, "command": command,
           "kernel_source_sha256_16": hashlib.sha256(open(_KERNEL_SRC, "rb").read()).hexdigest()[:16]}
    total = 0.0
    for counter, path in (("FETCH_SIZE", fetch_csv), ("WRITE_SIZE", write_csv)):
        vals = _per_dispatch(path, counter)
        ks = [k for k in vals if kernel in k]
        if not ks:
            raise SystemExit(f"kernel {kernel!r} not in {path}")
        kib = [v for k in ks for v in vals[k]]
        avg_kib = sum(kib) / len(kib)
        copy_kib = _copy_reading(vals, copy_bytes)
        factor = copy_bytes / (copy_kib * 1024.0)
        scaled = avg_kib * 1024.0 * factor
        res[counter] = {"avg_KiB_per_dispatch": round(avg_kib, 1), "dispatches": len(kib),
                        "copy_probe_KiB": round(copy_kib, 1), "scale_factor": round(factor, 4),
                        "bytes_per_launch": round(scaled)}
        total += scaled
    res["bytes_per_launch"] = round(total)
    return res


def counters(paths, kernel: str, command: str) -> str:
    """Average per-dispatch value of every counter in the given counter-collection CSVs for kernels
    whose name contains `kernel`."""
    out = [f"# counters of {kernel} (average per dispatch)", f"# command: {command}"]
    for path in paths:
        vals = defaultdict(list)
        for r in csv.DictReader(open(path)):
            if kernel in r["Kernel_Name"]:
                vals[r["Counter_Name"]].append(float(r["Counter_Value"]))
        for c, xs in sorted(vals.items()):
            out.append(f"{c:28s} {sum(xs) / len(xs):16.1f}   ({len(xs)} dispatches)")
    return "\n".join(out)


def backtoback(path: str, kernel: str) -> str:
    """Longest run of consecutive dispatches (in dispatch order) whose kernel name contains `kernel`,
    and the average, minimum and maximum duration of its dispatches in microseconds."""
    rows = sorted(csv.DictReader(open(path)), key=lambda r: int(r["Dispatch_Id"]))
    best, cur = [], []
    for r in rows:
        if kernel in r["Kernel_Name"]:
            cur.append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
            if len(cur) > len(best):
                best = list(cur)
        else:
            cur = []
    if not best:
        raise SystemExit(f"no dispatch of {kernel}")
    return (f"# {kernel}: longest back-to-back run {len(best)} dispatches, average {sum(best) / len(best):.2f} us "
            f"(min {min(best):.2f}, max {max(best):.2f})")


def main(argv=None):
    ap = argparse.ArgumentParser(description="rocprofv3 summaries for profiles/")
    sub = ap.add_subparsers(dest="cmd", required=True)
    a = sub.add_parser("stats")
    a.add_argument("csv")
    a.add_argument("--title", required=True)
    a.add_argument("--command", required=True)
    b = sub.add_parser("traffic")
    b.add_argument("--fetch", required=True)
    b.add_argument("--write", required=True)
    b.add_argument("--kernel", required=True)
    b.add_argument("--workload", required=True)
    b.add_argument("--copy-bytes", type=int, required=True)
    b.add_argument("--command", required=True)
    c = sub.add_parser("counters")
    c.add_argument("csv", nargs="+")
    c.add_argument("--kernel", required=True)
    c.add_argument("--command", required=True)
    d = sub.add_parser("backtoback")
    d.add_argument("csv")
    d.add_argument("--kernel", required=True)
    args = ap.parse_args(argv)
    if args.cmd == "backtoback":
        print(backtoback(args.csv, args.kernel))
    elif args.cmd == "counters":
        print(counters(args.csv, args.kernel, args.command))
    elif args.cmd == "stats":
        print(stats(args.csv, args.title, args.command))
    else:
        print(json.dumps(traffic(args.fetch, args.write, args.kernel, args.workload, args.copy_bytes, args.command),
                         indent=1))


if __name__ == "__main__":
    sys.exit(main())
