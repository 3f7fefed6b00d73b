"""HBM traffic of one kernel from rocprofv3 counters, calibrated on a plain copy.

The TCC counters FETCH_SIZE and WRITE_SIZE (KiB per dispatch) are read in two
separate counter runs (the hardware cannot collect both in one pass).  They
are scaled by what the same counters read for a device-to-device copy of a
known number of bytes, so that the result is in bytes of HBM traffic per
launch.  Steps, each under rocprofv3 on the GPU:

    rocprofv3 --pmc FETCH_SIZE --output-format csv -d D/cf -o run -- \\
        python3 -m matmul_affine_qmv_amd.traffic copy --mib 256
    rocprofv3 --pmc WRITE_SIZE --output-format csv -d D/cw -o run -- \\
        python3 -m matmul_affine_qmv_amd.traffic copy --mib 256
    rocprofv3 --pmc FETCH_SIZE --output-format csv -d D/kf -o run -- python3 bench.py --workload only:CALL ...
    rocprofv3 --pmc WRITE_SIZE --output-format csv -d D/kw -o run -- python3 bench.py --workload only:CALL ...

then, on any machine:

    python3 -m matmul_affine_qmv_amd.traffic summarize --dir D --call CALL --kernel SUBSTRING \\
        --label LABEL --copy-mib 256 --out profiles/traffic_CALL.json

The summary records a digest of the kernel sources; bench.py reports the
traffic only while the sources still match it.
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import statistics
import sys

HERE = os.path.dirname(os.path.abspath(__file__))


def source_digest() -> str:
    """sha256 over the library's kernel sources (csrc/*, without the
    calibration kernels, which are not part of it), in name order."""
    h = hashlib.sha256()
    for path in sorted(glob.glob(os.path.join(HERE, "csrc", "*"))):
        if os.path.basename(path).startswith("calib"):
            continue
        h.update(os.path.basename(path).encode())
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def _counter_values(run_dir: str, counter: str, kernel_substring: str):
    """Per-dispatch values of `counter` for dispatches whose kernel name holds the substring."""
    files = glob.glob(os.path.join(run_dir, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no counter_collection.csv under {run_dir}")
    vals, names = [], set()
    for path in files:
        with open(path, newline="") as f:
            for row in csv.DictReader(f):
                if row["Counter_Name"] != counter or kernel_substring not in row["Kernel_Name"]:
                    continue
                vals.append(float(row["Counter_Value"]))
                names.add(row["Kernel_Name"].split("(")[0].replace("void ", ""))
    if not vals:
        raise SystemExit(f"no {counter} values for '{kernel_substring}' under {run_dir}")
    return vals, sorted(names)


def run_copy(mib: int, reps: int) -> None:
    import torch
    n = mib * 2 ** 20 // 4
    src = torch.full((n,), 1.5, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(reps):
        torch.mul(src, 1.0, out=dst)   # one elementwise kernel: reads n floats, writes n floats
    torch.cuda.synchronize()
    print(f"copied {mib} MiB {reps} times", flush=True)


def summarize(args) -> dict:
    copy_bytes = args.copy_mib * 2 ** 20
    cf, _ = _counter_values(os.path.join(args.dir, "cf"), "FETCH_SIZE", args.copy_kernel)
    cw, _ = _counter_values(os.path.join(args.dir, "cw"), "WRITE_SIZE", args.copy_kernel)
    kf, names = _counter_values(os.path.join(args.dir, "kf"), "FETCH_SIZE", args.kernel)
    kw, _ = _counter_values(os.path.join(args.dir, "kw"), "WRITE_SIZE", args.kernel)
    # a copy of B bytes reads B and writes B: bytes per counted KiB
    f_scale = copy_bytes / statistics.median(cf)
    w_scale = copy_bytes / statistics.median(cw)
    fetch = statistics.median(kf) * f_scale
    write = statistics.median(kw) * w_scale
    return {
        "call": args.call,
        "kernel_label": args.label,
        "kernels": names,
        "dispatches": {"fetch": len(kf), "write": len(kw)},
        "fetch_size_kib_median": statistics.median(kf),
        "write_size_kib_median": statistics.median(kw),
        "copy_calibration": {"bytes": copy_bytes, "fetch_size_kib": statistics.median(cf),
                             "write_size_kib": statistics.median(cw), "fetch_bytes_per_kib": f_scale,
                             "write_bytes_per_kib": w_scale},
        "fetch_bytes_per_launch": fetch,
        "write_bytes_per_launch": write,
        "traffic_bytes_per_launch": fetch + write,
        "source_sha256": source_digest(),
    }


def kernel_stats_markdown(stats_csv: str, substring: str = "qmx::") -> str:
    """rocprofv3 --stats kernel table (run_kernel_stats.csv) as markdown, library kernels only."""
    out = ["| kernel | calls | avg µs | min µs | max µs |", "|---|---:|---:|---:|---:|"]
    with open(stats_csv, newline="") as f:
        for row in csv.DictReader(f):
            if substring not in row["Name"]:
                continue
            name = row["Name"].split("(")[0].replace("void ", "")
            out.append(f"| `{name}` | {row['Calls']} | {float(row['AverageNs']) / 1e3:.2f} | "
                       f"{float(row['MinNs']) / 1e3:.2f} | {float(row['MaxNs']) / 1e3:.2f} |")
    return "\n".join(out) + "\n"


def counters_markdown(run_dirs, substring: str, exclude: str = "") -> str:
    """Median per dispatch of every counter found in the counter_collection.csv
    files under `run_dirs` (one rocprofv3 --pmc pass each), for the dispatches
    whose kernel name holds `substring` (and not `exclude`), as markdown."""
    vals, names = {}, set()
    for d in run_dirs:
        for path in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
            with open(path, newline="") as f:
                for row in csv.DictReader(f):
                    k = row["Kernel_Name"]
                    if substring not in k or (exclude and exclude in k):
                        continue
                    vals.setdefault(row["Counter_Name"], []).append(float(row["Counter_Value"]))
                    names.add(k.split("(")[0].replace("void ", ""))
    if not vals:
        raise SystemExit(f"no counters for '{substring}' under {run_dirs}")
    out = ["kernels: " + ", ".join(f"`{n}`" for n in sorted(names)), "",
           "| counter | median per dispatch | dispatches |", "|---|---:|---:|"]
    for name in sorted(vals):
        v = vals[name]
        out.append(f"| `{name}` | {statistics.median(v):.6g} | {len(v)} |")
    return "\n".join(out) + "\n"


def timeline_markdown(trace_csv: str, per_step: int, steps: int, substring: str = "qmx::") -> str:
    """Per position of a replayed step: the median duration of its kernel and
    the median gap from the previous kernel's end, over the last `steps` steps
    of a --kernel-trace run (each step `per_step` library kernels in order)."""
    rows = []
    with open(trace_csv, newline="") as f:
        for r in csv.DictReader(f):
            if substring in r["Kernel_Name"]:
                rows.append((int(r["Start_Timestamp"]), int(r["End_Timestamp"]),
                             r["Kernel_Name"].split("(")[0].replace("void ", "")))
    rows.sort()
    last = rows[-per_step * steps:]
    if len(last) < per_step * steps:
        raise SystemExit(f"{trace_csv}: fewer than {per_step * steps} library kernels")
    out = ["| position | kernel | duration µs (median) | gap before it µs (median) |", "|---:|---|---:|---:|"]
    for i in range(per_step):
        ks = [last[per_step * j + i] for j in range(steps)]
        dur = statistics.median((e - b) / 1e3 for b, e, _ in ks)
        gaps = [(last[per_step * j + i][0] - last[per_step * j + i - 1][1]) / 1e3
                for j in range(steps) if per_step * j + i > 0]
        out.append(f"| {i} | `{ks[0][2]}` | {dur:.2f} | {statistics.median(gaps) if gaps else 0.0:.2f} |")
    span = statistics.median((last[per_step * j + per_step - 1][1] - last[per_step * j][0]) / 1e3 for j in range(steps))
    busy = statistics.median(sum((e - b) / 1e3 for b, e, _ in last[per_step * j:per_step * (j + 1)])
                             for j in range(steps))
    out += ["", f"Step span (first kernel's start to last kernel's end, median): {span:.1f} µs; "
            f"sum of its kernels' durations: {busy:.1f} µs."]
    return "\n".join(out) + "\n"


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    sub = ap.add_subparsers(dest="cmd", required=True)
    c = sub.add_parser("copy", help="elementwise device-to-device copy of a known size (calibration)")
    c.add_argument("--mib", type=int, default=256)
    c.add_argument("--reps", type=int, default=10)
    s = sub.add_parser("summarize", help="turn four counter runs into bytes per launch")
    s.add_argument("--dir", required=True)
    s.add_argument("--call", required=True)
    s.add_argument("--kernel", required=True, help="substring of the kernel name to keep")
    s.add_argument("--label", required=True, help="kernel label bench.py reports for this kernel")
    s.add_argument("--copy-kernel", default="MulFunctor", help="substring of the copy kernel's name")
    s.add_argument("--copy-mib", type=int, default=256)
    s.add_argument("--out", required=True)
    t = sub.add_parser("stats", help="markdown table of the library kernels in a --stats run")
    t.add_argument("csv", help="run_kernel_stats.csv")
    k = sub.add_parser("counters", help="median per dispatch of the counters of several --pmc passes")
    k.add_argument("dirs", nargs="+", help="one rocprofv3 output directory per pass")
    k.add_argument("--kernel", required=True, help="substring of the kernel name to keep")
    k.add_argument("--exclude", default="", help="substring of kernel names to drop")
    tl = sub.add_parser("timeline", help="per-position kernel durations and gaps of a replayed step")
    tl.add_argument("csv", help="run_kernel_trace.csv")
    tl.add_argument("--per-step", type=int, required=True, help="library kernels per step")
    tl.add_argument("--steps", type=int, required=True, help="the last N steps of the trace")
    args = ap.parse_args(argv)
    if args.cmd == "timeline":
        print(timeline_markdown(args.csv, args.per_step, args.steps), end="")
        return 0
    if args.cmd == "stats":
        print(kernel_stats_markdown(args.csv), end="")
        return 0
    if args.cmd == "counters":
        print(counters_markdown(args.dirs, args.kernel, args.exclude), end="")
        return 0
    if args.cmd == "copy":
        run_copy(args.mib, args.reps)
        return 0
    res = summarize(args)
    with open(args.out, "w") as f:
        json.dump(res, f, indent=1)
    print(json.dumps(res, indent=1))
    return 0


if __name__ == "__main__":
    sys.exit(main())
