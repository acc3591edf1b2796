"""Summaries of rocprofv3 runs of bench.py for profiles/.

Counters: two runs (FETCH_SIZE, then WRITE_SIZE) become the counter summary
that bench.py reads for its roofline ``traffic`` figures:

    cd /tmp && export TMPDIR=/tmp
    rocprofv3 --pmc FETCH_SIZE --kernel-trace --output-format csv -d <out>/fetch -o run -- \\
        python3 /root/repo/bench.py --steps 4 --warmup 1 --prof-steps 1 --no-cpu-baseline
    rocprofv3 --pmc WRITE_SIZE --kernel-trace --output-format csv -d <out>/write -o run -- \\
        python3 /root/repo/bench.py --steps 4 --warmup 1 --prof-steps 1 --no-cpu-baseline
    python3 bench_pmc.py --workload llama_gqa_128k --fetch <out>/fetch --write <out>/write

For every decode kernel it writes the mean counter value (KiB) per dispatch
over all dispatches of the run, and the hash of that kernel's sources (so
bench.py stops using a figure once the kernel changes).  The calibration
copy that every bench run makes (torch.neg over 512 MiB: reads and writes
512 MiB) gives the factor that turns each counter into bytes.

Kernel trace: ``python3 bench_pmc.py --trace <out>/trace --workload W
--bench-line <bench stdout> --cmd "..."`` writes a Markdown summary of a
``rocprofv3 --kernel-trace --stats`` run of bench.py: every decode kernel's
launch count and mean / min / max duration over the whole run, and its mean
over the bench's per-kernel event pass (the last prof-steps x L_rot launches
of each kernel), the region whose HIP-event timings the bench line reports.
"""
from __future__ import annotations

import argparse
import csv
import glob
import os
import re
import sys
from collections import defaultdict

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import bench  # noqa: E402

# kernel symbols of the decode path -> launch-plan names
SYMBOLS = {"k_step_score": "step_score", "k_score": "score", "k_select_attend": "select_attend",
           "k_select": "select", "k_attend_mfma": "attend", "k_attend": "attend", "k_combine": "combine",
           "k_append": "append", "k_state_add": "state_add", "k_step_fused": "step_fused"}
COPY_MARK = "neg_kernel"


def symbol_of(kernel_name: str):
    """Decode-path symbol of a demangled kernel name, if it is one."""
    # "void spla::(anonymous namespace)::k_name<...>(args)": the name ahead of
    # the first template or argument list
    m = re.search(r"(?:^|::|\s)(k_\w+?)(?:<|\()", kernel_name.replace("(anonymous namespace)", ""))
    return m.group(1) if m and m.group(1) in SYMBOLS else None


def per_dispatch(path: str, counter: str):
    """{symbol or 'copy': [value per dispatch]} from one counter run."""
    files = glob.glob(os.path.join(path, "**", "*counter_collection.csv"), recursive=True) if os.path.isdir(path) \
        else [path]
    if not files:
        raise FileNotFoundError(f"no counter_collection.csv under {path}")
    sums = defaultdict(float)
    names = {}
    for fn in files:
        with open(fn, newline="") as f:
            for row in csv.DictReader(f):
                if row.get("Counter_Name") != counter:
                    continue
                key = (fn, row.get("Dispatch_Id") or row.get("Correlation_Id"))
                sums[key] += float(row["Counter_Value"])
                names[key] = row["Kernel_Name"]
    out = defaultdict(list)
    for key, v in sums.items():
        name = names[key]
        sym = symbol_of(name)
        if sym is not None:
            out[sym].append(v)
        elif COPY_MARK in name:
            out["copy"].append(v)
    return out


def trace_summary(args) -> int:
    import json
    files = glob.glob(os.path.join(args.trace, "**", "*kernel_trace.csv"), recursive=True)
    if not files:
        raise FileNotFoundError(f"no kernel_trace.csv under {args.trace}")
    rows = []
    for fn in files:
        with open(fn, newline="") as f:
            for row in csv.DictReader(f):
                sym = symbol_of(row["Kernel_Name"])
                if sym is None:
                    continue
                rows.append((int(row["Start_Timestamp"]), int(row["End_Timestamp"]), sym, row["Kernel_Name"]))
    rows.sort()
    line = {}
    if args.bench_line:
        with open(args.bench_line) as f:
            for ln in f:
                ln = ln.strip()
                if ln.startswith("{"):
                    line = json.loads(ln)
    L = int(line.get("config", {}).get("l_rot", 0))
    P = args.prof_steps
    by = defaultdict(list)
    names = {}
    for t0, t1, sym, name in rows:
        by[sym].append((t1 - t0) / 1000.0)
        names.setdefault(sym, re.sub(r"^void\s+", "", name.replace("(anonymous namespace)::", "")).split("(")[0])
    out = [f"# Kernel trace: SPLA decode step, {args.workload} workload", "",
           "gfx950 (MI355X), ROCm 7.2, rocprofv3.  Summarised by bench_pmc.py from the run's kernel trace.", "",
           "Command:", "", "```", "cd /tmp && export TMPDIR=/tmp",
           f"rocprofv3 --kernel-trace --stats --output-format csv -d <out>/trace -o run -- {args.cmd}",
           f"python3 bench_pmc.py --trace <out>/trace --workload {args.workload} --bench-line <bench stdout>", "```",
           "", "## Decode kernels", "",
           "| kernel | launches | mean us | min us | max us | mean us, event pass |", "|---|---|---|---|---|---|"]
    for sym, d in sorted(by.items(), key=lambda kv: -sum(kv[1])):
        ev = d[-P * L:] if L and P and len(d) >= P * L else []
        out.append(f"| `{names[sym]}` | {len(d)} | {sum(d) / len(d):.2f} | {min(d):.2f} | {max(d):.2f} | "
                   + (f"{sum(ev) / len(ev):.2f}" if ev else "-") + " |")
    if line:
        out += ["", "## The bench line of the same workload without the tracer (HIP events)", ""]
        if args.bench_cmd:
            out += ["```", args.bench_cmd, "```", ""]
        ku = line.get("kernel_us", {})
        out.append("| kernel | bench us |")
        out.append("|---|---|")
        for k, v in ku.items():
            out.append(f"| `k_{k}` | {v:.2f} |")
        out += ["", f"Step: {line.get('ms_per_step', 0) * 1e3:.2f} us ({line.get('value', 0):.0f} tokens/s); "
                    f"step bytes {line.get('step_bytes', 0) / 1e6:.2f} MB, "
                    f"{line.get('step_frac_of_peak', 0):.3f} of the 8 TB/s peak.  "
                    "Under the tracer the graph-replayed timed region runs slower, so the step time is taken "
                    "from this run without it; the kernel means above are the tracer's own."]
    text = "\n".join(out) + "\n"
    dest = args.out or os.path.join(ROOT, "profiles", f"decode_{args.workload}_trace.md")
    with open(dest, "w") as f:
        f.write(text)
    print(text)
    return 0


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--workload", required=True)
    ap.add_argument("--fetch", help="output directory (or CSV) of the FETCH_SIZE run")
    ap.add_argument("--write", help="output directory (or CSV) of the WRITE_SIZE run")
    ap.add_argument("--trace", help="output directory of a --kernel-trace --stats run (trace summary mode)")
    ap.add_argument("--bench-line", help="stdout of bench.py (its JSON line) for the trace summary")
    ap.add_argument("--bench-cmd", default="", help="the untraced bench command whose line is given")
    ap.add_argument("--prof-steps", type=int, default=16, help="steps of the bench's per-kernel event pass")
    ap.add_argument("--cmd", default="python3 /root/repo/bench.py --steps 4 --warmup 1 --prof-steps 1 "
                                     "--no-cpu-baseline", help="the profiled command, as recorded")
    ap.add_argument("-o", "--out", default=None)
    args = ap.parse_args()
    if args.trace:
        return trace_summary(args)
    if not (args.fetch and args.write):
        ap.error("--fetch and --write are required without --trace")
    fetch = per_dispatch(args.fetch, "FETCH_SIZE")
    write = per_dispatch(args.write, "WRITE_SIZE")
    if not fetch.get("copy") or not write.get("copy"):
        raise RuntimeError("the calibration copy (torch.neg) is missing from a counter run")
    mean = lambda v: sum(v) / len(v)  # noqa: E731
    copy_fetch, copy_write = mean(fetch["copy"]), mean(write["copy"])
    cb = bench.CALIB_BYTES
    fs, ws = cb / (copy_fetch * 1024.0), cb / (copy_write * 1024.0)
    lines = [
        f"# HBM byte counters of the SPLA decode kernels, {args.workload} workload",
        "#",
        "# Two counter passes of the same command (gfx950, rocprofv3, one counter per run), summarised by",
        "# bench_pmc.py:",
        "#   cd /tmp && export TMPDIR=/tmp",
        f"#   rocprofv3 --pmc FETCH_SIZE --kernel-trace --output-format csv -d <out>/fetch -o run -- {args.cmd}",
        f"#   rocprofv3 --pmc WRITE_SIZE --kernel-trace --output-format csv -d <out>/write -o run -- {args.cmd}",
        f"#   python3 bench_pmc.py --workload {args.workload} --fetch <out>/fetch --write <out>/write",
        "# Values are the mean counter value (KiB) per dispatch over every dispatch of the kernel in the run.",
        f"# Calibration: torch.neg over a {cb >> 20} MiB float32 tensor (reads and writes {cb >> 20} MiB);",
        f"# FETCH_SIZE reads {copy_fetch:.1f} KiB for it (scale {fs:.4f}), WRITE_SIZE {copy_write:.1f} KiB "
        f"(scale {ws:.4f}).",
        "#",
        "# kernel              dispatches  FETCH_SIZE KiB  WRITE_SIZE KiB  scaled MB read  scaled MB written",
    ]
    syms = [s for s in SYMBOLS if s in fetch and s in write]
    for s in syms:
        f_, w_ = mean(fetch[s]), mean(write[s])
        lines.append(f"# {s:<20}{len(fetch[s]):>10}{f_:>16.1f}{w_:>16.1f}{f_ * 1024 * fs / 1e6:>16.3f}"
                     f"{w_ * 1024 * ws / 1e6:>18.3f}")
    lines += ["#", "# Read by bench.py (roofline traffic) while a kernel's source_sha256 matches its sources.",
              f"workload = {args.workload}", f"copy_bytes = {cb}", f"copy_fetch_kib = {copy_fetch:.3f}",
              f"copy_write_kib = {copy_write:.3f}"]
    for s in syms:
        name = SYMBOLS[s]
        if name not in bench.KERNEL_SOURCES:
            continue
        lines += ["", f"[k_{name}]", f"symbol = {s}", f"source_sha256 = {bench.kernel_source_hash(name)}",
                  f"dispatches = {len(fetch[s])}", f"fetch_kib_per_dispatch = {mean(fetch[s]):.3f}",
                  f"write_kib_per_dispatch = {mean(write[s]):.3f}"]
    text = "\n".join(lines) + "\n"
    out = args.out or os.path.join(ROOT, bench.PMC_SUMMARY.format(workload=args.workload))
    with open(out, "w") as f:
        f.write(text)
    print(text)
    return 0


if __name__ == "__main__":
    sys.exit(main())
