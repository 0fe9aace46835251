"""Text summary of a rocprofv3 kernel trace of one bench.py run.

    python -m jagged_embedding_sparse_amd.trace_summary STATS_CSV TRACE_CSV BENCH_OUT \
        --cmd "<the profiled command>" [--out FILE]

STATS_CSV and TRACE_CSV are rocprofv3's `--kernel-trace --stats` outputs
(`*_kernel_stats.csv`, `*_kernel_trace.csv`); BENCH_OUT is what the profiled
bench printed (its JSON line is read from it). The summary lists this
library's kernels by total time, then the bench line, then the update's
launch time from the trace: the update (fs_grad_reduce_update) is four
kernels (short, medium and long rows, the long rows' fix-up), on one stream
or as two row parts on two streams, so a launch is four consecutive update
dispatches and its time is the span from the first start to the last end --
the same interval the bench's HIP events bracket.
"""

from __future__ import annotations

import argparse
import csv
import json
import re

UPDATE_KERNELS = ("k_short", "k_medium", "k_long", "k_fix",
                  "k_short_set", "k_medium_set", "k_long_set", "k_fix_set")


def short_name(n: str) -> str:
    n = n.replace("(anonymous namespace)::", "").replace("fs::", "").replace("void ", "")
    m = re.match(r"([A-Za-z_0-9]+)(<[^(]*>)?", n)
    return (m.group(1) + (m.group(2) or "")) if m else n[:40]


def base_name(n: str) -> str:
    return short_name(n).split("<")[0]


def update_spans(trace_rows):
    """Per update launch: (span us, summed kernel us), from groups of four
    consecutive update dispatches."""
    upd = sorted((r for r in trace_rows if base_name(r["Kernel_Name"]) in UPDATE_KERNELS),
                 key=lambda r: int(r["Dispatch_Id"]))
    out = []
    for i in range(0, len(upd) - len(upd) % 4, 4):
        g = upd[i:i + 4]
        kinds = sorted(base_name(r["Kernel_Name"]).replace("_set", "") for r in g)
        if kinds != ["k_fix", "k_long", "k_medium", "k_short"]:
            raise ValueError(f"update dispatches out of step at {i}: {kinds}")
        start = min(int(r["Start_Timestamp"]) for r in g)
        end = max(int(r["End_Timestamp"]) for r in g)
        busy = sum(int(r["End_Timestamp"]) - int(r["Start_Timestamp"]) for r in g)
        out.append(((end - start) / 1e3, busy / 1e3))
    return out


def summarize(stats_csv, trace_csv, bench_out, cmd):
    rows = list(csv.DictReader(open(stats_csv)))
    lines = [f"Command: {cmd}",
             "tool: rocprofv3 --kernel-trace --stats --output-format csv (ROCm 7.2), "
             "MI355X (gfx950)", ""]
    lines.append(f"{'kernel':44s} {'calls':>6s} {'avg us':>9s} {'total ms':>9s} {'%':>6s}")
    other = 0
    for r in sorted(rows, key=lambda r: -float(r["TotalDurationNs"])):
        nm = r["Name"]
        if not ("fs::" in nm or nm.startswith("k_")):
            other += 1
            continue
        lines.append(f"{short_name(nm)[:44]:44s} {int(r['Calls']):6d} "
                     f"{float(r['AverageNs']) / 1e3:9.1f} "
                     f"{float(r['TotalDurationNs']) / 1e6:9.2f} {float(r['Percentage']):6.1f}")
    lines.append(f"(plus {other} torch / runtime kernels of table init, accounting and copies, "
                 "outside the timed region)")
    js = [ln for ln in open(bench_out).read().splitlines() if ln.startswith("{")]
    if js:
        d = json.loads(js[-1])
        rf = d["roofline"]
        lines += ["", "bench line of the same command (printed by the profiled run):",
                  f"  value {d['value']:.4g} IDs/s, {d['ms_per_step']:.4f} ms/step, schedule: "
                  f"{d['config']['schedule']}",
                  f"  step algorithmic {d['step_hbm']['GBps']:.0f} GB/s "
                  f"({d['step_hbm']['frac'] * 100:.1f}% of 8 TB/s)",
                  "  stages (ms; HIP events on each call's stream, from extra steps after the "
                  "timed ones): " + ", ".join(f"{k} {v:.3f}" for k, v in d["stages_ms"].items()),
                  f"  roofline: {rf['kernel']}: {rf['achieved']:.0f} GB/s = "
                  f"{rf['frac'] * 100:.1f}% of 8000, {rf['bytes_per_launch'] / 1e9:.3f} GB per "
                  f"launch, {rf['ms_per_launch']:.4f} ms per launch"]
        spans = update_spans(list(csv.DictReader(open(trace_csv))))
        if spans:
            sp = sum(s for s, _ in spans) / len(spans)
            busy = sum(b for _, b in spans) / len(spans)
            lines.append(f"  update launch from the trace ({len(spans)} launches): first start to "
                         f"last end of its four kernels {sp:.1f} us (their summed durations "
                         f"{busy:.1f} us); bench (HIP events on the caller's stream around the "
                         f"launch) {rf['ms_per_launch'] * 1e3:.1f} us")
    return "\n".join(lines) + "\n"


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("stats_csv")
    ap.add_argument("trace_csv")
    ap.add_argument("bench_out")
    ap.add_argument("--cmd", required=True)
    ap.add_argument("--out")
    a = ap.parse_args()
    txt = summarize(a.stats_csv, a.trace_csv, a.bench_out, a.cmd)
    if a.out:
        with open(a.out, "w") as f:
            f.write(txt)
    print(txt, end="")


if __name__ == "__main__":
    main()
