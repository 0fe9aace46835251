"""HBM traffic of the step's kernels from rocprofv3 counters.

Two passes over the same program, one counter each (the counter blocks do not
hold both at once):

    rocprofv3 --pmc FETCH_SIZE --output-format csv -d <dir_f> -o run -- \
        python3 jagged_embedding_sparse_amd/traffic.py run [--config K]
    rocprofv3 --pmc WRITE_SIZE --output-format csv -d <dir_w> -o run -- \
        python3 jagged_embedding_sparse_amd/traffic.py run [--config K]
    python3 jagged_embedding_sparse_amd/traffic.py summarize \
        <dir_f>/run_counter_collection.csv <dir_w>/run_counter_collection.csv \
        --config K --out profiles/traffic_workload<K>.json

`run` first copies 1 GiB device to device three times (the runtime's plain
copy kernel: exactly 1 GiB read and 1 GiB written per dispatch), then runs a
few steps of the synchronous schedule of bench.py. `summarize` divides each
kernel's counter by what the counter reads for that copy per KiB moved (the
calibration factor), and records per-dispatch bytes per kernel, the bytes of
one update launch (k_short + k_medium + k_long + k_fix) and one lookup
launch, and a hash of the kernel sources the figures belong to: bench.py
reports them only while the sources are unchanged. With --txt it also writes
a readable table: every kernel's bytes per step and the index kernels' total
beside their algorithmic bytes.
"""

from __future__ import annotations

import argparse
import csv
import hashlib
import json
import os
import sys
from collections import defaultdict

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CALIB_BYTES = 1 << 30

# kernels of each stage and the sources they are built from
STAGES = {
    "update_all": (("k_short", "k_short_set", "k_medium", "k_medium_set", "k_long",
                    "k_long_set", "k_fix", "k_fix_set"), ("reduce_update.hip", "common.hpp")),
    "lookup_all": (("k_lookup",), ("gather.hip", "common.hpp")),
}


def sources_sha(stage: str) -> str:
    h = hashlib.sha256()
    for f in STAGES[stage][1]:
        with open(os.path.join(HERE, "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def run(config: int) -> None:
    import torch

    torch.cuda.set_device(0)
    src = torch.empty(CALIB_BYTES, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst
    sys.path.insert(0, ROOT)
    import bench

    sys.argv = ["bench.py", "--config", str(config), "--sync", "--steps", "3", "--warmup", "1",
                "--batches", "3", "--no-cpu-baseline", "--no-per-config"]
    bench.main()


def _read(path: str):
    """kernel name -> list of counter values (KiB per dispatch)."""
    out = defaultdict(list)
    with open(path) as fh:
        for row in csv.DictReader(fh):
            out[row["Kernel_Name"]].append(float(row["Counter_Value"]))
    return out


def _short(name: str) -> str:
    base = name.replace("(anonymous namespace)::", "").replace("void ", "").strip()
    base = base.split("(")[0].split("<")[0]
    return base.split("::")[-1]


def summarize(fetch_csv: str, write_csv: str, config: int, out_path: str | None) -> dict:
    fetch, write = _read(fetch_csv), _read(write_csv)
    copy = [k for k in fetch if "copyBuffer" in k]
    assert copy, "no copy kernel in the fetch pass"
    kib = CALIB_BYTES / 1024
    # the three calibration copies are the largest copies of the run
    f_cal = sorted(fetch[copy[0]])[-3:]
    w_cal = sorted(write[copy[0]])[-3:]
    f_factor = (sum(f_cal) / len(f_cal)) / kib
    w_factor = (sum(w_cal) / len(w_cal)) / kib
    kernels = {}
    for name in sorted(set(fetch) | set(write)):
        s = _short(name)
        if not s.startswith("k_"):
            continue
        fv, wv = fetch.get(name, []), write.get(name, [])
        kernels[name] = {
            "short": s, "dispatches": max(len(fv), len(wv)),
            "fetch_bytes": (sum(fv) / len(fv)) * 1024 / f_factor if fv else None,
            "write_bytes": (sum(wv) / len(wv)) * 1024 / w_factor if wv else None}
    stages = {}
    for stage, (names, _) in STAGES.items():
        tot_f = tot_w = 0.0
        launches = None
        for v in kernels.values():
            if v["short"] in names and v["fetch_bytes"] is not None and v["write_bytes"] is not None:
                tot_f += v["fetch_bytes"] * v["dispatches"]
                tot_w += v["write_bytes"] * v["dispatches"]
                # a launch of the stage starts with its first kernel (a
                # table's own or the shared one; several tables' own
                # launches count once per table)
                if v["short"] in names[:2]:
                    launches = max(launches or 0, v["dispatches"])
        if launches:
            stages[stage] = {"fetch_bytes_per_launch": tot_f / launches,
                             "write_bytes_per_launch": tot_w / launches,
                             "bytes_per_launch": (tot_f + tot_w) / launches,
                             "launches": launches, "sources_sha": sources_sha(stage)}
    res = {"config": config,
           "calibration": {"copy_bytes": CALIB_BYTES, "fetch_factor": f_factor,
                           "write_factor": w_factor},
           "stages": stages, "kernels": kernels}
    text = json.dumps(res, indent=1)
    if out_path:
        with open(out_path, "w") as fh:
            fh.write(text + "\n")
    print(text)
    return res


# kernels of the index stages (balance, bucketize, dedup + collision split)
INDEX_KERNELS = ("k_rank_part", "k_place", "k_vbs_cut", "k_balance_small", "k_lens", "k_bal",
                 "k_tiles", "k_prep1", "k_hist", "k_colsum", "k_colscan", "k_colscan1",
                 "k_scatter", "k_seg_prep", "k_seg_hist", "k_seg_groups", "k_seg_scatter",
                 "k_heads", "k_heads_scan", "k_compact", "k_compact_scan", "k_dedup_small",
                 "k_collide", "k_collide_counts")


def table(res: dict, steps: int, index_algorithmic: float | None, cmd: str | None = None) -> str:
    """Per-kernel HBM bytes per iteration (`steps` iterations in the run) and
    the index kernels' total against their algorithmic bytes; `cmd`, the
    commands that made the counters, heads the table."""
    lines = [f"Commands: {cmd}", ""] if cmd else []
    lines.append("kernel                               dispatches   fetch MB/iter  write MB/iter")
    idx = 0.0
    for name, v in sorted(res["kernels"].items(), key=lambda kv: kv[1]["short"]):
        per = v["dispatches"] / steps
        f = (v["fetch_bytes"] or 0.0) * per / 1e6
        w = (v["write_bytes"] or 0.0) * per / 1e6
        label = v["short"] + ("<int64 in>" if "<long" in name else
                              "<u32 in>" if "<unsigned int" in name else "")
        lines.append(f"{label:36s} {v['dispatches']:10d} {f:15.2f} {w:14.2f}")
        if v["short"] in INDEX_KERNELS:
            idx += (f + w) * 1e6
    for st, v in res["stages"].items():
        lines.append(f"{st}: {v['fetch_bytes_per_launch'] / 1e9:.3f} GB fetched + "
                     f"{v['write_bytes_per_launch'] / 1e9:.3f} GB written = "
                     f"{v['bytes_per_launch'] / 1e9:.3f} GB per launch ({v['launches']} "
                     f"launches; kernel sources {v['sources_sha']})")
    extra = ""
    if index_algorithmic:
        extra = (f" against {index_algorithmic / 1e9:.3f} GB algorithmic "
                 f"({idx / index_algorithmic:.2f}x)")
    lines.append(f"index kernels (balance, bucketize, dedup, collision split): "
                 f"{idx / 1e9:.3f} GB per iteration{extra}")
    return "\n".join(lines) + "\n"


def load_traffic(config: int, stage: str):
    """Bytes per launch of `stage` from profiles/, or None when absent or taken
    on other kernel sources."""
    path = os.path.join(ROOT, "profiles", f"traffic_workload{config}.json")
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        res = json.load(fh)
    st = res.get("stages", {}).get(stage)
    if not st or st.get("sources_sha") != sources_sha(stage):
        return None
    return st["bytes_per_launch"]


def main() -> None:
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd", required=True)
    r = sub.add_parser("run")
    r.add_argument("--config", type=int, default=5)
    s = sub.add_parser("summarize")
    s.add_argument("fetch_csv")
    s.add_argument("write_csv")
    s.add_argument("--config", type=int, default=5)
    s.add_argument("--out", default=None)
    s.add_argument("--txt", default=None, help="also write the readable table here")
    s.add_argument("--steps", type=int, default=None,
                   help="iterations the run made (default: the lookup's launches)")
    s.add_argument("--index-bytes", type=float, default=None,
                   help="algorithmic bytes of the index stages per step")
    s.add_argument("--cmd", default=None, help="the commands that made the counters (for --txt)")
    a = ap.parse_args()
    if a.cmd == "run":
        run(a.config)
    else:
        res = summarize(a.fetch_csv, a.write_csv, a.config, a.out)
        if a.txt:
            # one lookup launch per iteration (the prologue's included)
            steps = a.steps or res["stages"]["lookup_all"]["launches"]
            with open(a.txt, "w") as fh:
                fh.write(table(res, steps, a.index_bytes, a.cmd))


if __name__ == "__main__":
    main()
