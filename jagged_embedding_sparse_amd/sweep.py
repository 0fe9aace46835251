"""Dispatch and combine latency against the number of virtual ranks.

"FreeScale: distributed training for sequence recommendation models",
section 4.2 and Figure 7 measure the ranged dispatch and ranged combine
kernels (the preparation of the ID and embedding AllToAll buffers) at world
sizes 32 .. 512. This runs the same two operations of this library on one
batch of a workload while W varies:

  dispatch  fs_bucketize_permute: balanced batch -> shard-major IDs and the
            W x W splits (after fs_balance_fbs, timed separately)
  combine   fs_ranged_combine: one row per dispatched ID (dim x dtype of the
            workload's first table) back to the batch-major slots

The same section names the keyed transpose (feature-major to batch-major
jagged tensors) among those kernels; `--transpose` times fs_keyed_transpose
on the workload's samples as F sequence features, each list as long as the
sample's token count, for F in `--features`, against HBM bytes
2 * n * 8 (values) + 4 * F * B (lengths) + 8 * (F * B + 1) (offsets), with
torch's device copy of the same n values beside it for context.

Each figure is the median over `--reps` calls timed with HIP events on the
calling stream, inputs resident in HBM. Usage:

  python -m jagged_embedding_sparse_amd.sweep [--config 5] [--reps 20] [--out FILE]
  python -m jagged_embedding_sparse_amd.sweep --transpose [--features 1,4,8,16]
"""

from __future__ import annotations

import argparse
import sys

import numpy as np
import torch

from . import lib, synth


def _time(fn, reps):
    fn()
    torch.cuda.synchronize()
    ts = []
    for _ in range(reps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        fn()
        b.record()
        torch.cuda.synchronize()
        ts.append(a.elapsed_time(b) * 1e3)
    return float(np.median(ts))


def transpose_lines(k, features, reps):
    w = synth.workload(k)
    b = synth.Batches(w, k).batch(0)
    per = np.diff(b["sample_offsets"]).astype(np.int32)
    B = len(per)
    lines = [f"workload {k}: {w.name}; keyed transpose of F features x {B} samples, "
             "int64 values, list (f, b) = sample b's token count",
             f"{'F':>4s} {'values':>11s} {'us':>9s} {'GB/s':>7s} {'of 8 TB/s':>10s} "
             f"{'copy us':>8s} {'copy GB/s':>10s}"]
    for F in features:
        lengths = torch.from_numpy(np.tile(per, (F, 1))).cuda()
        n = int(per.sum()) * F
        vals = torch.randint(0, 1 << 40, (n,), dtype=torch.int64, device="cuda")
        out = torch.empty_like(vals)
        offs = torch.empty(F * B + 1, dtype=torch.int64, device="cuda")
        ws = torch.empty(lib.keyed_transpose_workspace_size(F, B), dtype=torch.uint8,
                         device="cuda")
        t = _time(lambda: lib.fs_keyed_transpose(vals, lengths, out=out, out_offsets=offs,
                                                 ws=ws), reps)
        gbs = (16 * n + 12 * F * B + 8) / t / 1e3
        # context: torch's device copy of the same values
        tc = _time(lambda: out.copy_(vals), reps)
        lines.append(f"{F:4d} {n:11d} {t:9.1f} {gbs:7.0f} {gbs / 8000:10.1%} {tc:8.1f} "
                     f"{16 * n / tc / 1e3:10.0f}")
        del vals, out
    return lines


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--config", type=int, default=5)
    ap.add_argument("--worlds", default="32,64,128,256,512")
    ap.add_argument("--reps", type=int, default=20)
    ap.add_argument("--out", default=None)
    ap.add_argument("--transpose", action="store_true")
    ap.add_argument("--features", default="1,4,8,16")
    args = ap.parse_args(argv)
    if args.transpose:
        text = "\n".join(transpose_lines(args.config, [int(x) for x in args.features.split(",")],
                                         args.reps))
        print(text, flush=True)
        if args.out:
            with open(args.out, "w") as f:
                f.write(text + "\n")
        return 0
    w = synth.workload(args.config)
    b = synth.Batches(w, args.config).batch(0)
    dev = lambda x: torch.from_numpy(x).cuda()
    uih, so, ids = dev(b["uih_len"]), dev(b["sample_offsets"]), dev(b["ids"])
    rows = [t.rows for t in w.tables]
    T, n_tok, N = len(rows), b["n_tok"], len(b["uih_len"])
    spec = w.tables[0]
    dt = torch.bfloat16 if spec.dtype == "bf16" else torch.float32
    row_bytes = spec.dim * (2 if spec.dtype == "bf16" else 4)
    dims, dts = [spec.dim] * T, [dt] * T
    src = torch.randint(0, 256, (T * n_tok, row_bytes), dtype=torch.uint8, device="cuda")
    outs = [torch.empty((n_tok, spec.dim), dtype=dt, device="cuda") for _ in range(T)]
    lines = [f"workload {args.config}: {w.name}; {N} samples, {T} x {n_tok} IDs; combine rows "
             f"{row_bytes} B ({spec.dim} x {spec.dtype})",
             f"{'W':>5s} {'balance us':>11s} {'dispatch us':>12s} {'combine us':>11s} "
             f"{'dispatch GIDs/s':>16s} {'combine GB/s':>13s}"]
    for W in [int(x) for x in args.worlds.split(",")]:
        if W > lib.FS_MAX_RANKS:
            continue
        perm = torch.empty(N, dtype=torch.int32, device="cuda")
        ro = torch.empty(W + 1, dtype=torch.int32, device="cuda")
        ws_b = torch.empty(lib.balance_workspace_size(N, W), dtype=torch.uint8, device="cuda")
        ws_k = torch.empty(lib.bucketize_workspace_size(n_tok, N, T, W), dtype=torch.uint8,
                           device="cuda")
        bk = {}
        t_bal = _time(lambda: lib.fs_balance_fbs(uih, W, perm, ro, ws=ws_b), args.reps)
        t_dis = _time(lambda: bk.update(lib.fs_bucketize_permute(ids, so, rows, perm, ro, W,
                                                                  out=bk or None, ws=ws_k)),
                      args.reps)
        nv = int(bk["shard_offsets"][-1])
        t_com = _time(lambda: lib.fs_ranged_combine(src, bk, W, dims, dts, rows, n_tok, out=outs),
                      args.reps)
        lines.append(f"{W:5d} {t_bal:11.1f} {t_dis:12.1f} {t_com:11.1f} "
                     f"{T * n_tok / t_dis / 1e3:16.2f} {2 * nv * row_bytes / t_com / 1e3:13.0f}")
    text = "\n".join(lines)
    print(text, flush=True)
    if args.out:
        with open(args.out, "w") as f:
            f.write(text + "\n")
    return 0


if __name__ == "__main__":
    sys.exit(main())
