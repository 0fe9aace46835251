"""Benchmark of the prioritized jagged sparse step on one MI355X.

A step is one pass of the whole hot path over one batch. Default schedule
(--lookahead 2): on the caller's stream the update of every unique row of
iteration i (segment-reduce + optimizer), then the lookup of every row of
iteration i+1; beside them, on stream A, balance (FBS or VBS), indexed
permute + shard bucketize and dedup + collision split of the batch after
next. --lookahead 1 runs the index stages one iteration ahead instead, with
the exclusive rows' lookup ahead of the update where that pays (--lookup);
--sync runs everything on one stream in the order index, update, lookup.
Inputs (IDs, lengths, gradients, tables) are resident in HBM before the
timed region; the timed region is K steps bracketed by
torch.cuda.synchronize().

value = IDs/s (token x table lookups of the new batch per step, summed over
the K steps, divided by the elapsed time of the K steps). Extra steps after
the timed ones give the per-stage breakdown and the per-step median, minimum
and maximum.

Defaults: workload 5 (B=4096, W=512, one 200M x 128 bf16 table with row-wise
Adagrad, lognormal(6.5, 1.3) lengths capped at 32768, ~6.3M IDs per batch).
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "sparse-step IDs/s and achieved HBM GB/s (% of MI355X peak) per config"
HBM_PEAK_GBPS = 8000.0


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", type=int, default=5, help="workload 1..5")
    ap.add_argument("--balancer", choices=["fbs", "vbs"], default=None)
    ap.add_argument("--seed", type=int, default=None)
    ap.add_argument("--batches", type=int, default=None, help="distinct batches to cycle")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--sync", action="store_true",
                    help="one-stream synchronous schedule (analysis: isolated kernel times)")
    ap.add_argument("--lookup", choices=["auto", "split", "joined"], default="auto",
                    help="exclusive-row lookup ahead of the update (split), one lookup after "
                         "it (joined), or chosen from the first steps' timing (auto)")
    ap.add_argument("--lookahead", type=int, choices=[1, 2], default=2,
                    help="iterations the index stages run ahead of the lookup (2: beside the "
                         "update and the lookup of the iteration before)")
    ap.add_argument("--layout", choices=["dense", "rowstate", "rowstate256"], default="dense",
                    help="tables as dense [rows][dim] with a separate state array, or each "
                         "row's Adagrad state in the row's own padding")
    ap.add_argument("--autotune", action="store_true",
                    help="VBS AutoTune: shares of the weight moved every step by the modelled "
                         "per-rank time (VBS workloads only)")
    return ap.parse_args()


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def byte_model(w, t, n, U, kind):
    """Algorithmic bytes of one stage for table t: n occurrences (token
    lookups) of the class and U unique rows of it (the design notes' model)."""
    spec = w.tables[t]
    e = 2 if spec.dtype == "bf16" else 4
    D = spec.dim
    if kind == "lookup":
        return n * (D * e + 4) + U * (D * e + 12)
    return n * (4 * D + 4) + U * (2 * D * e + 16 + (8 if w.optim == "rw_adagrad" else 0))


def index_bytes(w, n, U):
    W = w.world
    return 20 * n + 8 * W * W + 12 * n + 12 * U + 34 * U


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the multi-GPU "
              "sharding of this path is described, not built.", file=sys.stderr)
        sys.exit(2)
    import torch

    from jagged_embedding_sparse_amd import lib, synth
    from jagged_embedding_sparse_amd.step import SparseStep, StageTimer

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    w = synth.workload(args.config, args.balancer)
    seed = args.seed if args.seed is not None else args.config
    NB = args.batches or min(w.iterations, args.warmup + args.steps + 1)
    NB = max(NB, 2)
    log(f"workload {args.config} {w.name} balancer={w.balancer} batches={NB}")

    t0 = time.time()
    gen = synth.Batches(w, seed)
    host_batches = [gen.batch(i) for i in range(NB)]
    log(f"generated {NB} batches in {time.time() - t0:.1f}s; IDs/batch "
        f"{np.mean([b['n_tok'] * len(w.tables) for b in host_batches]):.0f}")
    dev_batches = [dict(uih_len=torch.from_numpy(b["uih_len"]).cuda(),
                        sample_offsets=torch.from_numpy(b["sample_offsets"]).cuda(),
                        ids=torch.from_numpy(b["ids"]).cuda()) for b in host_batches]
    cap = max(b["n_tok"] for b in host_batches)
    weights, states = [], []
    ada = w.optim == "rw_adagrad"
    for t, spec in enumerate(w.tables):
        if args.layout.startswith("rowstate"):
            tdt = torch.float32 if spec.dtype == "f32" else torch.bfloat16
            wv, st = lib.alloc_table(spec.rows, spec.dim, tdt, ada, device="cuda",
                                     align=256 if args.layout == "rowstate256" else 16)
            weights.append(synth.init_table(spec.rows, spec.dim, spec.dtype, seed, "cuda",
                                            table=t, out=wv))
            states.append(st.zero_() if st is not None else None)
        else:
            weights.append(synth.init_table(spec.rows, spec.dim, spec.dtype, seed, "cuda",
                                            table=t))
            states.append(torch.zeros(spec.rows, dtype=torch.float32, device="cuda")
                          if ada else None)
    t0 = time.time()
    grads_host = [synth.gradient_rows(seed, 0, t, np.arange(cap), spec.dim)
                  for t, spec in enumerate(w.tables)]
    grads_dev = [torch.from_numpy(g).cuda() for g in grads_host]
    log(f"gradients {cap} x {[s.dim for s in w.tables]} in {time.time() - t0:.1f}s")

    ahead = args.lookahead == 2 and not args.sync
    step = SparseStep(w, weights, states, cap, lookup=args.lookup,
                      lookahead=2 if ahead else 1, autotune={} if args.autotune else None)
    n_tok = [b["n_tok"] for b in host_batches]
    step.prologue(dev_batches[0], batch_after=dev_batches[1 % NB] if ahead else None)
    if args.sync:
        def run_step(batch_next, grads, k_next):
            return step.step_sync(batch_next, grads)
    else:
        def run_step(batch_next, grads, k_next):
            # with lookahead 2 the step also indexes the batch after next
            return step.step(batch_next, grads,
                             batch_after=dev_batches[(k_next + 1) % NB] if ahead else None)
    k = 0
    for _ in range(args.warmup):
        k += 1
        run_step(dev_batches[k % NB], [g[:n_tok[(k - 1) % NB]] for g in grads_dev], k)
    step.join()
    torch.cuda.synchronize()

    # ---------------------------------------------------------------- timed region
    # Only the update (the roofline's kernel) carries timing events here:
    # every event record costs the GPU a few microseconds between kernels
    # (measured: 0.41 instead of 0.37 ms per step on workload 3 with all six
    # stages timed); the stage breakdown comes from extra steps afterwards.
    # A first, larger event pool, used and dropped, leaves the runtime enough
    # recycled event resources that the timed pool's records stay cheap
    # (without it, 1.5 ms of host time per step on the smallest workload).
    n_brk = min(args.steps, 10)
    warm = StageTimer(capacity=24 * (args.steps + n_brk), streams=(step.sA, step.sB))
    del warm
    timer = StageTimer(capacity=2 * args.steps, streams=(step.sA, step.sB),
                       only=("update_all",))
    step.timer = timer
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    pairs = []
    ids_timed = 0
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    # both events on the caller's stream: the steps' streams wait for it at
    # the start of each step, and it waits for both of them at the end
    ev0.record()
    for _ in range(args.steps):
        p = k % NB
        k += 1
        run_step(dev_batches[k % NB], [g[:n_tok[p]] for g in grads_dev], k)
        pairs.append(p)
        ids_timed += n_tok[k % NB] * len(w.tables)
    submit = time.perf_counter() - wall0
    step.join()
    ev1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    step.timer = None
    schedule = ("sync" if args.sync else "index two ahead, joined lookup" if ahead else
                ("joined" if step.joined else "split"))
    ms_total = ev0.elapsed_time(ev1)
    ms_step = ms_total / args.steps
    upd_ms = timer.ms()["update_all"]
    log(f"timed {args.steps} steps: {ms_total:.3f} ms (wall {wall * 1e3:.3f} ms, host "
        f"submission {submit * 1e3:.3f} ms)")

    # ---------------------------------------------------------------- stage breakdown
    brk = StageTimer(capacity=8 * n_brk, streams=(step.sA, step.sB))
    step.timer = brk
    for _ in range(n_brk):
        p = k % NB
        k += 1
        run_step(dev_batches[k % NB], [g[:n_tok[p]] for g in grads_dev], k)
    step.join()
    torch.cuda.synchronize()
    step.timer = None
    stage_ms = brk.ms()

    # ---------------------------------------------------------------- per-step spread
    # K more steps with one event per step on the stream that ends each step
    # (kept out of the timed region: each record costs the GPU a few
    # microseconds): with the index stages two ahead the caller's stream,
    # whose lookup waits for the index stream; otherwise stream A, whose
    # last lookup waits for the update (and with --sync runs everything).
    end_stream = torch.cuda.current_stream() if ahead else step.sA
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    for e in evs:  # first records take fresh runtime resources: not in the loop
        e.record(end_stream)
    torch.cuda.synchronize()
    evs[0].record(end_stream)
    for j in range(args.steps):
        p = k % NB
        k += 1
        run_step(dev_batches[k % NB], [g[:n_tok[p]] for g in grads_dev], k)
        evs[j + 1].record(end_stream)
    step.join()
    torch.cuda.synchronize()
    per_step = np.array([evs[j].elapsed_time(evs[j + 1]) for j in range(args.steps)])

    # ---------------------------------------------------------------- accounting
    # Units per batch pair (p -> p+1) depend only on the IDs, so one more cycle
    # of steps, synchronised, gives them for every pair the timed steps used.
    units = {}
    for _ in range(NB):
        p = k % NB
        k += 1
        prev = step.cur
        nxt = run_step(dev_batches[k % NB], [g[:n_tok[p]] for g in grads_dev], k)
        step.join()
        torch.cuda.synchronize()
        T, W = len(w.tables), w.world

        def per_table(st, cls_t):
            U = int(st.uq["counts"][0])
            uo = st.uq["unique_offsets"].cpu().numpy()
            seg = st.uq["seg_offsets"][:U + 1].long()
            ln = seg[1:] - seg[:-1]
            c = cls_t[:U].long()
            co, ex = [], []
            for t in range(T):
                a, b = int(uo[t * W]), int(uo[(t + 1) * W])
                co.append((int((ln[a:b] * c[a:b]).sum()), int(c[a:b].sum())))
                ex.append((int((ln[a:b] * (1 - c[a:b])).sum()), int((1 - c[a:b]).sum())))
            return co, ex, U

        lco, lex, U = per_table(nxt, nxt.uq["cls"])
        uco, uex, _ = per_table(prev, prev.cls_next)
        units[p] = dict(lookup_co=lco, lookup_ex=lex, update_co=uco, update_ex=uex,
                        n_new=n_tok[k % NB] * T, U_new=U)
    assert int(step.err.item()) == 0, f"device error flags {int(step.err.item())}"

    # per-stage bytes over the timed launches
    parts = {"lookup_co": ["lookup_co"], "lookup_ex": ["lookup_ex"], "update_co": ["update_co"],
             "update_ex": ["update_ex"], "lookup_all": ["lookup_co", "lookup_ex"],
             "update_all": ["update_co", "update_ex"]}
    stage_bytes = {}
    step_bytes = 0
    for p in pairs:
        u = units[p]
        per = {name: sum(byte_model(w, t, n, Uc, name.split("_")[0]) for t, (n, Uc) in
                         enumerate(u[name]))
               for name in ("lookup_co", "lookup_ex", "update_co", "update_ex")}
        for stage, names in parts.items():
            stage_bytes[stage] = stage_bytes.get(stage, 0) + sum(per[x] for x in names)
        step_bytes += sum(per.values()) + index_bytes(w, u["n_new"], u["U_new"])
    stage_avg = {k2: float(np.mean(v)) for k2, v in stage_ms.items()}
    cands = [x for x in parts if x in stage_avg]
    dom = max(cands, key=lambda s: stage_avg[s])
    # the roofline's kernel is timed inside the timed region (the update, the
    # dominant stage on every workload); any other stage from the breakdown
    dom_ms = upd_ms if dom == "update_all" else stage_ms[dom]
    dom_bytes_per_launch = stage_bytes[dom] / len(pairs)
    dom_gbps = dom_bytes_per_launch / (float(np.mean(dom_ms)) * 1e-3) / 1e9
    step_gbps = step_bytes / (ms_total * 1e-3) / 1e9
    value = ids_timed / (ms_total * 1e-3)

    kernel_of = {
        "lookup_co": "k_lookup (fs_jagged_lookup, collision rows)",
        "lookup_ex": "k_lookup (fs_jagged_lookup, exclusive rows)",
        "update_co": "k_short+k_long+k_fix (fs_grad_reduce_update, collision rows)",
        "update_ex": "k_short+k_long+k_fix (fs_grad_reduce_update, exclusive rows)",
        "lookup_all": "k_lookup (fs_jagged_lookup, all rows)",
        "update_all": "k_short+k_long+k_fix (fs_grad_reduce_update, all rows)"}

    # ---------------------------------------------------------------- CPU baseline
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(w, seed, host_batches, grads_host, weights, states)

    # HBM bytes per launch of the dominant stage from the committed counter
    # summary (rocprofv3 FETCH_SIZE / WRITE_SIZE, copy-calibrated), when it was
    # taken on the kernel sources built here and on the same (dense) tables
    from jagged_embedding_sparse_amd.traffic import load_traffic
    traffic = load_traffic(args.config, dom) if args.layout == "dense" else None

    tables = "+".join(f"{t.rows // 1_000_000}Mx{t.dim}-{t.dtype}" if t.rows >= 1_000_000 else
                      f"{t.rows // 1000}Kx{t.dim}-{t.dtype}" for t in w.tables)
    out = {
        "metric": METRIC,
        "value": value,
        "unit": "IDs/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": f"workload {args.config}: {w.name} ({w.balancer.upper()})",
            "global_batch": w.batch, "virtual_ranks": w.world, "tables": tables,
            "optimizer": w.optim, "ids_per_step": ids_timed / args.steps,
            "weights": sorted({t.dtype for t in w.tables}), "grad_accumulate": "f64",
            "distinct_batches": NB, "schedule": schedule,
            "autotune": bool(args.autotune), "layout": args.layout},
        "roofline": {
            "bound": "hbm", "achieved": dom_gbps, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
            "frac": dom_gbps / HBM_PEAK_GBPS, "traffic": traffic,
            "kernel": kernel_of[dom],
            "bytes_per_launch": dom_bytes_per_launch,
            "ms_per_launch": float(np.mean(dom_ms))},
        "step_hbm": {
            "algorithmic_bytes_per_step": step_bytes / args.steps, "GBps": step_gbps,
            "frac": step_gbps / HBM_PEAK_GBPS},
        "stages_ms": stage_avg,
        "stages_note": f"stage breakdown from {n_brk} extra steps with every stage timed",
        "per_step_ms": {"median": float(np.median(per_step)), "min": float(per_step.min()),
                        "max": float(per_step.max()),
                        "note": f"{args.steps} extra steps, one event per step on the stream "
                                "that ends it"},
        "cpu_baseline": cpu,
    }
    print(json.dumps(out))


def cpu_baseline(w, seed, host_batches, grads_host, weights, states):
    """The oracle, as it stands, on one synchronous iteration of the same
    workload (batch 1, collision split against batch 0), on one host core."""
    import torch

    from oracle import oracle as O

    b0, b1 = host_batches[0], host_batches[1]
    stores = []
    for t, spec in enumerate(w.tables):
        rid = np.unique(b1["ids"][t])
        idx = torch.from_numpy(rid).cuda()
        v = weights[t].index_select(0, idx)
        vals = (v.view(torch.int16).cpu().numpy().view(np.uint16) if v.dtype == torch.bfloat16
                else v.cpu().numpy())
        st = states[t].index_select(0, idx).cpu().numpy() if states[t] is not None else None
        stores.append(O.RowStore(rid, vals, st, bf16=v.dtype == torch.bfloat16))
    run = O.SyncRun(w, stores)
    run.prev_unique = run.index_stages(b0)["uniq"]["unique"]  # untimed: context for the split
    n = b1["n_tok"]
    g = [x[:n] for x in grads_host]
    t0 = time.perf_counter()
    run.step(b1, lambda o: g)
    dt = time.perf_counter() - t0
    ids = n * len(w.tables)
    log(f"oracle: {ids} IDs in {dt:.2f}s")
    return {"value": ids / dt, "unit": "IDs/s", "cores": 1, "kind": "oracle",
            "sample": f"one synchronous iteration (balance, bucketize, dedup, collision split, "
                      f"lookup, fp64 reduce, update) of batch 1 of the same workload, {ids} IDs, "
                      f"{dt:.2f} s",
            "host": f"{_cpu_model()}, {os.cpu_count()} logical CPUs visible, 1 used"}


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown CPU"


if __name__ == "__main__":
    main()
