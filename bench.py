"""Benchmark of the prioritized jagged sparse step on one MI355X.

A step is one pass of the whole hot path over one batch. Default schedule
(--schedule auto, --lookahead 3): on the caller's stream the update of every
unique row of iteration i (segment-reduce + optimizer; from 2^17 IDs its rows
of more than 64 occurrences on a second stream beside the rest), then the
lookup of every row of iteration i+1; beside them, on two index streams taken
in turn, balance (FBS or VBS), indexed permute + shard bucketize, dedup and
collision split of iteration i+3 (only the split waits for the dedup of i+2;
--lookahead 2: one index stream, iteration i+2). Batches of at most 8192 IDs
run the serial schedule instead (every stage on the caller's stream, no
events). --schedule prioritized splits update and lookup by class as the
pages' Algorithm 2 does (collision rows updated, then looked up, on the
caller's stream; exclusive rows of both iterations on two more streams).
--lookahead 1 runs the index stages one iteration ahead instead, with the
exclusive rows' lookup ahead of the update where that pays (--lookup);
--sync runs everything on one stream in the order index, update, lookup.
Inputs (IDs, lengths, gradients, tables) are resident in HBM before the
timed region; the timed region is K steps bracketed by
torch.cuda.synchronize().

value = IDs/s (token x table lookups of the new batch per step, summed over
the K steps, divided by the elapsed time of the K steps). Extra steps after
the timed ones give the per-stage breakdown and the per-step median, minimum
and maximum.

The headline line is workload 5 (B=4096, W=512, one 200M x 128 bf16 table
with row-wise Adagrad, lognormal(6.5, 1.3) lengths capped at 32768, ~6.3M IDs
per batch, FBS). Unless --no-per-config, `per_config` adds the same
measurement for workloads 1-4 and for workload 5 with VBS (alpha 3/2), each
in a process of its own (started after the headline run has released its
memory) with a shorter timed region, and `stats` gives, per workload, the realized
collision rate (by unique rows and by tokens), the padding sparsity of the
pages' Equation 1 (global batch, and the mean over each balancer's local
batches), per-rank token load max/mean under FBS and VBS, empty VBS ranks
and device memory.
"""

from __future__ import annotations

import argparse
import gc
import json
import os
import subprocess
import sys
import time
from dataclasses import dataclass

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "sparse-step IDs/s and achieved HBM GB/s (% of MI355X peak) per config"
HBM_PEAK_GBPS = 8000.0
PER_CONFIG = ((1, None), (2, None), (3, None), (4, None), (5, "vbs"))


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
    ap.add_argument("--no-per-config", action="store_true",
                    help="only the headline workload (profiling runs)")
    ap.add_argument("--per-config-steps", type=int, default=30)
    ap.add_argument("--entry", action="store_true",
                    help="print only this workload's per-config entry (one JSON line); the "
                         "headline run starts one such process per other workload")
    ap.add_argument("--sync", action="store_true",
                    help="one-stream synchronous schedule (analysis: isolated kernel times)")
    ap.add_argument("--schedule", choices=["auto", "joined", "prioritized", "serial"],
                    default="auto",
                    help="with --lookahead 2 or 3: every row updated, then every row looked up "
                         "(joined), or collision rows updated and looked up first with the "
                         "exclusive rows beside them (prioritized); serial: every stage on one "
                         "stream, one iteration at a time; auto: serial for batches of at most "
                         "8192 IDs, else joined")
    ap.add_argument("--lookup", choices=["auto", "split", "joined"], default="auto",
                    help="with --lookahead 1: exclusive-row lookup ahead of the update (split), "
                         "one lookup after it (joined), or chosen from the first steps' timing "
                         "(auto)")
    ap.add_argument("--lookahead", type=int, choices=[1, 2, 3], default=3,
                    help="iterations the index stages run ahead of the lookup (2: beside the "
                         "update and the lookup of the iteration before; 3: on two index "
                         "streams, so that one iteration's balance and bucketize overlap the "
                         "dedup of the one before)")
    ap.add_argument("--layout", choices=["dense", "rowstate", "rowstate256"], default="dense",
                    help="tables as dense [rows][dim] with a separate state array, or each "
                         "row's Adagrad state in the row's own padding")
    ap.add_argument("--graph", choices=["off", "on"], default="off",
                    help="replay each step as a HIP graph captured before the warm-up (index "
                         "stages 2 or 3 ahead; the update's launch time then comes from extra "
                         "steps run without graphs)")
    ap.add_argument("--autotune", action="store_true",
                    help="VBS AutoTune: shares of the weight moved every step by the modelled "
                         "per-rank time (VBS workloads only)")
    return ap.parse_args()


# batches of at most this many IDs (token x table) run the serial schedule
# under --schedule auto: with a few thousand IDs a step is a chain of short
# launches, and the host's cost of cross-stream events exceeds what overlap
# gains (workload 1: 0.125 against 0.140 ms/step; workload 2, 25 K IDs, is
# faster overlapped: 0.14-0.18 against 0.20)
SERIAL_MAX_IDS = 8192


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


@dataclass
class Ctx:
    """One workload's inputs, resident on the GPU."""
    k: int
    w: object
    seed: int
    host_batches: list
    dev_batches: list
    weights: list
    states: list
    grads_host: list
    grads_dev: list
    cap: int
    n_tok: list


def load(k, balancer, seed, nb, layout):
    import torch

    from jagged_embedding_sparse_amd import lib, synth
    w = synth.workload(k, balancer)
    seed = seed if seed is not None else k
    NB = max(2, nb or w.iterations)
    t0 = time.time()
    gen = synth.Batches(w, seed)
    host_batches = [gen.batch(i) for i in range(NB)]
    log(f"workload {k} {w.name} balancer={w.balancer}: {NB} batches in {time.time() - t0:.1f}s; "
        f"IDs/batch {np.mean([b['n_tok'] * len(w.tables) for b in host_batches]):.0f}")
    dev_batches = [dict(uih_len=torch.from_numpy(b["uih_len"]).cuda(),
                        sample_offsets=torch.from_numpy(b["sample_offsets"]).cuda(),
                        ids=torch.from_numpy(b["ids"]).cuda()) for b in host_batches]
    cap = max(b["n_tok"] for b in host_batches)
    weights, states = [], []
    ada = w.optim == "rw_adagrad"
    for t, spec in enumerate(w.tables):
        if layout.startswith("rowstate"):
            tdt = torch.float32 if spec.dtype == "f32" else torch.bfloat16
            wv, st = lib.alloc_table(spec.rows, spec.dim, tdt, ada, device="cuda",
                                     align=256 if layout == "rowstate256" else 16)
            weights.append(synth.init_table(spec.rows, spec.dim, spec.dtype, seed, "cuda",
                                            table=t, out=wv))
            states.append(st.zero_() if st is not None else None)
        else:
            weights.append(synth.init_table(spec.rows, spec.dim, spec.dtype, seed, "cuda",
                                            table=t))
            states.append(torch.zeros(spec.rows, dtype=torch.float32, device="cuda")
                          if ada else None)
    grads_host = [synth.gradient_rows(seed, 0, t, np.arange(cap), spec.dim)
                  for t, spec in enumerate(w.tables)]
    grads_dev = [torch.from_numpy(g).cuda() for g in grads_host]
    return Ctx(k, w, seed, host_batches, dev_batches, weights, states, grads_host, grads_dev,
               cap, [b["n_tok"] for b in host_batches])


def measure(ctx, steps, warmup, args, full):
    """Times `steps` steps after `warmup` untimed ones; with `full`, also the
    per-stage breakdown and the per-step spread from extra steps."""
    import torch

    from jagged_embedding_sparse_amd.hipevent import HipEvent
    from jagged_embedding_sparse_amd.step import SparseStep, StageTimer
    w, NB, n_tok, grads_dev = ctx.w, len(ctx.dev_batches), ctx.n_tok, ctx.grads_dev
    dev_batches = ctx.dev_batches
    asked = args.schedule
    if asked == "auto":  # batches of a few thousand IDs: the launch count sets the pace
        asked = "serial" if ctx.cap * len(w.tables) <= SERIAL_MAX_IDS else "joined"
    L = 1 if (args.sync or asked == "serial") else args.lookahead
    ahead = L >= 2
    sched = asked if (ahead or asked == "serial") else "joined"
    graph = args.graph == "on" and ahead and not args.sync
    step = SparseStep(w, ctx.weights, ctx.states, ctx.cap, lookup=args.lookup,
                      lookahead=L, autotune={} if args.autotune else None, schedule=sched,
                      graph=graph)
    step.prologue(dev_batches[0],
                  batch_after=[dev_batches[j % NB] for j in range(1, L)] if ahead else None)
    if graph:
        # the distinct steps repeat after lcm(batches, state slots, index
        # streams) steps: capture them all now, outside every timed step
        period = int(np.lcm.reduce([NB, L + 1, len(step.s_idx)]))
        t0 = time.perf_counter()
        n_graphs = step.record_graphs([
            (dev_batches[j % NB], [g[:n_tok[(j - 1) % NB]] for g in grads_dev],
             dev_batches[(j + L - 1) % NB]) for j in range(1, period + 1)])
        log(f"captured {n_graphs} step graphs in {time.perf_counter() - t0:.2f}s")
    if args.sync:
        def run_step(batch_next, grads, k_next):
            return step.step_sync(batch_next, grads)
    else:
        def run_step(batch_next, grads, k_next):
            # with lookahead L >= 2 the step also indexes batch k_next + L - 1
            return step.step(batch_next, grads,
                             batch_after=dev_batches[(k_next + L - 1) % NB] if ahead else None)
    k = 0
    for _ in range(warmup):
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
    n_brk = min(steps, 10) if full else 0
    streams = [s for s in step.s_idx + [step.sB, step.sC] if s is not None]
    warm = StageTimer(capacity=24 * (steps + n_brk), streams=streams)
    del warm
    upd_names = ("update_all", "update_co", "update_ex")
    timer = StageTimer(capacity=4 * steps, streams=streams, only=upd_names)
    step.timer = timer
    ev0, ev1 = HipEvent(enable_timing=True), HipEvent(enable_timing=True)
    pairs = []
    ids_timed = 0
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    # both events on the caller's stream: the steps' streams wait for it at
    # the start of each step, and it waits for all of them at the end
    ev0.record()
    for _ in range(steps):
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
    if graph:
        # graphs carry no timing events: the update's launch time from extra
        # steps issued without graphs (the same kernels on the same buffers)
        n_upd = min(steps, 10)
        step.set_graph(False)
        timer = StageTimer(capacity=4 * n_upd, streams=streams, only=upd_names)
        step.timer = timer
        for _ in range(n_upd):
            p = k % NB
            k += 1
            run_step(dev_batches[k % NB], [g[:n_tok[p]] for g in grads_dev], k)
        step.join()
        torch.cuda.synchronize()
        step.timer = None
        step.set_graph(True)
    if args.sync:
        schedule = "sync"
    elif sched == "serial":
        schedule = "serial (every stage on the caller's stream)"
    elif ahead:
        far = {2: "index two ahead", 3: "index three ahead on two index streams"}[L]
        schedule = (f"{far}, prioritized (collision rows first)" if sched == "prioritized"
                    else f"{far}, joined lookup")
    else:
        schedule = "joined" if step.joined else "split"
    if graph:
        schedule += ", one HIP graph per step"
    ms_total = ev0.elapsed_time(ev1)
    ms_step = ms_total / steps
    upd_ms = timer.ms()
    log(f"timed {steps} steps: {ms_total:.3f} ms (wall {wall * 1e3:.3f} ms, host "
        f"submission {submit * 1e3:.3f} ms)")

    stage_ms, per_step = {}, None
    if full:
        # ------------------------------------------------------------ stage breakdown
        brk = StageTimer(capacity=8 * n_brk, streams=streams)
        step.timer = brk
        if graph:
            step.set_graph(False)  # per-stage events: steps issued without graphs
        for _ in range(n_brk):
            p = k % NB
            k += 1
            run_step(dev_batches[k % NB], [g[:n_tok[p]] for g in grads_dev], k)
        step.join()
        torch.cuda.synchronize()
        step.timer = None
        if graph:
            step.set_graph(True)
        stage_ms = brk.ms()

        # ------------------------------------------------------------ per-step spread
        # K more steps with one event per step on the stream that ends each
        # step (kept out of the timed region: each record costs the GPU a few
        # microseconds): with the index stages two ahead the caller's stream,
        # whose lookup waits for the index stream; otherwise stream A, whose
        # last lookup waits for the update (and with --sync runs everything).
        end_stream = torch.cuda.current_stream() if (ahead or sched == "serial") else step.sA
        evs = [HipEvent(enable_timing=True) for _ in range(steps + 1)]
        for e in evs:  # first records take fresh runtime resources: not in the loop
            e.record(end_stream)
        torch.cuda.synchronize()
        evs[0].record(end_stream)
        for j in range(steps):
            p = k % NB
            k += 1
            run_step(dev_batches[k % NB], [g[:n_tok[p]] for g in grads_dev], k)
            evs[j + 1].record(end_stream)
        step.join()
        torch.cuda.synchronize()
        per_step = np.array([evs[j].elapsed_time(evs[j + 1]) for j in range(steps)])

    # ---------------------------------------------------------------- accounting
    # Units per batch pair (p -> p+1) depend only on the IDs, so one more cycle
    # of steps, synchronised, gives them for every pair the timed steps used.
    units = {}
    T, W = len(w.tables), w.world
    for _ in range(NB):
        p = k % NB
        k += 1
        prev = step.cur
        nxt = run_step(dev_batches[k % NB], [g[:n_tok[p]] for g in grads_dev], k)
        step.join()
        torch.cuda.synchronize()

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
                        n_new=n_tok[k % NB] * T, U_new=U,
                        counts=nxt.uq["counts"].cpu().numpy().tolist())
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
    # the roofline's kernel: the update launch (the dominant stage on every
    # workload), timed inside the timed region; with the prioritized schedule
    # the larger of its two class launches
    upd_avg = {s: float(np.mean(v)) for s, v in upd_ms.items()}
    dom = max(upd_avg, key=lambda s: upd_avg[s])
    dom_bytes_per_launch = stage_bytes[dom] / len(pairs)
    dom_gbps = dom_bytes_per_launch / (upd_avg[dom] * 1e-3) / 1e9
    step_gbps = step_bytes / (ms_total * 1e-3) / 1e9
    res = dict(step=step, schedule=schedule, ms_step=ms_step, value=ids_timed / (ms_total * 1e-3),
               ids_per_step=ids_timed / steps, dom=dom, dom_gbps=dom_gbps,
               dom_bytes=dom_bytes_per_launch, dom_ms=upd_avg[dom], upd_avg=upd_avg,
               step_bytes=step_bytes / steps, step_gbps=step_gbps,
               stage_avg={k2: float(np.mean(v)) for k2, v in stage_ms.items()},
               per_step=per_step, units=units, pairs=pairs, n_brk=n_brk)
    return res


# the update's kernels: short, medium and long rows and the long rows' fix-up
# (k_*_set when several tables share a launch)
KERNEL_OF = {
    "update_co": "k_short+k_medium+k_long+k_fix (fs_grad_reduce_update, collision rows)",
    "update_ex": "k_short+k_medium+k_long+k_fix (fs_grad_reduce_update, exclusive rows)",
    "update_all": "k_short+k_medium+k_long+k_fix (fs_grad_reduce_update, all rows)"}


def eq1_sparsity(L):
    """The pages' Equation 1: share of padded items when every sample of the
    batch is padded to the batch's longest UIH."""
    L = np.asarray(L, np.float64)
    return float(1.0 - L.sum() / (L.max() * len(L))) if len(L) and L.max() > 0 else 0.0


def stats(ctx, res):
    """Per-workload statistics: collision rates, Equation 1 sparsity, per-rank
    load under both balancers, empty VBS ranks, device memory."""
    import torch

    from jagged_embedding_sparse_amd import lib
    w, units = ctx.w, res["units"]
    # collision rate of iteration i+1 against i: by unique rows and by tokens
    by_u = [u["counts"][1] / max(1, u["counts"][0]) for u in units.values()]
    by_tok = [sum(n for n, _ in u["lookup_co"]) / max(1, u["n_new"]) for u in units.values()]
    alpha = w.alpha if w.balancer == "vbs" else (3, 2)
    fbs, vbs = dict(load=[], local=[]), dict(load=[], local=[], empty=[])
    glob = []
    for b, db in zip(ctx.host_batches, ctx.dev_batches):
        L = b["uih_len"]
        tok = np.diff(b["sample_offsets"])
        glob.append(eq1_sparsity(L))
        pf, rf = lib.fs_balance_fbs(db["uih_len"], w.world)
        pv, rv, _ = lib.fs_balance_vbs(db["uih_len"], w.world, alpha)
        for (pm, ro), acc in (((pf, rf), fbs), ((pv, rv), vbs)):
            pm, ro = pm.cpu().numpy(), ro.cpu().numpy()
            loads = np.array([tok[pm[ro[r]:ro[r + 1]]].sum() for r in range(w.world)], np.float64)
            acc["load"].append(float(loads.max() / loads.mean()))
            acc["local"].append(float(np.mean([eq1_sparsity(L[pm[ro[r]:ro[r + 1]]])
                                               for r in range(w.world) if ro[r + 1] > ro[r]])))
            if acc is vbs:
                acc["empty"].append(int(np.sum(np.diff(ro) == 0)))
    table_bytes = sum(x.numel() * x.element_size() for x in ctx.weights)
    state_bytes = sum(x.numel() * x.element_size() for x in ctx.states if x is not None)
    return {
        "collision_rate": {"by_unique_rows": float(np.mean(by_u)),
                           "by_tokens": float(np.mean(by_tok))},
        "eq1_sparsity": {"global_batch": float(np.mean(glob)),
                         "local_batches_fbs": float(np.mean(fbs["local"])),
                         "local_batches_vbs": float(np.mean(vbs["local"]))},
        "rank_token_load_max_over_mean": {"fbs": float(np.mean(fbs["load"])),
                                          "vbs": float(np.mean(vbs["load"]))},
        "vbs_alpha": f"{alpha[0]}/{alpha[1]}",
        "vbs_empty_ranks": float(np.mean(vbs["empty"])),
        "unique_rows_per_step": float(np.mean([u["U_new"] for u in units.values()])),
        "device_bytes": {"tables": int(table_bytes), "state": int(state_bytes),
                         "peak_allocated": int(torch.cuda.max_memory_allocated())},
        "note": "means over the distinct batches; load = tokens per virtual rank"}


def tables_name(w):
    return "+".join(f"{t.rows // 1_000_000}Mx{t.dim}-{t.dtype}" if t.rows >= 1_000_000 else
                    f"{t.rows // 1000}Kx{t.dim}-{t.dtype}" for t in w.tables)


def summary(ctx, res):
    """The per-config entry: throughput, step bandwidth, update roofline, stats."""
    return {
        "workload": f"workload {ctx.k}: {ctx.w.name} ({ctx.w.balancer.upper()})",
        "ids_per_s": res["value"], "ms_per_step": res["ms_step"],
        "ids_per_step": res["ids_per_step"], "schedule": res["schedule"],
        "step_hbm": {"algorithmic_bytes_per_step": res["step_bytes"], "GBps": res["step_gbps"],
                     "frac": res["step_gbps"] / HBM_PEAK_GBPS},
        "update_roofline": {"kernel": KERNEL_OF[res["dom"]], "achieved": res["dom_gbps"],
                            "frac": res["dom_gbps"] / HBM_PEAK_GBPS,
                            "ms_per_launch": res["dom_ms"],
                            "bytes_per_launch": res["dom_bytes"]},
        "stats": stats(ctx, res)}


def release():
    """Returns the memory of dropped tensors to the device (after the caller
    has dropped its references) and restarts the peak-memory count."""
    import torch
    gc.collect()
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    torch.cuda.reset_peak_memory_stats()


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the multi-GPU "
              "sharding of this path is described, not built.", file=sys.stderr)
        sys.exit(2)
    import torch

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    from jagged_embedding_sparse_amd import synth
    w = synth.workload(args.config, args.balancer)
    nb = args.batches or min(w.iterations, args.warmup + args.steps + 1)
    ctx = load(args.config, args.balancer, args.seed, nb, args.layout)
    if args.entry:
        entry = summary(ctx, measure(ctx, args.steps, args.warmup, args, full=False))
        log(f"{entry['workload']}: {entry['ms_per_step']:.3f} ms/step, "
            f"{entry['ids_per_s']:.3e} IDs/s, step {entry['step_hbm']['frac'] * 100:.1f}% "
            f"of peak, update {entry['update_roofline']['frac'] * 100:.1f}%")
        print(json.dumps(entry))
        return
    res = measure(ctx, args.steps, args.warmup, args, full=True)
    head_stats = stats(ctx, res) if not args.no_per_config else None

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(ctx)

    # HBM bytes per launch of the dominant stage from the committed counter
    # summary (rocprofv3 FETCH_SIZE / WRITE_SIZE, copy-calibrated), when it was
    # taken on the kernel sources built here and on the same (dense) tables
    from jagged_embedding_sparse_amd.traffic import load_traffic
    traffic = load_traffic(args.config, res["dom"]) if args.layout == "dense" else None

    per_config = None
    if not args.no_per_config:
        # each other workload in a process of its own, as the headline runs:
        # a workload measured after another one's tables were released in the
        # same process ran up to 45% slower (workload 4: 0.73 against 0.50 ms)
        res.pop("step", None)
        ctx = None
        release()
        per_config = []
        for k, bal in PER_CONFIG:
            wk = synth.workload(k, bal)
            if k == args.config and wk.balancer == w.balancer:
                continue
            cmd = [sys.executable, os.path.abspath(__file__), "--entry", "--config", str(k),
                   "--balancer", wk.balancer, "--steps", str(args.per_config_steps),
                   "--warmup", str(args.warmup), "--schedule", args.schedule,
                   "--lookup", args.lookup, "--lookahead", str(args.lookahead)]
            r = subprocess.run(cmd, stdout=subprocess.PIPE, text=True, timeout=300)
            if r.returncode != 0:
                raise RuntimeError(f"per-config run of workload {k} failed ({r.returncode})")
            per_config.append(json.loads(r.stdout.strip().splitlines()[-1]))

    out = {
        "metric": METRIC,
        "value": res["value"],
        "unit": "IDs/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": res["ms_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": f"workload {args.config}: {w.name} ({w.balancer.upper()})",
            "global_batch": w.batch, "virtual_ranks": w.world, "tables": tables_name(w),
            "optimizer": w.optim, "ids_per_step": res["ids_per_step"],
            "weights": sorted({t.dtype for t in w.tables}), "grad_accumulate": "f64",
            "distinct_batches": nb, "schedule": res["schedule"],
            "autotune": bool(args.autotune), "layout": args.layout},
        "roofline": {
            "bound": "hbm", "achieved": res["dom_gbps"], "peak": HBM_PEAK_GBPS, "unit": "GB/s",
            "frac": res["dom_gbps"] / HBM_PEAK_GBPS, "traffic": traffic,
            "kernel": KERNEL_OF[res["dom"]],
            "bytes_per_launch": res["dom_bytes"],
            "ms_per_launch": res["dom_ms"]},
        "step_hbm": {
            "algorithmic_bytes_per_step": res["step_bytes"], "GBps": res["step_gbps"],
            "frac": res["step_gbps"] / HBM_PEAK_GBPS},
        "stages_ms": res["stage_avg"],
        "stages_note": f"stage breakdown from {res['n_brk']} extra steps with every stage timed",
        "per_step_ms": {"median": float(np.median(res["per_step"])),
                        "min": float(res["per_step"].min()),
                        "max": float(res["per_step"].max()),
                        "note": f"{args.steps} extra steps, one event per step on the stream "
                                "that ends it"},
        "cpu_baseline": cpu,
        "stats": head_stats,
        "per_config": per_config,
    }
    print(json.dumps(out))


def cpu_baseline(ctx, iters=4):
    """The oracle, as it stands, on `iters` consecutive synchronous iterations
    of the same workload (batches 1.., the first split against batch 0), on
    one host core; per-stage seconds from the oracle loop's own timers."""
    import torch

    from oracle import oracle as O
    w, hb = ctx.w, ctx.host_batches
    iters = min(iters, len(hb) - 1)
    stores = []
    for t, spec in enumerate(w.tables):
        rid = np.unique(np.concatenate([b["ids"][t] for b in hb[1:iters + 1]]))
        idx = torch.from_numpy(rid).cuda()
        v = ctx.weights[t].index_select(0, idx)
        vals = (v.view(torch.int16).cpu().numpy().view(np.uint16) if v.dtype == torch.bfloat16
                else v.cpu().numpy())
        st = ctx.states[t].index_select(0, idx).cpu().numpy() if ctx.states[t] is not None \
            else None
        stores.append(O.RowStore(rid, vals, st, bf16=v.dtype == torch.bfloat16))
    run = O.SyncRun(w, stores)
    run.prev_unique = run.index_stages(hb[0])["uniq"]["unique"]  # untimed: context for the split
    run.seconds = {}
    ids = 0
    t0 = time.perf_counter()
    for b in hb[1:iters + 1]:
        n = b["n_tok"]
        g = [x[:n] for x in ctx.grads_host]
        run.step(b, lambda o, g=g: g)
        ids += n * len(w.tables)
    dt = time.perf_counter() - t0
    log(f"oracle: {ids} IDs in {dt:.2f}s")
    return {"value": ids / dt, "unit": "IDs/s", "cores": 1, "kind": "oracle",
            "sample": f"{iters} consecutive synchronous iterations (balance, bucketize, dedup, "
                      f"collision split, lookup, fp64 reduce, update) of batches 1..{iters} of "
                      f"the same workload, {ids} IDs, {dt:.2f} s",
            "stage_seconds": {k: round(v, 3) for k, v in run.seconds.items()},
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
