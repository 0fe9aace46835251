"""The prioritized sparse step: two HIP streams over the C-ABI calls.

One step consumes the gradients of iteration i and the IDs of iteration i+1
and leaves the embeddings of iteration i+1 in HBM ("FreeScale: distributed
training for sequence recommendation models", section 3.2 and Algorithm 2:
collision rows keep a strict write-then-read order, exclusive rows are
fetched ahead of the update):

  stream A  balance(i+1) -> bucketize(i+1) -> split(i+1 vs i) ->
            lookup(i+1, exclusive rows)          [prefetched past the update]
  stream B  update(i, every row of iteration i)  [concurrent with stream A]
  stream A  (waits for B) lookup(i+1, collision rows)

Exclusive rows of i+1 are never written by the update of i, so their lookup
may run before or during it; collision rows are read only after it. The
result equals the synchronous loop (update everything of i, then look up
everything of i+1), which `step_sync` runs on one stream for reference.

On one GPU the update of i does not wait for the index stages of i+1 (that
wait exists across GPUs only because the collision split decides which
gradients travel first), so the latency-bound index kernels overlap the
bandwidth-bound update.

When the update finishes before the index stages do, prefetching the
exclusive rows gains nothing and the split costs a second pass over the
occurrence indices; the lookup then runs once, for all rows, after the
update ("joined"). `lookup="auto"` times its first steps with HIP events and
keeps the split only if the update was still running when the index stages
ended; "split" and "joined" fix the choice. All three give the same result.

The index stages depend on nothing but the IDs (and the previous
iteration's unique rows), so with `lookahead=2` they run one more iteration
ahead, on the prefetched batch after next:

  caller's stream  update(i) -> lookup(i+1, every row)  [index(i+1) done last step]
  stream A         balance(i+2) -> bucketize(i+2) -> split(i+2 vs i+1)

The latency-bound index kernels then overlap both bandwidth-bound stages
instead of only the update. Three iteration states are alive at once (i being
updated, i+1 looked up, i+2 indexed); the result is again the synchronous
loop's.

With `lookahead=3` the index stages run three iterations ahead on two index
streams taken in turn, each with its own workspaces, so that one iteration's
index stages overlap the previous iteration's: the dedup runs as a call of
its own (every row exclusive) and only the collision split after it, which
reads the previous iteration's unique rows, waits for the previous dedup.
Where the index stages are a chain of latency-bound launches longer than the
update and the lookup, a step then costs about one collision split instead
of a whole index chain. Four iteration states are alive at once.

With the index stages ahead (joined lookup) and a batch of at least 2^17
IDs, the update runs as two concurrent parts: its rows of at most 64
occurrences on the caller's stream and its longer rows (chunked sums and
their fix-up) on stream B, joined before the lookup. The parts touch disjoint
rows, so the result is the same; each stream has one launch boundary fewer
and the parts' ramps and tails overlap.

With `schedule="prioritized"` (index stages two ahead) the update is split
by class as Algorithm 2 splits it, so that the next lookup waits only for the
rows it shares with the update:

  caller's stream  update(i, collision rows) -> lookup(i+1, collision rows)
  stream B         update(i, exclusive rows)          [own partial sums]
  stream C         lookup(i+1, exclusive rows)
  stream A         balance(i+2) -> bucketize(i+2) -> split(i+2 vs i+1)

Exclusive rows of i are not rows of i+1 and exclusive rows of i+1 are not
rows of i, so only the collision lookup orders against an update; the result
is again the synchronous loop's. The classes of i against i+1 must exist when
the update starts, which the two-ahead index stages provide.

With `autotune` (VBS only; section 4.1's AutoTune), the balance cuts at
per-rank shares of the weight, and right after each balance the modelled time
of the partition it made moves the shares for the next one -- two small
launches on the index stream, no host synchronisation.

With `graph=True` (index stages two or three ahead) each distinct step --
the state slots it uses and its input tensors -- is captured once as a HIP
graph and replayed after that: the host then submits one graph per step
instead of some 30 launches and their stream waits, which sets the pace of
small batches. A step's graph starts after the previous one has ended, so it
waits for nothing outside itself; inside it the index stages still run beside
the update and the lookup. `record_graphs` captures a known sequence of steps
ahead of time without running them.

Buffers are allocated once at capacity; per-iteration state is double
buffered (triple with lookahead=2), and every C call is marshalled once per
state slot. Every stream keeps the default priority.
"""

from __future__ import annotations

from collections import deque
from dataclasses import dataclass, field

import torch

from . import lib
from .hipevent import HipEvent


_CLS = {lib.FS_ALL: "all", lib.FS_COLLISION: "co", lib.FS_EXCLUSIVE: "ex"}


class _nullspan:
    def __enter__(self):
        return self

    def __exit__(self, *a):
        return False


class StageTimer:
    """HIP event pairs around each C call, on the stream the call runs on.

    Events come from a pool made before timing starts and recorded once on
    the streams that will use them. Records of timing events that need fresh
    runtime resources cost tens of microseconds of host time each, which
    inside the timed loop would let the host, not the GPU, set the pace of
    small steps; the runtime recycles those resources when events are
    dropped, so a larger pool made and dropped first keeps the timed
    records cheap. Each record also costs the GPU a few microseconds between
    kernels, so `only` limits the timed stages where that would distort the
    measurement; the events skip the system-scope fence (HipEvent), whose
    cache write-back would otherwise add to every timed span."""

    def __init__(self, capacity=0, streams=None, only=None):
        self.pairs = {}
        self.pool = []
        self.only = set(only) if only is not None else None  # stage names to time
        ss = list(streams) if streams else [torch.cuda.current_stream()]
        for i in range(capacity):
            a = HipEvent(enable_timing=True)
            b = HipEvent(enable_timing=True)
            a.record(ss[i % len(ss)])
            b.record(ss[i % len(ss)])
            self.pool.append((a, b))
        torch.cuda.synchronize()
        self.pool.reverse()

    def _pair(self):
        if self.pool:
            return self.pool.pop()
        return HipEvent(enable_timing=True), HipEvent(enable_timing=True)

    def span(self, name, stream):
        if self.only is not None and name not in self.only:
            return _nullspan()
        timer = self

        class _Span:
            def __enter__(self):
                self.a, self.b = timer._pair()
                self.a.record(stream)
                return self

            def __exit__(self, *exc):
                self.b.record(stream)
                timer.pairs.setdefault(name, []).append((self.a, self.b))
                return False

        return _Span()

    def ms(self):
        """name -> list of per-call milliseconds (call after synchronising)."""
        return {k: [a.elapsed_time(b) for a, b in v] for k, v in self.pairs.items()}


@dataclass
class IterState:
    """Everything one iteration's index stages produce (device tensors)."""

    n_tok: int = 0
    slot: int = -1  # index among the step's iteration states
    perm: torch.Tensor = None
    rank_offsets: torch.Tensor = None
    rank_weight: torch.Tensor = None
    bucket: dict = field(default_factory=dict)
    uq: dict = field(default_factory=dict)
    cls_next: torch.Tensor = None  # class of this iteration's rows vs the next one
    out: list = field(default_factory=list)  # lookup output per table
    idx_x: int = 0  # index stream that ran this iteration's index stages
    ev_uq: HipEvent = None  # dedup done (unique rows and counts[0] ready)
    ev_done: HipEvent = None  # index stages done (after the collision split)
    ev_bal: HipEvent = None  # balance (and AutoTune's share update) done
    graph: object = None  # the step graph whose capture indexed this iteration (graph mode)


_LOOKUP_MODES = ("split", "joined", "auto")
_SCHEDULES = ("joined", "prioritized", "serial")
# VBS AutoTune: modelled time c2 L^2 + c1 L + c0 per sample (coef), shares
# moved by max(1, share * step) outside a band of +-tol around the mean time,
# every share starting at init
AUTOTUNE_DEFAULTS = dict(coef=(1, 64, 0), step=(1, 16), tol=(1, 50), init=1 << 16)
_CALIB_STEPS = 3  # steps timed by lookup="auto" before it decides
# IDs (token x table) from which the joined schedule runs the update as two
# concurrent parts: below it the update is a few short launches whose split
# costs the host more than it saves
_SPLIT_MIN = 1 << 17


class SparseStep:
    def __init__(self, workload, weights, states, n_tok_cap, device=None, lookup="auto",
                 lookahead=1, autotune=None, schedule="joined", graph=False,
                 split_update="auto"):
        if lookup not in _LOOKUP_MODES:
            raise ValueError(f"lookup must be one of {_LOOKUP_MODES}, not {lookup!r}")
        if lookahead not in (1, 2, 3):
            raise ValueError(f"lookahead must be 1, 2 or 3, not {lookahead!r}")
        if schedule not in _SCHEDULES:
            raise ValueError(f"schedule must be one of {_SCHEDULES}, not {schedule!r}")
        if schedule == "prioritized" and lookahead < 2:
            raise ValueError("the prioritized schedule needs the index stages at least two "
                             "ahead (lookahead=2 or 3): the update of i starts from the classes "
                             "of i against i+1")
        if schedule == "serial" and (lookahead != 1 or graph):
            raise ValueError("the serial schedule runs every stage on the caller's stream, one "
                             "iteration at a time (lookahead=1, no graph)")
        if split_update not in ("auto", True, False):
            raise ValueError(f"split_update must be 'auto', True or False, not {split_update!r}")
        if graph and lookahead < 2:
            raise ValueError("graph replay needs the index stages ahead (lookahead=2 or 3): "
                             "a step's graph then holds no wait on work of the step before")
        self.schedule = schedule
        if autotune is not None and workload.balancer != "vbs":
            raise ValueError("autotune needs the VBS balancer")
        self.w = workload
        self.W = workload.world
        self.T = len(weights)
        self.weights = weights
        self.states = states
        self.rows = [int(x.shape[0]) for x in weights]
        self.dims = [int(x.shape[1]) for x in weights]
        self.cap = int(n_tok_cap)
        self.dev = device or weights[0].device
        d, W, T, cap = self.dev, self.W, self.T, self.cap
        N = workload.batch
        ncap = T * cap
        self.err = torch.zeros(1, dtype=torch.int32, device=d)
        # one balance and one bucketize workspace per index stream
        n_idx = 2 if lookahead == 3 else 1
        self.ws_bal = [torch.empty(lib.balance_workspace_size(N, W), dtype=torch.uint8, device=d)
                       for _ in range(n_idx)]
        self.ws_bkt = [torch.empty(lib.bucketize_workspace_size(cap, N, T, W), dtype=torch.uint8,
                                   device=d) for _ in range(n_idx)]
        # dedup and collision split per index stream: consecutive dedups run
        # side by side, only the collision splits wait for the previous dedup
        self.ws_uq = [torch.empty(lib.unique_workspace_size(ncap, T, W), dtype=torch.uint8,
                                  device=d) for _ in range(n_idx)]
        self.ws_co = [torch.empty(lib.collision_workspace_size(ncap, T, W), dtype=torch.uint8,
                                  device=d) for _ in range(n_idx)]
        rws = lib.reduce_workspace_size(cap, max(self.dims), T)
        self.ws_red = [torch.empty(rws, dtype=torch.uint8, device=d) for _ in range(2)]
        self.lookahead = lookahead
        self.states_buf = [self._alloc_iter() for _ in range(lookahead + 1)]
        for i, st in enumerate(self.states_buf):
            st.slot = i
        self._calls = {}  # prepared C calls by (stage, slots, ...)
        self.sA = torch.cuda.Stream(device=d)
        self.s_idx = [self.sA] + [torch.cuda.Stream(device=d) for _ in range(n_idx - 1)]
        self.sB = torch.cuda.Stream(device=d)
        # exclusive-row lookup of the prioritized schedule
        self.sC = torch.cuda.Stream(device=d) if schedule == "prioritized" else None
        self.ev_b = HipEvent()
        self._ahead = deque()  # iterations after i already indexed, oldest first
        self._n_indexed = 0  # iterations whose index stages were issued
        self.cur = None  # IterState of iteration i (already looked up)
        self.slot = 0
        self.timer = None  # optional StageTimer
        self.lookup = lookup
        # current choice (lookahead >= 2 always looks every row up after the update)
        self.joined = lookup == "joined" or lookahead >= 2
        self._calib = []  # (start, update end, index end) event triples
        self._calib_left = _CALIB_STEPS if (lookup == "auto" and lookahead == 1) else 0
        # VBS AutoTune: per-rank shares of the weight, moved after every
        # balance by the modelled time of the partition just made
        self.autotune = None
        if autotune is not None:
            self.autotune = {**AUTOTUNE_DEFAULTS, **autotune}
            self.shares = torch.full((W,), int(self.autotune["init"]), dtype=torch.int64,
                                     device=d)
            self.rank_cost = torch.empty(W, dtype=torch.int64, device=d)
        # graph mode: one HIP graph per distinct step (state slots, inputs)
        self.graph = graph
        self._graphs = {}
        self._capture = None  # the graph being captured or replayed
        self._dry = False  # replaying a captured step: Python state only
        self._record_only = False  # capturing without replaying
        self._forked = []  # streams forked from the capture stream
        self._cap_stream = torch.cuda.Stream(device=d) if graph else None
        # the joined schedule's update as two concurrent parts (rows of at
        # most 64 occurrences on the caller's stream, longer rows on stream B)
        self.split_update = split_update
        self._ev_fork, self._ev_join = HipEvent(), HipEvent()
        # one reused fork event per index stream (a new event per wait costs
        # the host more)
        self._ev_idx = [HipEvent() for _ in self.s_idx]
        self._cs_ev = None  # the event last recorded on the caller's stream this step

    def _t(self, name, stream):
        """Context that brackets one C call with HIP events on its stream."""
        if self.timer is None or self._capture is not None:
            return _nullspan()
        return self.timer.span(name, stream)

    # ------------------------------------------------------------------ issue
    # Every GPU operation of a step goes through these, so that a step whose
    # graph was captured before can replay it after running only the state
    # bookkeeping. Inside a captured step, waits on events of an earlier step
    # are left out: a step's graph starts after the previous one has ended.
    def _call(self, fn, **kw):
        if not self._dry:
            fn(**kw)

    def _fork(self, s, cs, ev=None, recorded=False):
        """Stream s waits for everything enqueued on cs so far (through event
        ev when given: a reused event costs the host less than a new one;
        `recorded`: ev was recorded on cs with nothing enqueued there since,
        so s waits for it without a new record)."""
        if self._capture is not None and s not in self._forked:
            self._forked.append(s)
        if self._dry:
            return
        if ev is None:
            s.wait_stream(cs)
        else:
            if not recorded:
                ev.record(cs)
            s.wait_event(ev)

    def _join(self, cs, s, ev=None):
        if self._dry:
            return
        if ev is None:
            cs.wait_stream(s)
        else:
            ev.record(s)
            cs.wait_event(ev)

    def _wait(self, s, ev, st):
        """Stream s waits for event ev of iteration state st; not when ev has
        already completed (outside a capture): then there is nothing to order,
        and the query costs the host less than a wait."""
        if self._dry or (self._capture is not None and st.graph is not self._capture):
            return
        if self._capture is None and ev.query():
            return
        s.wait_event(ev)

    def _record(self, ev, s, st):
        st.graph = self._capture
        if not self._dry and self.schedule != "serial":  # serial: no other stream waits
            ev.record(s)

    def _alloc_iter(self):
        d, W, T, cap = self.dev, self.W, self.T, self.cap
        N = self.w.batch
        ncap = max(T * cap, 1)
        st = IterState()
        st.perm = torch.empty(N, dtype=torch.int32, device=d)
        st.rank_offsets = torch.empty(W + 1, dtype=torch.int32, device=d)
        st.rank_weight = torch.empty(W, dtype=torch.int64, device=d)
        st.bucket = dict(
            bal_offsets=torch.empty(N + 1, dtype=torch.int64, device=d),
            shard_keys=torch.empty(ncap, dtype=torch.int64, device=d),
            shard_bm=torch.empty(ncap, dtype=torch.int32, device=d),
            splits=torch.empty(W * W, dtype=torch.int64, device=d),
            shard_offsets=torch.empty(W + 1, dtype=torch.int64, device=d))
        st.uq = dict(
            unique=torch.empty(ncap, dtype=torch.int64, device=d),
            unique_offsets=torch.empty(T * W + 1, dtype=torch.int64, device=d),
            seg_offsets=torch.empty(ncap + 1, dtype=torch.int32, device=d),
            occ_bm=torch.empty(ncap, dtype=torch.int32, device=d),
            occ_uid=torch.empty(ncap, dtype=torch.int32, device=d),
            cls=torch.empty(ncap, dtype=torch.uint8, device=d),
            counts=torch.empty(4, dtype=torch.int64, device=d))
        st.cls_next = torch.empty(ncap, dtype=torch.uint8, device=d)
        st.ev_uq = HipEvent()
        st.ev_done = HipEvent()
        st.ev_bal = HipEvent()
        st.out = [torch.empty((self.cap, D), dtype=w.dtype, device=d)
                  for D, w in zip(self.dims, self.weights)]
        return st

    # ------------------------------------------------------------------ stages
    # Every call goes through a C call prepared once per state slot (the
    # buffers never move): the generic wrappers' marshalling costs tens of us
    # of host time per call, which on small batches would set the pace.
    def _prep(self, key, make):
        c = self._calls.get(key)
        if c is None:
            c = self._calls[key] = make()
        return c

    def _index_stream(self):
        """(number, stream) of the index stream for the next iteration to index."""
        x = self._n_indexed % len(self.s_idx)
        return x, self.s_idx[x]

    def _index_stages(self, batch, st, prev, stream, x=0):
        """balance + bucketize + dedup + collision split of `batch` (device
        dict) into st, on index stream `x` (`stream`). Each index stream has
        its own workspaces; only the collision split waits for the previous
        iteration's dedup when another stream ran it (it reads that
        iteration's unique rows), and with AutoTune the balance waits for the
        previous share update."""
        W, T = self.W, self.T
        other = prev is not None and prev.idx_x != x
        st.idx_x = x
        self._n_indexed += 1
        ids, so, uih = batch["ids"], batch["sample_offsets"], batch["uih_len"]
        n_tok = int(ids.shape[1])
        st.n_tok = n_tok
        sh = stream.cuda_stream
        at = self.autotune
        if at is None:
            pb = self._prep(("bal", st.slot, x), lambda: lib.prepare_balance(
                self.w.balancer, W, self.w.alpha, st.perm, st.rank_offsets, st.rank_weight,
                self.err, self.ws_bal[x]))
        else:
            pb = self._prep(("bal", st.slot, x), lambda: lib.prepare_balance_shares(
                W, self.w.alpha, self.shares, st.perm, st.rank_offsets, st.rank_weight, self.err,
                self.ws_bal[x]))
            pc = self._prep(("cost", st.slot), lambda: lib.prepare_rank_cost(
                st.perm, st.rank_offsets, at["coef"], self.rank_cost))
            pa = self._prep(("tune",), lambda: lib.prepare_autotune(
                self.rank_cost, self.shares, at["step"], at["tol"], self.err))
        pk = self._prep(("bkt", st.slot, x), lambda: lib.prepare_bucketize(
            self.rows, st.perm, st.rank_offsets, W, st.bucket, self.err, self.ws_bkt[x]))
        pu = self._prep(("uq", st.slot, x), lambda: lib.prepare_unique(
            st.bucket, self.rows, W, st.uq, None, None, self.ws_uq[x]))
        pco = None if prev is None else self._prep(
            ("co", st.slot, prev.slot, x), lambda: lib.prepare_collision(
                st.uq, T, W, prev.uq, prev.cls_next, self.ws_co[x]))
        if at is not None and other:  # the shares the previous balance left
            self._wait(stream, prev.ev_bal, prev)
        with self._t("balance", stream):
            self._call(pb, uih=lib._ptr(uih), n=uih.numel(), stream=sh)
        if at is not None:  # the shares for the next balance
            with self._t("autotune", stream):
                self._call(pc, uih=lib._ptr(uih), n=uih.numel(), stream=sh)
                self._call(pa, stream=sh)
            self._record(st.ev_bal, stream, st)
        with self._t("bucketize", stream):
            self._call(pk, ids=lib._ptr(ids), n_tok=n_tok, so=lib._ptr(so), n=so.numel() - 1,
                       stream=sh)
        # the dedup alone (every row exclusive until the split below)
        with self._t("dedup", stream):
            self._call(pu, n_cap=T * n_tok, prev_cap=0, stream=sh)
        self._record(st.ev_uq, stream, st)
        if pco is not None:
            if other:
                self._wait(stream, prev.ev_uq, prev)
            with self._t("collision", stream):
                self._call(pco, n_cap=T * n_tok, prev_cap=T * prev.n_tok, stream=sh)
        self._record(st.ev_done, stream, st)

    def _lookup(self, st, which, stream):
        pl = self._prep(("lk", st.slot, which), lambda: lib.prepare_lookup(
            self.weights, self.W, st.uq, st.out, which, st.uq["cls"]))
        with self._t(f"lookup_{_CLS[which]}", stream):
            self._call(pl, n_tok=st.n_tok, stream=stream.cuda_stream)

    def _run_update(self, st, grads, which, ws, stream, name=None, aux=None, fork_ev=None):
        """The update of st's rows of class `which` on `stream`; with an `aux`
        stream and a batch of at least _SPLIT_MIN IDs (or split_update=True),
        its rows of more than 64 occurrences run on aux beside the rest (the
        two parts touch disjoint rows; only the long rows use the workspace),
        so that each stream has one launch boundary fewer and the parts' ramps
        and tails overlap. `fork_ev`: an event last recorded on `stream` with
        nothing enqueued there since, which aux may wait for instead of a new
        record (each record costs the host and the stream a few us). When the
        update is timed, aux waits for the span's start event instead, so that
        no part of the update starts before the measured span."""
        pu = self._prep(("upd", st.slot, which, id(ws)), lambda: lib.prepare_update(
            self.weights, self.states, self.W, st.uq, self.w.optim, self.w.lr, self.w.eps, which,
            st.cls_next, ws))
        g = pu.arrays["grads"]
        for t, x in enumerate(grads):
            g[t] = lib._ptr(x)
        split = aux is not None and (self.split_update is True or (
            self.split_update == "auto" and st.n_tok * self.T >= _SPLIT_MIN))
        with self._t(name or f"update_{_CLS[which]}", stream) as span:
            if not split:
                self._call(pu, n_tok=st.n_tok, rows=lib.FS_ROWS_ALL, stream=stream.cuda_stream)
                return
            ev = getattr(span, "a", None) or fork_ev
            if ev is not None:
                self._fork(aux, stream, ev, recorded=True)
            else:
                self._fork(aux, stream, self._ev_fork)
            self._call(pu, n_tok=st.n_tok, rows=lib.FS_ROWS_MANY, stream=aux.cuda_stream)
            self._call(pu, n_tok=st.n_tok, rows=lib.FS_ROWS_FEW, stream=stream.cuda_stream)
            self._join(stream, aux, self._ev_join)

    # ------------------------------------------------------------------ schedule
    def _nslots(self):
        return len(self.states_buf)

    def prologue(self, batch, batch_after=None):
        """Index stages + full lookup of the first iteration; with lookahead
        >= 2, also the index stages of the next lookahead - 1 batches
        (`batch_after`: one batch, or a list of them)."""
        st = self.states_buf[self.slot]
        cs = torch.cuda.current_stream()
        for s_ in self.s_idx:
            s_.wait_stream(cs)
        x, s0 = self._index_stream()
        if self.schedule == "serial":
            s0 = cs
        self._index_stages(batch, st, None, s0, x)
        self._lookup(st, lib.FS_ALL, s0)
        self.cur = st
        self._ahead.clear()
        if self.lookahead >= 2 and batch_after is not None:
            ahead = batch_after if isinstance(batch_after, (list, tuple)) else [batch_after]
            prev = st
            for k, b in enumerate(ahead[:self.lookahead - 1]):
                nxt = self.states_buf[(self.slot + 1 + k) % self._nslots()]
                x, s_ = self._index_stream()
                self._index_stages(b, nxt, prev, s_, x)
                self._ahead.append(nxt)
                prev = nxt
        if self.graph:  # the first step's graph starts after all of it
            for s_ in self.s_idx:
                cs.wait_stream(s_)
        return st

    def _decide(self):
        """lookup="auto": once the calibration steps have run on the GPU, join
        the lookups if the update ended before the index stages in most of
        them. Checks events without waiting for them."""
        if self._calib_left > 0 or not self._calib:
            return
        if not all(e.query() for trip in self._calib for e in trip):
            return
        ahead = [e0.elapsed_time(ei) - e0.elapsed_time(eu) for e0, eu, ei in self._calib]
        self.joined = sum(a > 0 for a in ahead) * 2 > len(ahead)
        self._calib = []

    def step(self, batch_next, grads_cur, batch_after=None):
        """Prioritized step: update iteration i, look up iteration i+1 (and,
        with lookahead L >= 2, index `batch_after`, iteration i+L)."""
        if self.graph:
            return self._step_graph(batch_next, grads_cur, batch_after)
        if self.schedule == "serial":
            return self._step_serial(batch_next, grads_cur)
        if self.schedule == "prioritized":
            return self._step_prioritized(batch_next, grads_cur, batch_after)
        if self.lookahead >= 2:
            return self._step_ahead(batch_next, grads_cur, batch_after)
        self._decide()
        cur = self.cur
        nxt = self.states_buf[1 - self.slot]
        sA, sB = self.sA, self.sB
        sA.wait_stream(torch.cuda.current_stream())  # inputs made on the caller's stream
        calib = None
        if self._calib_left > 0:
            calib = [HipEvent(enable_timing=True) for _ in range(3)]
            calib[0].record(sA)
        # B may start once A has finished the previous step (iteration i's
        # index outputs and lookups; the slot A is about to overwrite is free)
        sB.wait_stream(sA)
        self._run_update(cur, grads_cur, lib.FS_ALL, self.ws_red[1], sB)
        self.ev_b.record(sB)
        if calib:
            calib[1].record(sB)
        self._index_stages(batch_next, nxt, cur, sA)
        if calib:
            calib[2].record(sA)
            self._calib.append(tuple(calib))
            self._calib_left -= 1
        if self.joined:
            sA.wait_event(self.ev_b)
            self._lookup(nxt, lib.FS_ALL, sA)
        else:
            self._lookup(nxt, lib.FS_EXCLUSIVE, sA)
            sA.wait_event(self.ev_b)
            self._lookup(nxt, lib.FS_COLLISION, sA)
        self.cur = nxt
        self.slot = 1 - self.slot
        return nxt

    def _next_states(self, batch_next, batch_after, cs):
        """Index stream waits at the start of a step, and iteration i+1's
        state (indexed now if it was not indexed ahead). Returns (nxt, the
        index stream number and stream for batch_after or None); leaves in
        _cs_ev the event last recorded on cs (None if none was)."""
        cur = self.cur
        n = self._nslots()
        self._cs_ev = None
        # the index streams about to work wait for everything enqueued so far
        # on the caller's stream: the batches, and the update of i-1 and the
        # lookups whose state slots the new index stages overwrite; enqueued
        # before this step's update, so they overlap it
        aft_s = None
        if not self._ahead:  # iteration i+1 was not indexed ahead: index it now
            nxt = self.states_buf[(self.slot + 1) % n]
            x, s_ = self._index_stream()
            self._fork(s_, cs, self._ev_idx[x])
            self._cs_ev = self._ev_idx[x]
            self._index_stages(batch_next, nxt, cur, s_, x)
        else:
            nxt = self._ahead.popleft()
        if batch_after is not None:
            x, s_ = self._index_stream()
            self._fork(s_, cs, self._ev_idx[x])
            self._cs_ev = self._ev_idx[x]
            aft_s = (x, s_)
        return nxt, aft_s

    def _index_after(self, batch_after, nxt, aft_s):
        if batch_after is None:
            return
        x, s_ = aft_s
        prev = self._ahead[-1] if self._ahead else nxt
        aft = self.states_buf[(self.slot + self.lookahead) % self._nslots()]
        self._index_stages(batch_after, aft, prev, s_, x)
        self._ahead.append(aft)

    def _step_ahead(self, batch_next, grads_cur, batch_after):
        # The update and the lookup run on the caller's stream (its inputs are
        # there, and so are the lookup results it reads next); the index
        # streams run the index stages. Each stream wait costs the host ~15 us.
        cur = self.cur
        cs = torch.cuda.current_stream()
        nxt, aft_s = self._next_states(batch_next, batch_after, cs)
        # the update of i needs nothing from the index stages of i+1 (they
        # only read iteration i's unique rows), so only the lookup waits
        self._run_update(cur, grads_cur, lib.FS_ALL, self.ws_red[1], cs, aux=self.sB,
                         fork_ev=self._cs_ev)
        self._wait(cs, nxt.ev_done, nxt)
        self._lookup(nxt, lib.FS_ALL, cs)
        self._index_after(batch_after, nxt, aft_s)
        self.cur = nxt
        self.slot = (self.slot + 1) % self._nslots()
        return nxt

    def _step_prioritized(self, batch_next, grads_cur, batch_after):
        # Algorithm 2's order on one GPU: the collision rows of i are updated
        # first and their lookup for i+1 follows on the caller's stream; the
        # exclusive rows of both iterations go beside it on streams B and C.
        cur = self.cur
        sB, sC = self.sB, self.sC
        cs = torch.cuda.current_stream()
        nxt, aft_s = self._next_states(batch_next, batch_after, cs)
        # streams B and C after the work on the caller's stream: the
        # gradients, and the previous step (joined into it), whose buffers
        # this one reuses
        self._fork(sB, cs)
        self._fork(sC, cs)
        # the classes of i against i+1 (the update's) and of i+1 (the lookups')
        for s_ in (cs, sB, sC):
            self._wait(s_, nxt.ev_done, nxt)
        self._run_update(cur, grads_cur, lib.FS_COLLISION, self.ws_red[1], cs)
        self._lookup(nxt, lib.FS_COLLISION, cs)
        self._run_update(cur, grads_cur, lib.FS_EXCLUSIVE, self.ws_red[0], sB)
        self._lookup(nxt, lib.FS_EXCLUSIVE, sC)
        self._index_after(batch_after, nxt, aft_s)
        self._join(cs, sB)
        self._join(cs, sC)
        self.cur = nxt
        self.slot = (self.slot + 1) % self._nslots()
        return nxt

    # ------------------------------------------------------------------ graph mode
    # A step is a fixed set of launches on fixed buffers, chosen by the state
    # slots in use and the input tensors: each distinct step is captured once
    # as a HIP graph (every stream it uses forked from the capture stream and
    # joined back) and replayed after that, so the host submits one graph
    # instead of some 30 launches and their stream waits. Graphs of
    # consecutive steps run one after the other; the index stages still run
    # ahead, beside the update and the lookup of the same step.
    def _graph_key(self, batch_next, grads_cur, batch_after):
        def bk(b):
            if b is None:
                return None
            return (b["ids"].data_ptr(), tuple(b["ids"].shape), b["sample_offsets"].data_ptr(),
                    b["uih_len"].data_ptr(), b["uih_len"].numel())
        # the launches depend on the token counts of the iterations alive
        # (updated, indexed ahead) and on the shapes of the new batches; the
        # slot about to be overwritten holds nothing they read
        return (self.slot, tuple(st.slot for st in self._ahead),
                self._n_indexed % len(self.s_idx),
                None if self._ahead else bk(batch_next), bk(batch_after),
                tuple((g.data_ptr(), tuple(g.shape)) for g in grads_cur),
                self.cur.n_tok, tuple(st.n_tok for st in self._ahead))

    def _step_graph(self, batch_next, grads_cur, batch_after):
        key = self._graph_key(batch_next, grads_cur, batch_after)
        body = self._step_prioritized if self.schedule == "prioritized" else self._step_ahead
        g = self._graphs.get(key)
        if g is None:
            g = torch.cuda.CUDAGraph()
            self._capture, self._forked = g, []
            try:
                with torch.cuda.graph(g, stream=self._cap_stream):
                    cs = torch.cuda.current_stream()
                    nxt = body(batch_next, grads_cur, batch_after)
                    for s_ in self._forked:
                        cs.wait_stream(s_)
            finally:
                self._capture, self._forked = None, []
            self._graphs[key] = g
        else:
            self._capture, self._dry = g, True
            try:
                nxt = body(batch_next, grads_cur, batch_after)
            finally:
                self._capture, self._dry = None, False
        if not self._record_only:
            g.replay()
        return nxt

    def set_graph(self, on):
        """Switches graph mode on or off between steps (captured graphs are
        kept). Switching on first makes the caller's stream wait for all work
        issued without graphs, which a step's graph does not wait for."""
        if on and self.lookahead < 2:
            raise ValueError("graph replay needs lookahead=2 or 3")
        if on and not self.graph:
            if self._cap_stream is None:
                self._cap_stream = torch.cuda.Stream(device=self.dev)
            cs = torch.cuda.current_stream()
            for s_ in self.s_idx + [self.sB] + ([self.sC] if self.sC is not None else []):
                cs.wait_stream(s_)
        self.graph = bool(on)

    def record_graphs(self, calls):
        """Graph mode: captures the graphs of a sequence of step() calls
        (argument tuples, in the order they will be made) without running
        them, and leaves the step's state as it was, so that later calls
        only replay."""
        if not self.graph:
            raise RuntimeError("record_graphs needs graph=True")
        snap = (self.slot, self.cur, list(self._ahead), self._n_indexed,
                [(st.idx_x, st.n_tok, st.graph) for st in self.states_buf])
        self._record_only = True
        try:
            for a in calls:
                self.step(*a)
        finally:
            self._record_only = False
            self.slot, self.cur, ahead, self._n_indexed, per = snap
            self._ahead = deque(ahead)
            for st, (x, n, g) in zip(self.states_buf, per):
                st.idx_x, st.n_tok, st.graph = x, n, g
        return len(self._graphs)

    def _step_serial(self, batch_next, grads_cur):
        # every stage on the caller's stream in the loop's order: no events
        # and no stream waits, whose host cost sets the pace of small batches
        cur = self.cur
        nxt = self.states_buf[(self.slot + 1) % self._nslots()]
        cs = torch.cuda.current_stream()
        self._index_stages(batch_next, nxt, cur, cs, 0)
        self._run_update(cur, grads_cur, lib.FS_ALL, self.ws_red[0], cs)
        self._lookup(nxt, lib.FS_ALL, cs)
        self.cur = nxt
        self.slot = (self.slot + 1) % self._nslots()
        return nxt

    def step_sync(self, batch_next, grads_cur):
        """Reference schedule on one stream: update all of i, then look up all of i+1."""
        if self._ahead:
            raise RuntimeError("step_sync after a step that indexed its batch_after")
        cur = self.cur
        nxt = self.states_buf[(self.slot + 1) % self._nslots()]
        sA = self.sA
        sA.wait_stream(torch.cuda.current_stream())
        sA.wait_stream(self.sB)
        self._index_stages(batch_next, nxt, cur, sA, 0)
        self._run_update(cur, grads_cur, lib.FS_ALL, self.ws_red[0], sA)
        self._lookup(nxt, lib.FS_ALL, sA)
        self.cur = nxt
        self.slot = (self.slot + 1) % self._nslots()
        return nxt

    def epilogue(self, grads_last):
        """Update of the last iteration (no lookahead: every row exclusive)."""
        cur = self.cur
        if self.schedule == "serial":
            self._run_update(cur, grads_last, lib.FS_ALL, self.ws_red[0],
                             torch.cuda.current_stream())
            return
        self.sA.wait_stream(torch.cuda.current_stream())
        self.sA.wait_stream(self.sB)
        self._run_update(cur, grads_last, lib.FS_ALL, self.ws_red[0], self.sA)

    def join(self):
        cs = torch.cuda.current_stream()
        for s_ in self.s_idx + [self.sB] + ([self.sC] if self.sC is not None else []):
            cs.wait_stream(s_)
