"""The prioritized sparse step: two HIP streams over the C-ABI calls.

One step consumes the gradients of iteration i and the IDs of iteration i+1
and leaves the embeddings of iteration i+1 in HBM ("FreeScale: distributed
training for sequence recommendation models", section 3.2 and Algorithm 2):

  stream A  balance(i+1) -> bucketize(i+1) -> split(i+1 vs i) --event-->
            update(i, collision rows) -> lookup(i+1, collision rows)
  stream B  (waits for the split) lookup(i+1, exclusive rows) ->
            update(i, exclusive rows)
  join      stream A waits for stream B.

Collision rows are written before they are read; exclusive rows of i+1 are
never written by step i and exclusive rows of i are never read by i+1, so
the two streams touch disjoint rows and the result equals the synchronous
loop (update everything of i, then look up everything of i+1).

Buffers are allocated once at capacity; per-iteration state is double
buffered. Every stream keeps the default priority.
"""

from __future__ import annotations

from dataclasses import dataclass, field

import torch

from . import lib


@dataclass
class IterState:
    """Everything one iteration's index stages produce (device tensors)."""

    n_tok: int = 0
    perm: torch.Tensor = None
    rank_offsets: torch.Tensor = None
    rank_weight: torch.Tensor = None
    bucket: dict = field(default_factory=dict)
    uq: dict = field(default_factory=dict)
    cls_next: torch.Tensor = None  # class of this iteration's rows vs the next one
    out: list = field(default_factory=list)  # lookup output per table


class SparseStep:
    def __init__(self, workload, weights, states, n_tok_cap, device=None):
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
        self.ws_bal = torch.empty(lib.balance_workspace_size(N, W), dtype=torch.uint8, device=d)
        self.ws_bkt = torch.empty(lib.bucketize_workspace_size(cap, N, T, W), dtype=torch.uint8,
                                  device=d)
        self.ws_uq = torch.empty(lib.unique_workspace_size(ncap, T, W), dtype=torch.uint8,
                                 device=d)
        rws = lib.reduce_workspace_size(cap, max(self.dims))
        self.ws_red = [torch.empty(rws, dtype=torch.uint8, device=d) for _ in range(2)]
        self.states_buf = [self._alloc_iter() for _ in range(2)]
        self.sA = torch.cuda.Stream(device=d)
        self.sB = torch.cuda.Stream(device=d)
        self.ev_split = torch.cuda.Event()
        self.ev_b = torch.cuda.Event()
        self.cur = None  # IterState of iteration i (already looked up)
        self.slot = 0

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
        st.out = [torch.empty((self.cap, D), dtype=w.dtype, device=d)
                  for D, w in zip(self.dims, self.weights)]
        return st

    # ------------------------------------------------------------------ stages
    def _index_stages(self, batch, st, prev, stream):
        """balance + bucketize + split of `batch` (device dict) into st."""
        W, T = self.W, self.T
        n_tok = int(batch["ids"].shape[1])
        st.n_tok = n_tok
        if self.w.balancer == "fbs":
            lib.fs_balance_fbs(batch["uih_len"], W, st.perm, st.rank_offsets, err=self.err,
                               stream=stream)
        else:
            lib.fs_balance_vbs(batch["uih_len"], W, self.w.alpha, st.perm, st.rank_offsets,
                               st.rank_weight, err=self.err, ws=self.ws_bal, stream=stream)
        lib.fs_bucketize_permute(batch["ids"], batch["sample_offsets"], self.rows, st.perm,
                                 st.rank_offsets, W, out=st.bucket, err=self.err, ws=self.ws_bkt,
                                 stream=stream)
        out = dict(st.uq)
        if prev is not None:
            out["prev_cls"] = prev.cls_next
        lib.fs_unique_collision_split(
            st.bucket["shard_keys"], st.bucket["shard_bm"], st.bucket["shard_offsets"],
            T * n_tok, self.rows, W,
            prev_unique=prev.uq["unique"] if prev is not None else None,
            prev_counts=prev.uq["counts"] if prev is not None else None,
            prev_cap=T * prev.n_tok if prev is not None else 0, out=out, ws=self.ws_uq,
            stream=stream)

    def _lookup(self, st, which, stream):
        outs = [o[:st.n_tok] for o in st.out]
        lib.fs_jagged_lookup(self.weights, self.W, st.uq, st.n_tok, which=which,
                             cls=st.uq["cls"], out=outs, stream=stream)

    def _update(self, st, grads, which, stream, ws):
        lib.fs_grad_reduce_update(self.weights, self.states, self.W, grads, st.n_tok, st.uq,
                                  self.w.optim, self.w.lr, self.w.eps, which=which,
                                  cls=st.cls_next, ws=ws, stream=stream)

    # ------------------------------------------------------------------ schedule
    def prologue(self, batch):
        """Index stages + full lookup of the first iteration."""
        st = self.states_buf[self.slot]
        self.sA.wait_stream(torch.cuda.current_stream())
        self._index_stages(batch, st, None, self.sA)
        self._lookup(st, lib.FS_ALL, self.sA)
        self.cur = st
        return st

    def step(self, batch_next, grads_cur):
        """Prioritized step: update iteration i, look up iteration i+1."""
        cur = self.cur
        nxt = self.states_buf[1 - self.slot]
        sA, sB = self.sA, self.sB
        self._index_stages(batch_next, nxt, cur, sA)
        self.ev_split.record(sA)
        self._update(cur, grads_cur, lib.FS_COLLISION, sA, self.ws_red[0])
        self._lookup(nxt, lib.FS_COLLISION, sA)
        sB.wait_event(self.ev_split)
        self._lookup(nxt, lib.FS_EXCLUSIVE, sB)
        self._update(cur, grads_cur, lib.FS_EXCLUSIVE, sB, self.ws_red[1])
        self.ev_b.record(sB)
        sA.wait_event(self.ev_b)
        self.cur = nxt
        self.slot = 1 - self.slot
        return nxt

    def step_sync(self, batch_next, grads_cur):
        """Reference schedule on one stream: update all of i, then look up all of i+1."""
        cur = self.cur
        nxt = self.states_buf[1 - self.slot]
        sA = self.sA
        self._index_stages(batch_next, nxt, cur, sA)
        lib.fs_grad_reduce_update(self.weights, self.states, self.W, grads_cur, cur.n_tok,
                                  cur.uq, self.w.optim, self.w.lr, self.w.eps, which=lib.FS_ALL,
                                  ws=self.ws_red[0], stream=sA)
        self._lookup(nxt, lib.FS_ALL, sA)
        self.cur = nxt
        self.slot = 1 - self.slot
        return nxt

    def epilogue(self, grads_last):
        """Update of the last iteration (no lookahead: every row exclusive)."""
        cur = self.cur
        lib.fs_grad_reduce_update(self.weights, self.states, self.W, grads_last, cur.n_tok,
                                  cur.uq, self.w.optim, self.w.lr, self.w.eps, which=lib.FS_ALL,
                                  ws=self.ws_red[0], stream=self.sA)

    def join(self):
        torch.cuda.current_stream().wait_stream(self.sA)
