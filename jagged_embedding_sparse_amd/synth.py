"""Seeded synthetic inputs for the jagged sparse step.

This module is the one piece shared by the HIP path and the CPU oracle. It
holds only input generation (lengths, candidate counts, embedding IDs,
gradients, initial tables) and none of the method's arithmetic: no balancing,
no sharding, no dedup, no reduction, no optimizer.

The production workloads of the FreeScale paper (section 5, "Evaluation", and
section 5.2, "Exposed Embedding Communications") are not public. The five
workloads below are their synthetic stand-ins: skewed user-interaction-history
(UIH) lengths, a handful of candidates per sample, Zipf-distributed IDs over
row-wise sharded tables, with the sizes listed in ``WORKLOADS``.

Recipe (all draws from numpy PCG64 generators seeded by ``[seed, iteration,
stream]``):

* UIH lengths: the workload's distribution, then ``ceil``, then capped, with a
  minimum of 1. Pareto(shape, scale) is the classical one, ``scale * U**(-1/shape)``.
* candidates: uniform integers ``1..k`` (0 when the workload has none). A
  sample has ``L_uih + N_can`` tokens, UIH tokens first, and every token holds
  one ID per table.
* IDs: bounded Zipf over ranks ``1..R`` with exponent ``s`` (exact CDF for the
  first 2**20 ranks, a continuous power-law tail beyond), mapped to rows by a
  seeded permutation of ``[0, R)`` so hot rows spread over all shards.
* locality (optional): token ``j >= 1`` of a sample copies, with probability
  ``p``, the ID of a uniformly chosen earlier token of the same sample and table.
* drift (optional): before each iteration after the first, ``ceil(f * R)``
  ranks picked at random swap their row assignments among themselves.
* gradients: a counter-based hash (splitmix64's finaliser) of
  ``(seed, iteration, table, token, column)``, mapped to a multiple of 2**-23
  in [-1, 1); such values add exactly in float64.
* tables: ``N(0, 0.01**2)`` from torch's seeded generator on the target device,
  rounded to the table dtype.
"""

from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np

# ----------------------------------------------------------------------------
# workloads


@dataclass(frozen=True)
class TableSpec:
    rows: int
    dim: int
    dtype: str  # "f32" or "bf16"
    zipf_s: float


@dataclass(frozen=True)
class Workload:
    name: str
    batch: int  # global batch N
    world: int  # virtual ranks / shards W
    tables: tuple
    optim: str  # "sgd" or "rw_adagrad"
    lr: float
    eps: float
    balancer: str  # "fbs" or "vbs"
    alpha: tuple  # (num, den) for VBS weights L**alpha
    iterations: int
    lengths: tuple  # distribution spec
    max_uih: int
    cand_max: int  # candidates uniform 1..cand_max, 0 = none
    locality: float = 0.0
    drift: float = 0.0
    extra: dict = field(default_factory=dict)


WORKLOADS = {
    1: Workload(
        "B64-W4-100Kx64-f32-sgd", 64, 4,
        (TableSpec(100_000, 64, "f32", 1.05),),
        "sgd", 0.01, 0.0, "fbs", (1, 1), 2,
        ("lognormal", 3.5, 1.0), 256, 4),
    2: Workload(
        "B512-W16-10Mx128-f32-adagrad", 512, 16,
        (TableSpec(10_000_000, 128, "f32", 1.1),),
        "rw_adagrad", 0.05, 1e-8, "fbs", (1, 1), 4,
        ("pareto", 1.5, 16.0), 2048, 8),
    3: Workload(
        "B1024-W64-50Mx128-bf16-adagrad-vbs1.5", 1024, 64,
        (TableSpec(50_000_000, 128, "bf16", 1.05),),
        "rw_adagrad", 0.05, 1e-8, "vbs", (3, 2), 8,
        ("mixture", 0.9, 5.0, 1.0, 2048, 8192), 8192, 16, locality=0.3),
    4: Workload(
        "B2048-W256-4tables-f32-sgd-vbs2", 2048, 256,
        (TableSpec(20_000_000, 64, "f32", 1.0),
         TableSpec(20_000_000, 128, "f32", 1.05),
         TableSpec(20_000_000, 256, "f32", 1.1),
         TableSpec(5_000_000, 64, "f32", 1.2)),
        "sgd", 0.01, 0.0, "vbs", (2, 1), 8,
        ("pareto", 1.2, 32.0), 16384, 0),
    5: Workload(
        "B4096-W512-200Mx128-bf16-adagrad", 4096, 512,
        (TableSpec(200_000_000, 128, "bf16", 1.05),),
        "rw_adagrad", 0.05, 1e-8, "fbs", (3, 2), 16,
        ("lognormal", 6.5, 1.3), 32768, 0, drift=0.01),
}


def workload(k: int, balancer: str | None = None, scale_rows: int | None = None) -> Workload:
    """Workload ``k`` (1..5), optionally with another balancer or fewer table rows.

    ``scale_rows`` divides every table's row count (used by CPU-sized tests to
    keep tables small while keeping the length and ID mix).
    """
    w = WORKLOADS[k]
    kw = dict(w.__dict__)
    if balancer is not None:
        kw["balancer"] = balancer
    if scale_rows:
        kw["tables"] = tuple(TableSpec(max(1, t.rows // scale_rows), t.dim, t.dtype, t.zipf_s)
                             for t in w.tables)
    return Workload(**kw)


# ----------------------------------------------------------------------------
# random streams

_S_LEN, _S_CAND, _S_MIX, _S_LOC, _S_DRIFT, _S_PERM, _S_ID = 0, 1, 2, 3, 4, 5, 16


def _rng(seed: int, it: int, stream: int) -> np.random.Generator:
    return np.random.default_rng([int(seed), int(it), int(stream)])


def draw_lengths(w: Workload, seed: int, it: int) -> np.ndarray:
    rng = _rng(seed, it, _S_LEN)
    n = w.batch
    kind = w.lengths[0]
    if kind == "lognormal":
        x = rng.lognormal(w.lengths[1], w.lengths[2], size=n)
    elif kind == "pareto":
        shape, scale = w.lengths[1], w.lengths[2]
        u = 1.0 - rng.random(n)  # (0, 1]
        x = scale * u ** (-1.0 / shape)
    elif kind == "mixture":
        p_ln, mu, sigma, lo, hi = w.lengths[1:]
        ln = rng.lognormal(mu, sigma, size=n)
        un = rng.integers(lo, hi + 1, size=n).astype(np.float64)
        pick = _rng(seed, it, _S_MIX).random(n) < p_ln
        x = np.where(pick, ln, un)
    else:
        raise ValueError(kind)
    L = np.minimum(np.ceil(x), w.max_uih)
    return np.maximum(L, 1).astype(np.int32)


def draw_candidates(w: Workload, seed: int, it: int) -> np.ndarray:
    if w.cand_max <= 0:
        return np.zeros(w.batch, np.int32)
    return _rng(seed, it, _S_CAND).integers(1, w.cand_max + 1, size=w.batch).astype(np.int32)


class ZipfSampler:
    """Bounded Zipf over ranks 1..R: exact CDF for the head, power-law tail."""

    HEAD = 1 << 20

    def __init__(self, R: int, s: float):
        self.R, self.s = int(R), float(s)
        K = min(self.R, self.HEAD)
        w = np.arange(1, K + 1, dtype=np.float64) ** (-self.s)
        self.cdf = np.cumsum(w)
        self.head_mass = float(self.cdf[-1])
        self.K = K
        self.tail_mass = self._F(self.R + 0.5) - self._F(K + 0.5) if self.R > K else 0.0
        self.total = self.head_mass + self.tail_mass

    def _F(self, x):  # antiderivative of x**-s
        if abs(self.s - 1.0) < 1e-12:
            return np.log(x)
        return x ** (1.0 - self.s) / (1.0 - self.s)

    def _Finv(self, y):
        if abs(self.s - 1.0) < 1e-12:
            return np.exp(y)
        return (y * (1.0 - self.s)) ** (1.0 / (1.0 - self.s))

    def ranks(self, rng: np.random.Generator, size: int) -> np.ndarray:
        """0-based ranks (0 = hottest)."""
        u = rng.random(size) * self.total
        out = np.empty(size, np.int64)
        head = u < self.head_mass
        out[head] = np.searchsorted(self.cdf, u[head], side="right")
        if self.R > self.K:
            ut = u[~head] - self.head_mass
            x = self._Finv(self._F(self.K + 0.5) + ut)
            k = np.floor(x + 0.5).astype(np.int64)  # 1-based rank
            out[~head] = np.clip(k, self.K + 1, self.R) - 1
        np.minimum(out, self.R - 1, out=out)
        return out


def _par_chunks(n: int, fn, block: int = 1 << 16):
    """Run fn(lo, hi) over [0, n) in cache-sized blocks on a small thread pool.

    numpy releases the GIL inside its ufuncs, so blocks run in parallel.
    """
    starts = list(range(0, n, block))
    workers = max(1, min(8, os.cpu_count() or 1, len(starts)))
    if workers == 1:
        for lo in starts:
            fn(lo, min(n, lo + block))
        return
    with ThreadPoolExecutor(workers) as ex:
        list(ex.map(lambda lo: fn(lo, min(n, lo + block)), starts))


def _perm_key(seed: int, table: int) -> int:
    return int(_rng(seed, 0, _S_PERM + 100 * table).integers(0, 2**62))


def feistel_permutation(R: int, key: int) -> np.ndarray:
    """A seeded permutation of [0, R) as an explicit array.

    Built from a 4-round balanced Feistel network over the smallest even-bit
    power-of-two domain covering R, with cycle walking back into [0, R)
    (the standard construction of a keyed bijection on an arbitrary range).
    Much faster than a Fisher-Yates shuffle at hundreds of millions of rows.
    """
    R = int(R)
    bits = max(2, int(math.ceil(math.log2(max(R, 2)))))
    bits += bits & 1
    h = bits // 2
    mask = np.uint64((1 << h) - 1)
    keys = mix64(np.array([key + i for i in range(4)], np.uint64))

    def enc(x):
        lo = x & mask
        hi = x >> np.uint64(h)
        for k in keys:
            f = mix64(lo ^ k) & mask
            lo, hi = hi ^ f, lo
        return (hi << np.uint64(h)) | lo

    out = np.empty(R, np.int32 if R < 2**31 else np.int64)

    def work(a, b):
        y = enc(np.arange(a, b, dtype=np.uint64))
        bad = np.nonzero(y >= np.uint64(R))[0]
        while len(bad):
            y[bad] = enc(y[bad])
            bad = bad[y[bad] >= np.uint64(R)]
        out[a:b] = y

    _par_chunks(R, work, block=1 << 18)
    return out


class Batches:
    """Iteration-by-iteration inputs of one workload (drift is cumulative)."""

    def __init__(self, w: Workload, seed: int):
        self.w, self.seed = w, int(seed)
        self.samplers = [ZipfSampler(t.rows, t.zipf_s) for t in w.tables]
        self.rank_to_row = [feistel_permutation(t.rows, _perm_key(seed, ti))
                            for ti, t in enumerate(w.tables)]
        self._next_it = 0

    def _drift(self, it: int):
        for ti, t in enumerate(self.w.tables):
            m = int(math.ceil(self.w.drift * t.rows))
            if m < 2:
                continue
            rng = _rng(self.seed, it, _S_DRIFT + 100 * ti)
            sel = np.unique(rng.integers(0, t.rows, size=m + m // 64 + 16))
            sel = rng.permutation(sel)[:m]
            perm = self.rank_to_row[ti]
            perm[sel] = perm[sel[rng.permutation(len(sel))]]

    def batch(self, it: int) -> dict:
        """Inputs of iteration ``it``; iterations must be requested in order."""
        if it != self._next_it:
            raise ValueError(f"iterations are generated in order; expected {self._next_it}")
        if it > 0 and self.w.drift > 0:
            self._drift(it)
        self._next_it += 1
        w = self.w
        L = draw_lengths(w, self.seed, it)
        C = draw_candidates(w, self.seed, it)
        ntok = L.astype(np.int64) + C
        so = np.zeros(w.batch + 1, np.int64)
        np.cumsum(ntok, out=so[1:])
        n = int(so[-1])
        ids = np.empty((len(w.tables), n), np.int64)
        for ti, t in enumerate(w.tables):
            rng = _rng(self.seed, it, _S_ID + ti)
            r = self.samplers[ti].ranks(rng, n)
            if w.locality > 0:
                r = _apply_locality(r, so, w.locality, _rng(self.seed, it, _S_LOC + 100 * ti))
            ids[ti] = self.rank_to_row[ti][r]
        return dict(uih_len=L, num_cand=C, sample_offsets=so, ids=ids, n_tok=n)


def _apply_locality(r: np.ndarray, so: np.ndarray, p: float, rng: np.random.Generator) -> np.ndarray:
    n = len(r)
    seg_start = np.repeat(so[:-1], np.diff(so))
    j = np.arange(n, dtype=np.int64) - seg_start
    copy = (rng.random(n) < p) & (j >= 1)
    pick = np.floor(rng.random(n) * np.maximum(j, 1)).astype(np.int64)
    src = np.where(copy, seg_start + pick, np.arange(n, dtype=np.int64))
    # follow copy chains to the first fresh draw (src[k] < k when copying)
    root = src.copy()
    while True:
        nxt = src[root]
        if np.array_equal(nxt, root):
            break
        root = nxt
    return r[root]


# ----------------------------------------------------------------------------
# gradients (counter-based hash) and tables

_M64 = np.uint64(0xFFFFFFFFFFFFFFFF)
_GAMMA = np.uint64(0x9E3779B97F4A7C15)
_C1 = np.uint64(0xBF58476D1CE4E5B9)
_C2 = np.uint64(0x94D049BB133111EB)


def mix64(z: np.ndarray) -> np.ndarray:
    """splitmix64 output function (Vigna), elementwise on uint64."""
    with np.errstate(over="ignore"):
        z = z.astype(np.uint64, copy=True)
        z ^= z >> np.uint64(30)
        z *= _C1
        z ^= z >> np.uint64(27)
        z *= _C2
        z ^= z >> np.uint64(31)
    return z


def token_keys(seed: int, it: int, table: int, tok: np.ndarray) -> np.ndarray:
    base = mix64(np.array([(int(seed) << 40) ^ (int(it) << 20) ^ int(table)], np.uint64))[0]
    with np.errstate(over="ignore"):
        return mix64(base + _GAMMA * (tok.astype(np.uint64) + np.uint64(1)))


def gradient_rows(seed: int, it: int, table: int, tok: np.ndarray, dim: int,
                  out: np.ndarray | None = None) -> np.ndarray:
    """fp32 gradient rows for token indices ``tok`` (shape [len(tok), dim])."""
    tok = np.asarray(tok, np.int64)
    if out is None:
        out = np.empty((len(tok), dim), np.float32)
    cols = _GAMMA * (np.arange(dim, dtype=np.uint64) + np.uint64(1))

    def work(lo, hi):
        k = token_keys(seed, it, table, tok[lo:hi])
        with np.errstate(over="ignore"):
            h = mix64(k[:, None] + cols[None, :])
        v = (h >> np.uint64(40)).astype(np.int64) - (1 << 23)
        out[lo:hi] = (v.astype(np.float32) * np.float32(2.0 ** -23))

    _par_chunks(len(tok), work, block=max(1, (1 << 17) // max(dim, 1)))
    return out


def init_table(rows: int, dim: int, dtype: str, seed: int, device="cpu", table: int = 0,
               out=None):
    """N(0, 0.01**2) table from torch's seeded generator, rounded to ``dtype``;
    written into ``out`` (a [rows, dim] tensor or row view) when given."""
    import torch

    g = torch.Generator(device=device)
    g.manual_seed(int(seed) * 1000 + int(table))
    tdt = torch.float32 if dtype == "f32" else torch.bfloat16
    if out is None:
        out = torch.empty((rows, dim), dtype=tdt, device=device)
    assert out.shape == (rows, dim) and out.dtype == tdt
    chunk = max(1, (1 << 28) // max(dim, 1))
    for lo in range(0, rows, chunk):
        hi = min(rows, lo + chunk)
        x = torch.randn((hi - lo, dim), generator=g, device=device, dtype=torch.float32)
        x.mul_(0.01)
        out[lo:hi].copy_(x)
    return out
