"""ctypes binding of the CPU oracle (fs_oracle.c) and its synchronous loop.

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, ``__graft_entry__.smoke()``
and the CPU-baseline leg of ``bench.py``. The product path never imports it.

``SyncRun`` is the plain synchronous training loop that the prioritized
schedule must reproduce exactly (FreeScale paper, section 3.2: keeping a strict
write-then-read order on the collision rows gives numerical parity with the
synchronized baseline): per iteration, balance, permute, dedup, look up every
row from the current table, reduce the gradients and update every row.
"""

from __future__ import annotations

import ctypes as C
import os
import subprocess
import time

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "fs_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")


def build(force: bool = False) -> str:
    """Compile the oracle with gcc (single-threaded, no FP contraction)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-ffp-contract=off", "-fPIC", "-shared",
                               "-Wall", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


class _Store(C.Structure):
    _fields_ = [("row_ids", C.c_void_p), ("n_rows", C.c_int64), ("vals", C.c_void_p),
                ("state", C.c_void_p), ("dim", C.c_int32), ("bf16", C.c_int32)]


def lib():
    global _lib
    if _lib is None:
        L = C.CDLL(build())
        P = C.c_void_p
        i32, i64 = C.c_int32, C.c_int64
        L.or_fbs_rank_of_position.argtypes = [i64, i32]
        L.or_fbs_rank_of_position.restype = i32
        L.or_balance_fbs.argtypes = [P, i32, i32, P, P]
        L.or_balance_fbs.restype = C.c_int
        L.or_vbs_weight.argtypes = [i64, i32, i32]
        L.or_vbs_weight.restype = i64
        L.or_balance_vbs.argtypes = [P, i32, i32, i32, i32, P, P, P]
        L.or_balance_vbs.restype = C.c_int
        L.or_balance_vbs_shares.argtypes = [P, i32, i32, i32, i32, P, P, P, P]
        L.or_balance_vbs_shares.restype = C.c_int
        L.or_rank_cost.argtypes = [P, P, P, i32, i64, i64, i64, P]
        L.or_rank_cost.restype = None
        L.or_vbs_autotune.argtypes = [P, i32, i32, i32, i32, i32, P]
        L.or_vbs_autotune.restype = None
        L.or_bucketize.argtypes = [P, i64, P, i32, i32, P, P, P, P, i32, P, P, P, P, P, P]
        L.or_bucketize.restype = i64
        L.or_unique.argtypes = [P, P, i64, i32, P, P, i32, P, P, P, P, P]
        L.or_unique.restype = i64
        L.or_collision.argtypes = [P, i64, P, i64, P, P, P]
        L.or_collision.restype = None
        L.or_ranged_combine.argtypes = [P, i64, P, P, i64, i32, P, P, C.POINTER(P)]
        L.or_ranged_combine.restype = None
        L.or_keyed_transpose.argtypes = [P, P, i32, i32, P, P]
        L.or_keyed_transpose.restype = None
        L.or_lookup.argtypes = [C.POINTER(_Store), i64, i64, i64, P, P, P, P, i32, P]
        L.or_lookup.restype = i64
        L.or_reduce.argtypes = [i32, i64, i64, P, P, P, P]
        L.or_reduce.restype = None
        L.or_update.argtypes = [C.POINTER(_Store), i64, i64, i64, P, P, i32, P, i32, C.c_float,
                                C.c_float]
        L.or_update.restype = i64
        L.or_bf16_to_f32.argtypes = [C.c_uint16]
        L.or_bf16_to_f32.restype = C.c_float
        L.or_f32_to_bf16.argtypes = [C.c_float]
        L.or_f32_to_bf16.restype = C.c_uint16
        _lib = L
    return _lib


def _p(a: np.ndarray):
    assert a.flags.c_contiguous
    return a.ctypes.data


def _c(a, dt):
    return np.ascontiguousarray(a, dtype=dt)


# ----------------------------------------------------------------------------
# stage wrappers


def balance_fbs(uih_len, W):
    L = _c(uih_len, np.int32)
    perm = np.empty(len(L), np.int32)
    ro = np.empty(W + 1, np.int32)
    assert lib().or_balance_fbs(_p(L), len(L), W, _p(perm), _p(ro)) == 0
    return perm, ro


def balance_vbs(uih_len, W, alpha=(3, 2)):
    L = _c(uih_len, np.int32)
    perm = np.empty(len(L), np.int32)
    ro = np.empty(W + 1, np.int32)
    rw = np.empty(W, np.int64)
    rc = lib().or_balance_vbs(_p(L), len(L), W, int(alpha[0]), int(alpha[1]), _p(perm), _p(ro),
                              _p(rw))
    if rc != 0:
        raise ValueError(f"or_balance_vbs failed ({rc})")
    return perm, ro, rw


def balance_vbs_shares(uih_len, W, shares, alpha=(3, 2)):
    """[FS] 4.1 VBS with per-rank shares of the weight (the AutoTune reading)."""
    L = _c(uih_len, np.int32)
    sh = _c(shares, np.int64)
    assert len(sh) == W
    perm = np.empty(len(L), np.int32)
    ro = np.empty(W + 1, np.int32)
    rw = np.empty(W, np.int64)
    rc = lib().or_balance_vbs_shares(_p(L), len(L), W, int(alpha[0]), int(alpha[1]), _p(sh),
                                     _p(perm), _p(ro), _p(rw))
    if rc != 0:
        raise ValueError(f"or_balance_vbs_shares failed ({rc})")
    return perm, ro, rw


def rank_cost(uih_len, perm, rank_offsets, coef):
    """Modelled per-rank time: sum of c2 L^2 + c1 L + c0 over the rank's samples."""
    L = _c(uih_len, np.int32)
    pm = _c(perm, np.int32)
    ro = _c(rank_offsets, np.int32)
    W = len(ro) - 1
    out = np.empty(W, np.int64)
    c2, c1, c0 = (int(c) for c in coef)
    lib().or_rank_cost(_p(L), _p(pm), _p(ro), W, c2, c1, c0, _p(out))
    return out


def vbs_autotune(times, shares, step=(1, 16), tol=(1, 20)):
    """One AutoTune step; returns the new shares (the input is not changed)."""
    t = _c(times, np.int64)
    sh = np.array(shares, dtype=np.int64, copy=True)
    assert len(t) == len(sh)
    lib().or_vbs_autotune(_p(t), len(t), int(step[0]), int(step[1]), int(tol[0]), int(tol[1]),
                          _p(sh))
    return sh


def vbs_weight(L, alpha):
    return int(lib().or_vbs_weight(int(L), int(alpha[0]), int(alpha[1])))


def fbs_rank_of_position(p, W):
    return int(lib().or_fbs_rank_of_position(int(p), int(W)))


def bucketize(ids, sample_offsets, rows, perm, rank_offsets, W):
    ids = _c(np.atleast_2d(ids), np.int64)
    T, n_tok = ids.shape
    so = _c(sample_offsets, np.int64)
    N = len(so) - 1
    rows_a = _c(rows, np.int64)
    rb = np.zeros(T, np.int64)
    rb[1:] = np.cumsum(rows_a)[:-1]
    perm = _c(perm, np.int32)
    ro = _c(rank_offsets, np.int32)
    n = T * n_tok
    bal = np.empty(N + 1, np.int64)
    keys = np.empty(max(n, 1), np.int64)
    bm = np.empty(max(n, 1), np.int32)
    splits = np.empty(W * W, np.int64)
    sho = np.empty(W + 1, np.int64)
    err = np.zeros(1, np.int32)
    nv = lib().or_bucketize(_p(ids), n_tok, _p(so), N, T, _p(rows_a), _p(rb), _p(perm), _p(ro), W,
                            _p(bal), _p(keys), _p(bm), _p(splits), _p(sho), _p(err))
    return dict(bal_offsets=bal, shard_keys=keys[:nv], shard_bm=bm[:nv],
                splits=splits.reshape(W, W), shard_offsets=sho, err=int(err[0]), row_base=rb)


def ranged_combine(src, shard_keys, shard_bm, rows, row_bytes, n_tok):
    """[FS] 4.2 ranged combine (one GPU, every virtual rank): row k of src
    (uint8 [n_valid, stride]) goes to slot shard_bm[k] of its table's output
    (uint8 [n_tok, row_bytes[t]], zero where no item maps)."""
    src = _c(src, np.uint8)
    keys = _c(shard_keys, np.int64)
    bm = _c(shard_bm, np.int32)
    T = len(rows)
    rb = np.zeros(T + 1, np.int64)
    rb[1:] = np.cumsum(_c(rows, np.int64))
    rbytes = _c(row_bytes, np.int64)
    outs = [np.zeros((n_tok, int(r)), np.uint8) for r in rbytes]
    arr = (C.c_void_p * T)(*[o.ctypes.data for o in outs])
    lib().or_ranged_combine(_p(src), src.shape[1] if src.ndim == 2 else 0, _p(keys), _p(bm),
                            len(keys), T, _p(rb), _p(rbytes), arr)
    return outs


def keyed_transpose(values, lengths):
    """[FS] 4.2 keyed transpose: lengths int [F, B] (feature-major), values the
    feature-major concatenation. Returns (batch-major values, out_offsets
    [B*F + 1] with out_offsets[b*F + f] the start of (b, f))."""
    lengths = _c(lengths, np.int32)
    F, B = lengths.shape
    values = _c(values, np.int64)
    out = np.empty(max(len(values), 1), np.int64)
    off = np.empty(F * B + 1, np.int64)
    lib().or_keyed_transpose(_p(values), _p(lengths), F, B, _p(out), _p(off))
    return out[:len(values)], off


def unique(shard_keys, shard_bm, rows, W):
    keys = _c(shard_keys, np.int64)
    bm = _c(shard_bm, np.int32)
    n = len(keys)
    rows_a = _c(rows, np.int64)
    T = len(rows_a)
    rb = np.zeros(T, np.int64)
    rb[1:] = np.cumsum(rows_a)[:-1]
    uq = np.empty(max(n, 1), np.int64)
    uo = np.empty(T * W + 1, np.int64)
    seg = np.empty(n + 1, np.int32)
    occ_bm = np.empty(max(n, 1), np.int32)
    occ_uid = np.empty(max(n, 1), np.int32)
    U = lib().or_unique(_p(keys), _p(bm), n, T, _p(rows_a), _p(rb), W, _p(uq), _p(uo), _p(seg),
                        _p(occ_bm), _p(occ_uid))
    return dict(unique=uq[:U].copy(), unique_offsets=uo, seg_offsets=seg[:U + 1].copy(),
                occ_bm=occ_bm[:n].copy(), occ_uid=occ_uid[:n].copy())


def collision(unique_new, unique_prev):
    a = _c(unique_new, np.int64)
    b = _c(unique_prev if unique_prev is not None else np.zeros(0, np.int64), np.int64)
    cls = np.empty(max(len(a), 1), np.uint8)
    pcls = np.empty(max(len(b), 1), np.uint8)
    counts = np.empty(4, np.int64)
    lib().or_collision(_p(a), len(a), _p(b), len(b), _p(cls), _p(pcls), _p(counts))
    return cls[:len(a)].copy(), pcls[:len(b)].copy(), counts


def bf16_to_f32(h):
    return float(lib().or_bf16_to_f32(int(h)))


def f32_to_bf16(f):
    return int(lib().or_f32_to_bf16(float(f)))


class RowStore:
    """Touched rows of one table: ascending row ids, values, Adagrad state."""

    def __init__(self, row_ids, vals, state=None, bf16=False):
        self.row_ids = _c(row_ids, np.int64)
        self.bf16 = bool(bf16)
        self.vals = _c(vals, np.uint16 if bf16 else np.float32)
        assert self.vals.shape[0] == len(self.row_ids)
        self.dim = self.vals.shape[1]
        self.state = _c(state if state is not None else np.zeros(len(self.row_ids)), np.float32)

    def _s(self):
        return _Store(_p(self.row_ids), len(self.row_ids), _p(self.vals), _p(self.state),
                      self.dim, int(self.bf16))

    def rows_of(self, row_ids):
        idx = np.searchsorted(self.row_ids, row_ids)
        assert np.all(self.row_ids[idx] == row_ids)
        return self.vals[idx], self.state[idx]


def lookup(store, row_base, u_lo, u_hi, uq, n_tok, which=-1, out=None):
    if out is None:
        out = np.zeros((n_tok, store.dim), store.vals.dtype)
    s = store._s()
    miss = lib().or_lookup(C.byref(s), row_base, u_lo, u_hi, _p(uq["unique"]),
                           _p(uq["seg_offsets"]), _p(uq["occ_bm"]),
                           _p(uq.get("cls", np.zeros(max(len(uq["unique"]), 1), np.uint8))),
                           which, _p(out))
    assert miss == 0, f"{miss} rows missing from the store"
    return out


def reduce(dim, u_lo, u_hi, uq, grad):
    grad = _c(grad, np.float32)
    g = np.empty((max(u_hi - u_lo, 1), dim), np.float32)
    lib().or_reduce(dim, u_lo, u_hi, _p(uq["seg_offsets"]), _p(uq["occ_bm"]), _p(grad), _p(g))
    return g[:u_hi - u_lo]


def update(store, row_base, u_lo, u_hi, unique_keys, g, optim, lr, eps, cls=None, which=-1):
    s = store._s()
    g = _c(g, np.float32)
    cls_a = _c(cls if cls is not None else np.zeros(max(len(unique_keys), 1)), np.uint8)
    miss = lib().or_update(C.byref(s), row_base, u_lo, u_hi, _p(_c(unique_keys, np.int64)),
                           _p(cls_a), which, _p(g), 1 if optim == "rw_adagrad" else 0,
                           np.float32(lr), np.float32(eps))
    assert miss == 0, f"{miss} rows missing from the store"


# ----------------------------------------------------------------------------
# the synchronous loop


class SyncRun:
    """Plain synchronous sparse steps over a sequence of batches.

    ``stores[t]`` holds at least every row of table t that the run touches.
    ``step(batch, grad_fn)`` runs one iteration and returns every stage output;
    ``grad_fn(t, n_tok, bal) -> fp32 [n_tok, dim]`` supplies the batch-major
    gradient of the balanced batch.
    """

    def __init__(self, workload, stores, autotune=None):
        """autotune: None, or dict(coef, step, tol, init) -- VBS cut at
        per-rank shares, moved after each balance by the modelled time of
        the partition it made ([FS] 4.1 autotune)."""
        self.w = workload
        self.stores = stores
        self.autotune = autotune
        if autotune is not None:
            self.shares = np.full(workload.world, int(autotune["init"]), np.int64)
        self.rows = np.array([t.rows for t in workload.tables], np.int64)
        self.row_base = np.zeros(len(self.rows), np.int64)
        self.row_base[1:] = np.cumsum(self.rows)[:-1]
        self.prev_unique = None
        self.seconds = {}  # wall seconds per stage, summed over the run's iterations

    def _timed(self, name, fn, *a):
        t0 = time.perf_counter()
        r = fn(*a)
        self.seconds[name] = self.seconds.get(name, 0.0) + time.perf_counter() - t0
        return r

    def index_stages(self, batch):
        w = self.w
        tm = self._timed
        if w.balancer == "fbs":
            perm, ro = tm("balance", balance_fbs, batch["uih_len"], w.world)
            rw = None
        elif self.autotune is None:
            perm, ro, rw = tm("balance", balance_vbs, batch["uih_len"], w.world, w.alpha)
        else:
            at = self.autotune
            perm, ro, rw = tm("balance", balance_vbs_shares, batch["uih_len"], w.world,
                              self.shares, w.alpha)
            cost = rank_cost(batch["uih_len"], perm, ro, at["coef"])
            self.shares = vbs_autotune(cost, self.shares, at["step"], at["tol"])
        bk = tm("bucketize", bucketize, batch["ids"], batch["sample_offsets"], self.rows, perm,
                ro, w.world)
        uq = tm("dedup", unique, bk["shard_keys"], bk["shard_bm"], self.rows, w.world)
        cls, pcls, counts = tm("collision", collision, uq["unique"], self.prev_unique)
        uq["cls"] = cls
        return dict(perm=perm, rank_offsets=ro, rank_weight=rw, bucket=bk, uniq=uq,
                    prev_cls=pcls, counts=counts)

    def lookup_all(self, out, n_tok):
        """Lookup of every unique row from the current rows (before the update)."""
        uq = out["uniq"]
        W = self.w.world
        emb = []
        for t, st in enumerate(self.stores):
            lo = int(uq["unique_offsets"][t * W])
            hi = int(uq["unique_offsets"][(t + 1) * W])
            emb.append(lookup(st, int(self.row_base[t]), lo, hi, uq, n_tok))
        return emb

    def reduce_update(self, out, grads):
        """Reduce the balanced batch-major gradients per unique row and update."""
        uq = out["uniq"]
        W = self.w.world
        red = []
        for t, st in enumerate(self.stores):
            lo = int(uq["unique_offsets"][t * W])
            hi = int(uq["unique_offsets"][(t + 1) * W])
            g = reduce(st.dim, lo, hi, uq, grads[t])
            update(st, int(self.row_base[t]), lo, hi, uq["unique"], g, self.w.optim, self.w.lr,
                   self.w.eps)
            red.append(g)
        return red

    def step(self, batch, grads_fn):
        """One synchronous iteration. grads_fn(index_outputs) -> list of T
        balanced batch-major fp32 gradients."""
        out = self.index_stages(batch)
        out["emb"] = self._timed("lookup", self.lookup_all, out, batch["n_tok"])
        g = grads_fn(out)
        out["reduced"] = self._timed("reduce_update", self.reduce_update, out, g)
        self.prev_unique = out["uniq"]["unique"]
        return out
