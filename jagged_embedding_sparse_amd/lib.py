"""ctypes binding of libfs_sparse.so (the C ABI in include/fs_sparse.h).

Argument marshalling only: every function takes torch tensors on the GPU,
allocates any output the caller did not pass, hands raw pointers and the
current HIP stream to the C call and raises on a non-zero return code. All
computation happens in the library's HIP kernels; there is no fallback: if
the library is missing, importing this module raises.
"""

from __future__ import annotations

import ctypes as C
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.environ.get("FS_SPARSE_LIB", os.path.join(_HERE, "libfs_sparse.so"))

FS_OK, FS_ERR_INVALID_ARG, FS_ERR_WORKSPACE, FS_ERR_HIP, FS_ERR_UNSUPPORTED = 0, -1, -2, -3, -4
FS_ERR_TOO_LARGE = -5
FS_NOALLOC_SCRATCH_BYTES = 64 << 20
FS_EF_ID_RANGE, FS_EF_SHAPE, FS_EF_LEN_RANGE = 1, 2, 4
FS_F32, FS_BF16 = 0, 1
FS_SGD, FS_RW_ADAGRAD = 0, 1
FS_ALL, FS_EXCLUSIVE, FS_COLLISION = -1, 0, 1
FS_ROWS_FEW, FS_ROWS_MANY, FS_ROWS_ALL = 1, 2, 3
FS_MAX_SAMPLES, FS_MAX_RANKS, FS_MAX_TABLES, FS_MAX_UIH = 16384, 1024, 8, 65535

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is not built: run `python __graft_entry__.py build` "
                      "(or jagged_embedding_sparse_amd/build.py) first")


class FsTable(C.Structure):
    _fields_ = [("weights", C.c_void_p), ("state", C.c_void_p), ("rows", C.c_int64),
                ("dim", C.c_int32), ("dtype", C.c_int32), ("stride", C.c_int64),
                ("state_stride", C.c_int64)]


_L = C.CDLL(LIB_PATH)
_P, _i32, _i64, _sz, _f = C.c_void_p, C.c_int32, C.c_int64, C.c_size_t, C.c_float
_TP = C.POINTER(FsTable)


def _sig(name, res, *args):
    fn = getattr(_L, name)
    fn.restype = res
    fn.argtypes = list(args)
    return fn


_c_balance_fbs = _sig("fs_balance_fbs", C.c_int, _P, _i32, _i32, _P, _P, _P, _P, _sz, _P)
_c_balance_vbs = _sig("fs_balance_vbs", C.c_int, _P, _i32, _i32, _i32, _i32, _P, _P, _P, _P, _P,
                      _sz, _P)
_c_balance_ws = _sig("fs_balance_workspace_size", _sz, _i32, _i32)
_c_balance_shares = _sig("fs_balance_vbs_shares", C.c_int, _P, _i32, _i32, _i32, _i32, _P, _P,
                         _P, _P, _P, _P, _sz, _P)
_c_rank_cost = _sig("fs_rank_cost", C.c_int, _P, _i32, _P, _P, _i32, _i64, _i64, _i64, _P, _P)
_c_autotune = _sig("fs_vbs_autotune", C.c_int, _P, _i32, _i32, _i32, _i32, _i32, _P, _P, _P)
_c_bucketize = _sig("fs_bucketize_permute", C.c_int, _P, _i64, _P, _i32, _TP, _i32, _P, _P, _i32,
                    _P, _P, _P, _P, _P, _P, _P, _sz, _P)
_c_bucketize_ws = _sig("fs_bucketize_workspace_size", _sz, _i64, _i32, _i32, _i32)
_c_unique = _sig("fs_unique_collision_split", C.c_int, _P, _P, _P, _i64, _TP, _i32, _i32, _P, _P,
                 _P, _i64, _P, _P, _P, _P, _P, _P, _P, _P, _P, _sz, _P)
_c_unique_ws = _sig("fs_unique_workspace_size", _sz, _i64, _i64, _i32, _i32)
_c_collide = _sig("fs_collision_split", C.c_int, _P, _P, _i64, _i32, _i32, _P, _P, _P, _i64, _P,
                  _P, _P, _P, _sz, _P)
_c_collide_ws = _sig("fs_collision_split_workspace_size", _sz, _i64, _i32, _i32)
_c_lookup = _sig("fs_jagged_lookup", C.c_int, _TP, _i32, _i32, _P, _P, _P, _P, _P, _P, _i32,
                 C.POINTER(_P), _i64, _P)
_c_combine = _sig("fs_ranged_combine", C.c_int, _P, _i64, _P, _P, _P, _i32, _TP, _i32,
                  C.POINTER(_P), _i64, _P)
_c_kt = _sig("fs_keyed_transpose", C.c_int, _P, _i64, _i32, _P, _i32, _i32, _P, _P, _P, _P, _sz,
             _P)
_c_kt_ws = _sig("fs_keyed_transpose_workspace_size", _sz, _i32, _i32)
_c_reduce = _sig("fs_grad_reduce_update", C.c_int, _TP, _i32, _i32, C.POINTER(_P), _i64, _P, _P,
                 _P, _P, _P, _P, _i32, _i32, _i32, _f, _f, C.POINTER(_P), _P, _sz, _P)
_c_reduce_ws = _sig("fs_grad_reduce_update_workspace_size", _sz, _i64, _i32, _i32)
_c_reduce_noalloc = _sig("fs_grad_reduce_update_noalloc", C.c_int, _TP, _i32, _i32,
                         C.POINTER(_P), _i64, _P, _P, _P, _P, _P, _P, _i32, _i32, _i32, _f, _f,
                         C.POINTER(_P), _P)
_c_strerror = _sig("fs_strerror", C.c_char_p, C.c_int)
_c_version = _sig("fs_version", C.c_int)

EXPORTED = ["fs_balance_fbs", "fs_balance_vbs", "fs_balance_workspace_size",
            "fs_balance_vbs_shares", "fs_rank_cost", "fs_vbs_autotune",
            "fs_bucketize_permute", "fs_bucketize_workspace_size", "fs_unique_collision_split",
            "fs_unique_workspace_size", "fs_collision_split", "fs_collision_split_workspace_size",
            "fs_jagged_lookup", "fs_ranged_combine",
            "fs_keyed_transpose", "fs_keyed_transpose_workspace_size",
            "fs_grad_reduce_update", "fs_grad_reduce_update_noalloc",
            "fs_grad_reduce_update_workspace_size", "fs_strerror", "fs_version"]


class FsError(RuntimeError):
    def __init__(self, fn, code):
        super().__init__(f"{fn}: {strerror(code)} ({code})")
        self.code = code


def strerror(code: int) -> str:
    return _c_strerror(int(code)).decode()


def version() -> int:
    return int(_c_version())


def _ptr(t):
    if t is None:
        return None
    assert t.is_cuda and t.is_contiguous(), "device tensors must be contiguous CUDA tensors"
    return t.data_ptr()


def _stream(stream):
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


def _check(fn, rc):
    if rc != FS_OK:
        raise FsError(fn, rc)


def _dev():
    return torch.device("cuda", torch.cuda.current_device())


def _get(o, key, make):
    """o[key] if present, else a fresh tensor from make() (evaluated lazily)."""
    return o[key] if key in o and o[key] is not None else make()


def _ws(nbytes, ws):
    if ws is not None:
        assert ws.numel() * ws.element_size() >= nbytes
        return ws
    return torch.empty(max(int(nbytes), 1), dtype=torch.uint8, device=_dev())


def _rows_ptr(t):
    """Device pointer and row stride in bytes of a [rows, dim] tensor whose
    rows are contiguous (the rows themselves may be spaced further apart)."""
    assert t.is_cuda and t.stride(-1) == 1, "table rows must be contiguous CUDA memory"
    return t.data_ptr(), (t.stride(0) * t.element_size() if t.dim() == 2 else 0)


def _state_ptr(st):
    """Device pointer and spacing in bytes of a [rows] fp32 state tensor."""
    assert st.is_cuda and st.dtype == torch.float32 and st.dim() == 1
    return st.data_ptr(), st.stride(0) * 4


def make_tables(weights, states=None):
    """Host array of fs_table for a list of [rows, dim] weight tensors (dense,
    or row views of a wider buffer as alloc_table makes) and their [rows]
    states (dense, or views with the rows' spacing)."""
    T = len(weights)
    arr = (FsTable * T)()
    for t, w in enumerate(weights):
        st = states[t] if states is not None else None
        assert w.dtype in (torch.float32, torch.bfloat16) and w.dim() == 2
        arr[t].weights, arr[t].stride = _rows_ptr(w)
        if st is not None:
            arr[t].state, arr[t].state_stride = _state_ptr(st)
        arr[t].rows = w.shape[0]
        arr[t].dim = w.shape[1]
        arr[t].dtype = FS_F32 if w.dtype == torch.float32 else FS_BF16
    return arr


def alloc_table(rows, dim, dtype, with_state, device=None, align=16):
    """Table memory with each row's fp32 state in the row's own padding: one
    buffer of rows x stride bytes (stride = the row plus 4 bytes, rounded up
    to `align`, a multiple of 16). Returns (weights [rows, dim] view, state
    [rows] view or None)."""
    assert align % 16 == 0
    e = 4 if dtype == torch.float32 else 2
    rb = dim * e
    stride = (rb + (4 if with_state else 0) + align - 1) // align * align
    buf = torch.empty((rows, stride), dtype=torch.uint8, device=device or _dev())
    w = buf[:, :rb].view(dtype)
    st = buf[:, rb:rb + 4].view(torch.float32)[:, 0] if with_state else None
    return w, st


def make_row_tables(rows, dims=None):
    """Host fs_table array that only carries row counts (bucketize, unique)."""
    T = len(rows)
    arr = (FsTable * T)()
    for t, r in enumerate(rows):
        arr[t].rows = int(r)
        arr[t].dim = int(dims[t]) if dims is not None else 0
    return arr


# ---------------------------------------------------------------------------- calls


def balance_workspace_size(n, W):
    return int(_c_balance_ws(n, W))


def fs_balance_fbs(uih_len, W, perm=None, rank_offsets=None, err=None, ws=None, stream=None):
    n = uih_len.numel()
    perm = perm if perm is not None else torch.empty(n, dtype=torch.int32, device=_dev())
    ro = rank_offsets if rank_offsets is not None else torch.empty(W + 1, dtype=torch.int32,
                                                                   device=_dev())
    ws = _ws(balance_workspace_size(n, W), ws)
    _check("fs_balance_fbs", _c_balance_fbs(_ptr(uih_len), n, W, _ptr(perm), _ptr(ro), _ptr(err),
                                            _ptr(ws), ws.numel(), _stream(stream)))
    return perm, ro


def fs_balance_vbs(uih_len, W, alpha=(3, 2), perm=None, rank_offsets=None, rank_weight=None,
                   err=None, ws=None, stream=None):
    n = uih_len.numel()
    perm = perm if perm is not None else torch.empty(n, dtype=torch.int32, device=_dev())
    ro = rank_offsets if rank_offsets is not None else torch.empty(W + 1, dtype=torch.int32,
                                                                   device=_dev())
    rw = rank_weight if rank_weight is not None else torch.empty(W, dtype=torch.int64,
                                                                 device=_dev())
    nb = balance_workspace_size(n, W)
    ws = _ws(nb, ws)
    _check("fs_balance_vbs", _c_balance_vbs(_ptr(uih_len), n, W, int(alpha[0]), int(alpha[1]),
                                            _ptr(perm), _ptr(ro), _ptr(rw), _ptr(err), _ptr(ws),
                                            ws.numel(), _stream(stream)))
    return perm, ro, rw


def fs_balance_vbs_shares(uih_len, W, shares, alpha=(3, 2), perm=None, rank_offsets=None,
                          rank_weight=None, err=None, ws=None, stream=None):
    """VBS cut at per-rank shares (device int64 [W]) of the weight."""
    n = uih_len.numel()
    perm = perm if perm is not None else torch.empty(n, dtype=torch.int32, device=_dev())
    ro = rank_offsets if rank_offsets is not None else torch.empty(W + 1, dtype=torch.int32,
                                                                   device=_dev())
    rw = rank_weight if rank_weight is not None else torch.empty(W, dtype=torch.int64,
                                                                 device=_dev())
    assert shares.dtype == torch.int64 and shares.numel() == W
    ws = _ws(balance_workspace_size(n, W), ws)
    _check("fs_balance_vbs_shares",
           _c_balance_shares(_ptr(uih_len), n, W, int(alpha[0]), int(alpha[1]), _ptr(shares),
                             _ptr(perm), _ptr(ro), _ptr(rw), _ptr(err), _ptr(ws), ws.numel(),
                             _stream(stream)))
    return perm, ro, rw


def fs_rank_cost(uih_len, perm, rank_offsets, coef=(1, 0, 0), cost=None, stream=None):
    """Modelled per-rank time: sum of c2 L^2 + c1 L + c0 over each rank's samples."""
    W = rank_offsets.numel() - 1
    cost = cost if cost is not None else torch.empty(W, dtype=torch.int64, device=_dev())
    c2, c1, c0 = (int(c) for c in coef)
    _check("fs_rank_cost", _c_rank_cost(_ptr(uih_len), uih_len.numel(), _ptr(perm),
                                        _ptr(rank_offsets), W, c2, c1, c0, _ptr(cost),
                                        _stream(stream)))
    return cost


def fs_vbs_autotune(times, shares, step=(1, 16), tol=(1, 20), err=None, stream=None):
    """One AutoTune step on shares (device int64 [W], in place) from per-rank
    times (device int64 [W])."""
    W = shares.numel()
    assert times.dtype == torch.int64 and times.numel() == W
    _check("fs_vbs_autotune", _c_autotune(_ptr(times), W, int(step[0]), int(step[1]),
                                          int(tol[0]), int(tol[1]), _ptr(shares), _ptr(err),
                                          _stream(stream)))
    return shares


def bucketize_workspace_size(n_tok, n, T, W):
    return int(_c_bucketize_ws(n_tok, n, T, W))


def fs_bucketize_permute(ids, sample_offsets, rows, perm, rank_offsets, W, out=None, err=None,
                         ws=None, stream=None):
    """ids: int64 [T, n_tok]. Returns dict of bal_offsets, shard_keys, shard_bm, splits,
    shard_offsets."""
    T, n_tok = ids.shape
    n = sample_offsets.numel() - 1
    d = _dev()
    o = out or {}
    bal = _get(o, "bal_offsets", lambda: torch.empty(n + 1, dtype=torch.int64, device=d))
    keys = _get(o, "shard_keys", lambda: torch.empty(max(T * n_tok, 1), dtype=torch.int64, device=d))
    bm = _get(o, "shard_bm", lambda: torch.empty(max(T * n_tok, 1), dtype=torch.int32, device=d))
    splits = _get(o, "splits", lambda: torch.empty(W * W, dtype=torch.int64, device=d))
    sho = _get(o, "shard_offsets", lambda: torch.empty(W + 1, dtype=torch.int64, device=d))
    tabs = make_row_tables(rows)
    ws = _ws(bucketize_workspace_size(n_tok, n, T, W), ws)
    _check("fs_bucketize_permute",
           _c_bucketize(_ptr(ids), n_tok, _ptr(sample_offsets), n, tabs, T, _ptr(perm),
                        _ptr(rank_offsets), W, _ptr(bal), _ptr(keys), _ptr(bm), _ptr(splits),
                        _ptr(sho), _ptr(err), _ptr(ws), ws.numel(), _stream(stream)))
    return dict(bal_offsets=bal, shard_keys=keys, shard_bm=bm, splits=splits, shard_offsets=sho)


def unique_workspace_size(n_cap, T, W, prev_cap=None):
    return int(_c_unique_ws(n_cap, n_cap if prev_cap is None else prev_cap, T, W))


def fs_unique_collision_split(shard_keys, shard_bm, shard_offsets, n_cap, rows, W,
                              prev_unique=None, prev_counts=None, prev_cap=0, out=None, ws=None,
                              stream=None, prev_unique_offsets=None):
    d = _dev()
    T = len(rows)
    cap = max(int(n_cap), 1)
    o = out or {}
    uq = _get(o, "unique", lambda: torch.empty(cap, dtype=torch.int64, device=d))
    uo = _get(o, "unique_offsets", lambda: torch.empty(T * W + 1, dtype=torch.int64, device=d))
    seg = _get(o, "seg_offsets", lambda: torch.empty(cap + 1, dtype=torch.int32, device=d))
    occ_bm = _get(o, "occ_bm", lambda: torch.empty(cap, dtype=torch.int32, device=d))
    occ_uid = _get(o, "occ_uid", lambda: torch.empty(cap, dtype=torch.int32, device=d))
    cls = _get(o, "cls", lambda: torch.empty(cap, dtype=torch.uint8, device=d))
    pcls = o.get("prev_cls", None)
    if prev_unique is not None and pcls is None:
        pcls = torch.empty(max(int(prev_cap), 1), dtype=torch.uint8, device=d)
    counts = _get(o, "counts", lambda: torch.empty(4, dtype=torch.int64, device=d))
    tabs = make_row_tables(rows)
    ws = _ws(unique_workspace_size(n_cap, T, W, prev_cap), ws)
    _check("fs_unique_collision_split",
           _c_unique(_ptr(shard_keys), _ptr(shard_bm), _ptr(shard_offsets), int(n_cap), tabs, T,
                     W, _ptr(prev_unique), _ptr(prev_unique_offsets), _ptr(prev_counts),
                     int(prev_cap) if prev_unique
                     is not None else 0, _ptr(uq), _ptr(uo), _ptr(seg), _ptr(occ_bm),
                     _ptr(occ_uid), _ptr(cls), _ptr(pcls) if prev_unique is not None else None,
                     _ptr(counts), _ptr(ws), ws.numel(), _stream(stream)))
    return dict(unique=uq, unique_offsets=uo, seg_offsets=seg, occ_bm=occ_bm, occ_uid=occ_uid,
                cls=cls, prev_cls=pcls, counts=counts)


def collision_workspace_size(n_cap, T, W):
    return int(_c_collide_ws(n_cap, T, W))


def fs_collision_split(uq, n_cap, T, W, prev_unique=None, prev_unique_offsets=None,
                       prev_counts=None, prev_cap=0, prev_cls=None, ws=None, stream=None):
    """The collision split alone on a dedup call's outputs `uq` (its cls and
    counts are rewritten; counts[0] is read). Returns prev_cls (allocated
    when not given and there are previous rows)."""
    d = _dev()
    has = prev_unique is not None
    if has and prev_cls is None:
        prev_cls = torch.empty(max(int(prev_cap), 1), dtype=torch.uint8, device=d)
    ws = _ws(collision_workspace_size(n_cap, T, W), ws)
    _check("fs_collision_split",
           _c_collide(_ptr(uq["unique"]), _ptr(uq["unique_offsets"]), int(n_cap), T, W,
                      _ptr(prev_unique), _ptr(prev_unique_offsets), _ptr(prev_counts),
                      int(prev_cap) if has else 0, _ptr(uq["cls"]),
                      _ptr(prev_cls) if has else None, _ptr(uq["counts"]), _ptr(ws), ws.numel(),
                      _stream(stream)))
    return prev_cls


def _ptr_array(ts):
    arr = (C.c_void_p * len(ts))()
    for i, t in enumerate(ts):
        arr[i] = _ptr(t) if t is not None else None
    return arr


def fs_jagged_lookup(weights, W, uq, n_tok, which=FS_ALL, cls=None, out=None, stream=None):
    """weights: list of [rows, dim] tensors; uq: the split call's outputs."""
    d = _dev()
    T = len(weights)
    if out is None:
        out = [torch.zeros((n_tok, w.shape[1]), dtype=w.dtype, device=d) for w in weights]
    tabs = make_tables(weights)
    cls_t = cls if cls is not None else uq.get("cls")
    _check("fs_jagged_lookup",
           _c_lookup(tabs, T, W, _ptr(uq["unique"]), _ptr(uq["unique_offsets"]),
                     _ptr(uq["seg_offsets"]), _ptr(uq["occ_bm"]), _ptr(uq["occ_uid"]),
                     _ptr(cls_t) if which != FS_ALL else None, which, _ptr_array(out), n_tok,
                     _stream(stream)))
    return out


def fs_ranged_combine(src, bucket, W, dims, dtypes, rows, n_tok, out=None, stream=None):
    """src: device uint8 [n_items, stride] rows in the dispatch's shard-major
    order; bucket: fs_bucketize_permute's outputs; dims / dtypes / rows: per
    table (dtype torch.float32 or torch.bfloat16). Returns one device tensor
    per table, [n_tok, dim] of that dtype (slots no item maps to: zeros when
    the outputs are allocated here)."""
    T = len(dims)
    tabs = (FsTable * T)()
    for t in range(T):
        tabs[t].rows = int(rows[t])
        tabs[t].dim = int(dims[t])
        tabs[t].dtype = FS_F32 if dtypes[t] == torch.float32 else FS_BF16
    if out is None:
        out = [torch.zeros((n_tok, int(dims[t])), dtype=dtypes[t], device=_dev())
               for t in range(T)]
    stride = src.shape[1] * src.element_size() if src.dim() == 2 else 0
    _check("fs_ranged_combine",
           _c_combine(_ptr(src), stride, _ptr(bucket["shard_keys"]), _ptr(bucket["shard_bm"]),
                      _ptr(bucket["shard_offsets"]), W, tabs, T, _ptr_array(out), n_tok,
                      _stream(stream)))
    return out


def keyed_transpose_workspace_size(F, B):
    return int(_c_kt_ws(F, B))


def fs_keyed_transpose(values, lengths, out=None, out_offsets=None, err=None, ws=None,
                       stream=None):
    """values: device 1-D tensor of 4- or 8-byte elements, the feature-major
    concatenation of the lists; lengths: device int32 [F, B] (feature-major).
    Returns (batch-major values, int64 out_offsets [B*F + 1], out_offsets[b*F + f]
    being where list (b, f) starts)."""
    assert lengths.dtype == torch.int32 and lengths.dim() == 2
    F, B = lengths.shape
    n = values.numel()
    if out is None:
        out = torch.empty_like(values)
    if out_offsets is None:
        out_offsets = torch.empty(F * B + 1, dtype=torch.int64, device=_dev())
    ws = _ws(keyed_transpose_workspace_size(F, B), ws)
    _check("fs_keyed_transpose",
           _c_kt(_ptr(values) if n else None, n, values.element_size(), _ptr(lengths), F, B,
                 _ptr(out) if n else None, _ptr(out_offsets), _ptr(err), _ptr(ws),
                 ws.numel() * ws.element_size(), _stream(stream)))
    return out, out_offsets


def reduce_workspace_size(n_tok, max_dim, T=1):
    return int(_c_reduce_ws(n_tok, T, max_dim))


def fs_grad_reduce_update(weights, states, W, grads, n_tok, uq, optim, lr, eps=0.0,
                          which=FS_ALL, cls=None, reduced_out=None, ws=None, stream=None,
                          rows=FS_ROWS_ALL):
    T = len(weights)
    tabs = make_tables(weights, states)
    max_dim = max(w.shape[1] for w in weights)
    ws = _ws(reduce_workspace_size(n_tok, max_dim, T), ws)
    red = _ptr_array(reduced_out) if reduced_out is not None else None
    _check("fs_grad_reduce_update",
           _c_reduce(tabs, T, W, _ptr_array(grads), n_tok, _ptr(uq["unique"]),
                     _ptr(uq["unique_offsets"]), _ptr(uq["seg_offsets"]), _ptr(uq["occ_bm"]),
                     _ptr(uq["occ_uid"]), _ptr(cls) if which != FS_ALL else None, which, rows,
                     FS_RW_ADAGRAD if optim in ("rw_adagrad", FS_RW_ADAGRAD) else FS_SGD,
                     float(lr), float(eps), red, _ptr(ws), ws.numel(), _stream(stream)))


def fs_grad_reduce_update_noalloc(weights, states, W, grads, n_tok, uq, optim, lr, eps=0.0,
                                  which=FS_ALL, cls=None, reduced_out=None, stream=None,
                                  rows=FS_ROWS_ALL):
    """fs_grad_reduce_update without a workspace (the library's fixed per-GPU
    scratch; raises FsError FS_ERR_TOO_LARGE beyond it)."""
    T = len(weights)
    tabs = make_tables(weights, states)
    red = _ptr_array(reduced_out) if reduced_out is not None else None
    _check("fs_grad_reduce_update_noalloc",
           _c_reduce_noalloc(tabs, T, W, _ptr_array(grads), n_tok, _ptr(uq["unique"]),
                             _ptr(uq["unique_offsets"]), _ptr(uq["seg_offsets"]),
                             _ptr(uq["occ_bm"]), _ptr(uq["occ_uid"]),
                             _ptr(cls) if which != FS_ALL else None, which, rows,
                             FS_RW_ADAGRAD if optim in ("rw_adagrad", FS_RW_ADAGRAD) else FS_SGD,
                             float(lr), float(eps), red, _stream(stream)))


# ---------------------------------------------------------------------------- prepared calls


class Prepared:
    """One C call marshalled once for fixed buffers: only the arguments named
    in `var` change between calls (raw values: pointers as ints, counts, the
    stream handle), and `arrays` holds host pointer arrays the caller refills
    in place. For a loop that issues the same call on the same buffers many
    times, where the per-call marshalling of the wrappers above would cost
    more host time than the launches."""

    __slots__ = ("name", "fn", "args", "pos", "arrays")

    def __init__(self, name, fn, args, var, arrays=None):
        self.name, self.fn, self.args = name, fn, list(args)
        self.pos = dict(var)
        self.arrays = arrays or {}

    def __call__(self, **kw):
        a = self.args
        for k, v in kw.items():
            a[self.pos[k]] = v
        rc = self.fn(*a)
        if rc != FS_OK:
            raise FsError(self.name, rc)


def prepare_balance(balancer, W, alpha, perm, rank_offsets, rank_weight, err, ws):
    """fs_balance_fbs / fs_balance_vbs; call with uih=, n=, stream=."""
    if balancer == "fbs":
        args = [None, 0, W, _ptr(perm), _ptr(rank_offsets), _ptr(err), _ptr(ws), ws.numel(), None]
        return Prepared("fs_balance_fbs", _c_balance_fbs, args, dict(uih=0, n=1, stream=8))
    args = [None, 0, W, int(alpha[0]), int(alpha[1]), _ptr(perm), _ptr(rank_offsets),
            _ptr(rank_weight), _ptr(err), _ptr(ws), ws.numel(), None]
    return Prepared("fs_balance_vbs", _c_balance_vbs, args, dict(uih=0, n=1, stream=11))


def prepare_balance_shares(W, alpha, shares, perm, rank_offsets, rank_weight, err, ws):
    """fs_balance_vbs_shares; call with uih=, n=, stream=."""
    args = [None, 0, W, int(alpha[0]), int(alpha[1]), _ptr(shares), _ptr(perm),
            _ptr(rank_offsets), _ptr(rank_weight), _ptr(err), _ptr(ws), ws.numel(), None]
    return Prepared("fs_balance_vbs_shares", _c_balance_shares, args, dict(uih=0, n=1, stream=12))


def prepare_rank_cost(perm, rank_offsets, coef, cost):
    """fs_rank_cost into `cost`; call with uih=, n=, stream=."""
    c2, c1, c0 = (int(c) for c in coef)
    args = [None, 0, _ptr(perm), _ptr(rank_offsets), rank_offsets.numel() - 1, c2, c1, c0,
            _ptr(cost), None]
    return Prepared("fs_rank_cost", _c_rank_cost, args, dict(uih=0, n=1, stream=9))


def prepare_autotune(times, shares, step, tol, err):
    """fs_vbs_autotune on `shares` from `times`; call with stream=."""
    args = [_ptr(times), shares.numel(), int(step[0]), int(step[1]), int(tol[0]), int(tol[1]),
            _ptr(shares), _ptr(err), None]
    return Prepared("fs_vbs_autotune", _c_autotune, args, dict(stream=8))


def prepare_bucketize(rows, perm, rank_offsets, W, out, err, ws):
    """fs_bucketize_permute into `out` (the dict fs_bucketize_permute returns);
    call with ids=, n_tok=, so=, n=, stream=."""
    tabs = make_row_tables(rows)
    args = [None, 0, None, 0, tabs, len(rows), _ptr(perm), _ptr(rank_offsets), W,
            _ptr(out["bal_offsets"]), _ptr(out["shard_keys"]), _ptr(out["shard_bm"]),
            _ptr(out["splits"]), _ptr(out["shard_offsets"]), _ptr(err), _ptr(ws), ws.numel(), None]
    return Prepared("fs_bucketize_permute", _c_bucketize, args,
                    dict(ids=0, n_tok=1, so=2, n=3, stream=17))


def prepare_unique(bucket, rows, W, uq, prev_uq, prev_cls, ws):
    """fs_unique_collision_split of `bucket` into `uq` against `prev_uq` (None:
    first iteration); call with n_cap=, prev_cap=, stream=."""
    tabs = make_row_tables(rows)
    has = prev_uq is not None
    args = [_ptr(bucket["shard_keys"]), _ptr(bucket["shard_bm"]), _ptr(bucket["shard_offsets"]),
            0, tabs, len(rows), W, _ptr(prev_uq["unique"]) if has else None,
            _ptr(prev_uq["unique_offsets"]) if has else None,
            _ptr(prev_uq["counts"]) if has else None, 0, _ptr(uq["unique"]),
            _ptr(uq["unique_offsets"]), _ptr(uq["seg_offsets"]), _ptr(uq["occ_bm"]),
            _ptr(uq["occ_uid"]), _ptr(uq["cls"]), _ptr(prev_cls) if has else None,
            _ptr(uq["counts"]), _ptr(ws), ws.numel(), None]
    return Prepared("fs_unique_collision_split", _c_unique, args,
                    dict(n_cap=3, prev_cap=10, stream=21))


def prepare_collision(uq, T, W, prev_uq, prev_cls, ws):
    """fs_collision_split of the dedup result `uq` against `prev_uq` (None:
    every row exclusive); call with n_cap=, prev_cap=, stream=."""
    has = prev_uq is not None
    args = [_ptr(uq["unique"]), _ptr(uq["unique_offsets"]), 0, T, W,
            _ptr(prev_uq["unique"]) if has else None,
            _ptr(prev_uq["unique_offsets"]) if has else None,
            _ptr(prev_uq["counts"]) if has else None, 0, _ptr(uq["cls"]),
            _ptr(prev_cls) if has else None, _ptr(uq["counts"]), _ptr(ws), ws.numel(), None]
    return Prepared("fs_collision_split", _c_collide, args, dict(n_cap=2, prev_cap=8, stream=14))


def prepare_lookup(weights, W, uq, out, which=FS_ALL, cls=None):
    """fs_jagged_lookup into the tensors `out` (one per table, at least n_tok
    rows); call with n_tok=, stream=."""
    args = [make_tables(weights), len(weights), W, _ptr(uq["unique"]),
            _ptr(uq["unique_offsets"]), _ptr(uq["seg_offsets"]), _ptr(uq["occ_bm"]),
            _ptr(uq["occ_uid"]), _ptr(cls) if which != FS_ALL else None, which, _ptr_array(out),
            0, None]
    return Prepared("fs_jagged_lookup", _c_lookup, args, dict(n_tok=11, stream=12))


def prepare_update(weights, states, W, uq, optim, lr, eps, which, cls, ws):
    """fs_grad_reduce_update with the gradient pointers in arrays["grads"]
    (set them before each call); call with n_tok=, stream= (and rows=, all
    rows unless given)."""
    grads = (C.c_void_p * len(weights))()
    args = [make_tables(weights, states), len(weights), W, grads, 0, _ptr(uq["unique"]),
            _ptr(uq["unique_offsets"]), _ptr(uq["seg_offsets"]), _ptr(uq["occ_bm"]),
            _ptr(uq["occ_uid"]), _ptr(cls) if which != FS_ALL else None, which, FS_ROWS_ALL,
            FS_RW_ADAGRAD if optim in ("rw_adagrad", FS_RW_ADAGRAD) else FS_SGD, float(lr),
            float(eps), None, _ptr(ws), ws.numel(), None]
    return Prepared("fs_grad_reduce_update", _c_reduce, args, dict(n_tok=4, rows=12, stream=19),
                    arrays=dict(grads=grads))
