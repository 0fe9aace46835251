"""The C ABI without a GPU: the library loads, exports every call the header
declares, answers host-only queries and rejects bad arguments on the host
(before any launch) with the documented return codes."""

import ctypes as C
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fs_sparse.h")


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:int|size_t|const char\*)\s+(fs_\w+)\s*\(", src,
                                 flags=re.M)))


@pytest.fixture(scope="module")
def L():
    from jagged_embedding_sparse_amd import lib
    return lib


def test_every_declared_symbol_is_exported(L):
    names = _declared()
    assert len(names) >= 12
    raw = C.CDLL(L.LIB_PATH)
    for n in names:
        assert hasattr(raw, n), n
    assert sorted(L.EXPORTED) == names


def test_strerror_and_version(L):
    assert L.strerror(0) == "ok"
    for code in (-1, -2, -3, -4):
        assert L.strerror(code) and L.strerror(code) != "unknown error"
    assert L.strerror(-99) == "unknown error"
    assert L.version() >= 1


def test_workspace_queries_are_host_only_and_monotone(L):
    assert L.balance_workspace_size(4096, 512) >= 4096 * 16
    # per-tile shard counts: grows with the batch, the tables and W
    a = L.bucketize_workspace_size(1 << 20, 4096, 1, 512)
    assert 0 < a < L.bucketize_workspace_size(1 << 22, 4096, 1, 512)
    assert a >= 4 * 513 * 512
    assert a < L.bucketize_workspace_size(1 << 20, 4096, 2, 512) < \
        L.bucketize_workspace_size(1 << 20, 4096, 2, 1024)
    assert L.unique_workspace_size(1 << 22, 1, 512) >= 16 * (1 << 22)
    # the collision split needs no space per previous row
    assert L.unique_workspace_size(1 << 20, 1, 512, prev_cap=1 << 24) == \
        L.unique_workspace_size(1 << 20, 1, 512, prev_cap=1 << 20)
    assert L.reduce_workspace_size(1 << 20, 256) > L.reduce_workspace_size(1 << 20, 64)
    # a region of partial sums per table: the tables' rows run side by side
    one = L.reduce_workspace_size(1 << 20, 128) - 256
    assert L.reduce_workspace_size(1 << 20, 128, T=4) - 256 == 4 * one


def test_workspace_sized_for_a_capacity_serves_every_smaller_call(L):
    """Each call rejects a workspace below its query's size for the call's own
    sizes, so a workspace sized for a capacity must be at least the query of
    every smaller size: the queries never decrease. The update's long-row
    chunk grows at 2 621 440 and 5 242 880 occurrences and the balance's
    slice count falls as the batch grows; both are checked around every such
    step."""
    for D in (64, 128, 1024):
        prev = 0
        for n in list(range(1, 4096)) + [x + d for x in (2_621_440, 5_242_880)
                                         for d in range(-600, 600)] + [1 << 23, 1 << 24]:
            sz = L.reduce_workspace_size(n, D)
            assert sz >= prev, (n, D)
            prev = sz
        cap = L.reduce_workspace_size(5_300_000, D)
        for n in (2_621_439, 2_621_440, 5_242_879, 5_242_880, 5_200_000):
            assert L.reduce_workspace_size(n, D) <= cap, (n, D)
    prev = 0
    for n in range(0, L.FS_MAX_SAMPLES + 1):
        sz = L.balance_workspace_size(n, 64)
        assert sz >= prev, n
        prev = sz
    for n in (1, 1000, 5000, 16384):
        assert L.bucketize_workspace_size(n, 64, 2, 64) <= L.bucketize_workspace_size(
            n + 1, 64, 2, 64)
        assert L.unique_workspace_size(n, 2, 64) <= L.unique_workspace_size(n + 1, 2, 64)


def test_noalloc_update_rejects_sizes_beyond_its_scratch(L):
    """The allocation-free update checks on the host that the batch's partial
    sums fit its fixed scratch: FS_ERR_TOO_LARGE past the limit, and the
    other argument checks as the workspace-taking call. Nothing is launched."""
    F = 0x1000
    tabs = _tables(L, [(5000, 1024, L.FS_F32, False)])
    grads = (C.c_void_p * 1)(F)
    call = L._c_reduce_noalloc
    # 524 160 occurrences at 1024 columns fit; one more does not
    assert L.reduce_workspace_size(524_160, 1024) <= L.FS_NOALLOC_SCRATCH_BYTES
    assert L.reduce_workspace_size(524_161, 1024) > L.FS_NOALLOC_SCRATCH_BYTES
    assert call(tabs, 1, 4, grads, 524_161, F, F, F, F, F, None, L.FS_ALL, L.FS_ROWS_ALL, L.FS_SGD, 0.1, 0.0,
                None, None) == L.FS_ERR_TOO_LARGE
    assert call(tabs, 1, 4, grads, 1 << 25, F, F, F, F, F, None, L.FS_ALL, L.FS_ROWS_ALL, L.FS_SGD, 0.1, 0.0,
                None, None) == L.FS_ERR_TOO_LARGE
    assert call(tabs, 1, 4, grads, 1000, F, F, F, F, F, None, 7, L.FS_ROWS_ALL, L.FS_SGD, 0.1, 0.0,
                None, None) == L.FS_ERR_INVALID_ARG
    assert call(tabs, 1, 4, grads, 1000, None, F, F, F, F, None, L.FS_ALL, L.FS_ROWS_ALL, L.FS_SGD, 0.1, 0.0,
                None, None) == L.FS_ERR_INVALID_ARG
    for rows in (0, 4, -1):  # the row parts are a mask of FS_ROWS_FEW and FS_ROWS_MANY
        assert call(tabs, 1, 4, grads, 1000, F, F, F, F, F, None, L.FS_ALL, rows, L.FS_SGD, 0.1,
                    0.0, None, None) == L.FS_ERR_INVALID_ARG
    assert L.strerror(L.FS_ERR_TOO_LARGE) != "unknown error"


FAKE = 0x1000  # never dereferenced: every case below fails host-side validation


def test_balance_rejects(L):
    f = L._c_balance_fbs
    assert f(None, 10, 4, None, None, None, None, 0, None) == L.FS_ERR_INVALID_ARG
    assert f(FAKE, 10, 0, FAKE, FAKE, None, None, 0, None) == L.FS_ERR_INVALID_ARG
    assert f(FAKE, 10, L.FS_MAX_RANKS + 1, FAKE, FAKE, None, None, 0, None) == L.FS_ERR_INVALID_ARG
    assert f(FAKE, L.FS_MAX_SAMPLES + 1, 4, FAKE, FAKE, None, None, 0, None) == \
        L.FS_ERR_INVALID_ARG
    # the sort's per-slice counts need the workspace
    assert f(FAKE, 10, 4, FAKE, FAKE, None, None, 0, None) == L.FS_ERR_WORKSPACE
    assert f(FAKE, 10, 4, FAKE, FAKE, None, FAKE, 8, None) == L.FS_ERR_WORKSPACE
    v = L._c_balance_vbs
    assert v(FAKE, 10, 4, 1, 3, FAKE, FAKE, None, None, FAKE, 1 << 20, None) == \
        L.FS_ERR_UNSUPPORTED
    assert v(FAKE, 10, 4, 5, 2, FAKE, FAKE, None, None, FAKE, 1 << 20, None) == \
        L.FS_ERR_UNSUPPORTED
    assert v(FAKE, 10, 4, 3, 2, FAKE, FAKE, None, None, FAKE, 8, None) == L.FS_ERR_WORKSPACE


def _tables(L, specs):
    arr = (L.FsTable * len(specs))()
    for i, (rows, dim, dt, st) in enumerate(specs):
        arr[i].weights = FAKE
        arr[i].state = FAKE + (1 << 20) if st else None
        arr[i].rows = rows
        arr[i].dim = dim
        arr[i].dtype = dt
    return arr


def test_bucketize_rejects(L):
    f = L._c_bucketize
    tab = _tables(L, [(1000, 64, L.FS_F32, False)])
    args = lambda T, ws_bytes, tabs=tab: f(FAKE, 100, FAKE, 8, tabs, T, FAKE, FAKE, 4, FAKE, FAKE,
                                           FAKE, FAKE, FAKE, None, FAKE, ws_bytes, None)
    assert args(0, 1 << 20) == L.FS_ERR_INVALID_ARG
    assert args(L.FS_MAX_TABLES + 1, 1 << 20) == L.FS_ERR_INVALID_ARG
    assert args(1, 16) == L.FS_ERR_WORKSPACE
    big = _tables(L, [(1 << 31, 64, L.FS_F32, False), (1 << 31, 64, L.FS_F32, False),
                      (8, 64, L.FS_F32, False)])
    assert args(3, 1 << 30, big) == L.FS_ERR_UNSUPPORTED  # key space beyond 2^32
    zero = _tables(L, [(0, 64, L.FS_F32, False)])
    assert args(1, 1 << 20, zero) == L.FS_ERR_INVALID_ARG


def test_unique_rejects(L):
    f = L._c_unique
    tab = _tables(L, [(1000, 64, L.FS_F32, False)])
    call = lambda prev_u, prev_o, prev_c, ws: f(FAKE, FAKE, FAKE, 100, tab, 1, 4, prev_u, prev_o,
                                                prev_c, 100, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                                                FAKE, FAKE, FAKE, ws, None)
    # the previous iteration's arrays come all three or none
    assert call(FAKE, FAKE, None, 1 << 20) == L.FS_ERR_INVALID_ARG
    assert call(FAKE, None, FAKE, 1 << 20) == L.FS_ERR_INVALID_ARG
    assert call(None, FAKE, None, 1 << 20) == L.FS_ERR_INVALID_ARG
    assert call(None, None, None, 64) == L.FS_ERR_WORKSPACE


def test_lookup_and_update_reject_unsupported_rows(L):
    lk = L._c_lookup
    outs = (C.c_void_p * 1)(FAKE)
    for dim, dt in [(48, L.FS_F32), (100, L.FS_BF16), (8, L.FS_F32)]:
        tab = _tables(L, [(1000, dim, dt, False)])
        assert lk(tab, 1, 4, FAKE, FAKE, FAKE, FAKE, FAKE, None, L.FS_ALL, outs, 10, None) == \
            L.FS_ERR_UNSUPPORTED
    tab = _tables(L, [(1000, 64, L.FS_F32, False)])
    assert lk(tab, 1, 4, FAKE, FAKE, FAKE, FAKE, FAKE, None, L.FS_COLLISION, outs, 10, None) == \
        L.FS_ERR_INVALID_ARG  # class filter without classes
    assert lk(tab, 1, 4, FAKE, FAKE, FAKE, FAKE, FAKE, None, 7, outs, 10, None) == \
        L.FS_ERR_INVALID_ARG
    ru = L._c_reduce
    grads = (C.c_void_p * 1)(FAKE)
    for dim in (96, 32, 2048):
        tab = _tables(L, [(1000, dim, L.FS_F32, True)])
        assert ru(tab, 1, 4, grads, 10, FAKE, FAKE, FAKE, FAKE, FAKE, None, L.FS_ALL, L.FS_ROWS_ALL,
                  L.FS_SGD, 0.1, 0.0, None, FAKE, 1 << 30, None) == L.FS_ERR_UNSUPPORTED
    tab = _tables(L, [(1000, 128, L.FS_F32, False)])  # Adagrad needs state
    assert ru(tab, 1, 4, grads, 10, FAKE, FAKE, FAKE, FAKE, FAKE, None, L.FS_ALL, L.FS_ROWS_ALL,
              L.FS_RW_ADAGRAD, 0.1, 0.0, None, FAKE, 1 << 30, None) == L.FS_ERR_INVALID_ARG
    tab = _tables(L, [(1000, 128, L.FS_F32, True)])
    assert ru(tab, 1, 4, grads, 10, FAKE, FAKE, FAKE, FAKE, FAKE, None, L.FS_ALL, L.FS_ROWS_ALL,
              L.FS_RW_ADAGRAD, 0.1, 0.0, None, FAKE, 8, None) == L.FS_ERR_WORKSPACE


def test_collision_split_rejects(L):
    """The standalone collision split validates on the host: sizes, the
    three previous-row pointers together, prev_cls with previous rows, and
    its workspace."""
    f = L._c_collide
    ws_need = L.collision_workspace_size(1000, 2, 8)
    names = ["unique", "unique_offsets", "n_cap", "T", "W", "prev_unique", "prev_off",
             "prev_counts", "prev_cap", "cls", "prev_cls", "counts", "ws", "ws_bytes", "stream"]
    ok = [FAKE, FAKE, 1000, 2, 8, None, None, None, 0, FAKE, None, FAKE, FAKE, ws_need, None]

    def call(**kw):
        a = list(ok)
        for k, v in kw.items():
            a[names.index(k)] = v
        return f(*a)
    bad = L.FS_ERR_INVALID_ARG
    assert call(counts=None) == bad
    assert call(unique_offsets=None) == bad
    assert call(cls=None) == bad
    assert call(n_cap=-1) == bad
    assert call(T=0) == bad and call(T=L.FS_MAX_TABLES + 1) == bad
    assert call(W=0) == bad and call(W=L.FS_MAX_RANKS + 1) == bad
    assert call(prev_unique=FAKE) == bad  # without its offsets and counts
    assert call(prev_unique=FAKE, prev_off=FAKE, prev_counts=FAKE, prev_cap=10) == bad
    assert call(ws_bytes=ws_need - 1) == L.FS_ERR_WORKSPACE
    assert call(ws=None) == L.FS_ERR_WORKSPACE
    assert L.collision_workspace_size(1 << 20, 2, 8) >= ws_need


def test_lookup_and_update_reject_bad_table_layouts(L):
    """Row strides and in-row states: checked on the host before any launch."""
    lk, ru = L._c_lookup, L._c_reduce
    outs = (C.c_void_p * 1)(FAKE)
    grads = (C.c_void_p * 1)(FAKE)

    def tab(stride=0, state_stride=0, weights=FAKE, state=None, dim=128, dt=None):
        t = _tables(L, [(1000, dim, L.FS_BF16 if dt is None else dt, False)])
        t[0].weights, t[0].state = weights, state
        t[0].stride, t[0].state_stride = stride, state_stride
        return t

    def look(t):
        return lk(t, 1, 4, FAKE, FAKE, FAKE, FAKE, FAKE, None, L.FS_ALL, outs, 10, None)

    def upd(t, optim=None):
        return ru(t, 1, 4, grads, 10, FAKE, FAKE, FAKE, FAKE, FAKE, None, L.FS_ALL, L.FS_ROWS_ALL,
                  L.FS_RW_ADAGRAD if optim is None else optim, 0.1, 0.0, None, FAKE, 8, None)
    bad = L.FS_ERR_INVALID_ARG
    # bf16 x 128 = 256-byte rows
    assert look(tab(stride=264)) == bad             # not a multiple of 16
    assert look(tab(stride=240)) == bad             # shorter than the row
    assert look(tab(weights=FAKE + 8)) == bad       # weights not 16-byte aligned
    assert upd(tab(stride=272, state=FAKE + (1 << 20), state_stride=2)) == bad
    assert upd(tab(stride=272, state=FAKE + (1 << 20) + 2)) == bad  # state not 4-aligned
    # a state inside the row's stride that overlaps the row's weights
    assert upd(tab(stride=272, state=FAKE + 252, state_stride=272)) == bad
    assert upd(tab(stride=272, state=FAKE + 270, state_stride=272)) == bad  # past the stride
    # valid layouts get past the layout check (and stop at the workspace)
    ws = L.FS_ERR_WORKSPACE
    assert upd(tab(stride=272, state=FAKE + 256, state_stride=272)) == ws
    assert upd(tab(stride=272, state=FAKE + 268, state_stride=272)) == ws
    assert upd(tab(state=FAKE + (1 << 20))) == ws
    # SGD ignores the state's layout
    assert upd(tab(stride=272, state=FAKE + 252, state_stride=2), optim=L.FS_SGD) == ws


def test_step_rejects_unknown_lookup_schedule():
    from jagged_embedding_sparse_amd.step import SparseStep
    with pytest.raises(ValueError):
        SparseStep(None, [], [], 1, lookup="eager")
    with pytest.raises(ValueError):
        SparseStep(None, [], [], 1, lookahead=4)
    with pytest.raises(ValueError):  # the prioritized schedule needs the index stages ahead
        SparseStep(None, [], [], 1, lookahead=1, schedule="prioritized")
    with pytest.raises(ValueError):  # graph replay needs the index stages ahead
        SparseStep(None, [], [], 1, lookahead=1, graph=True)
    from jagged_embedding_sparse_amd import synth
    with pytest.raises(ValueError):  # AutoTune moves VBS shares: no FBS
        SparseStep(synth.workload(1), [], [], 1, autotune={})


def test_prepared_calls_match_the_c_signatures(L, monkeypatch):
    """Each prepared call holds exactly as many arguments as its C function
    takes, and the per-call arguments sit at placeholder positions (checked
    without a GPU: pointers are stand-in integers, nothing is called)."""
    import torch
    monkeypatch.setattr(L, "_ptr", lambda t: None if t is None else 0x1000)
    monkeypatch.setattr(L, "_rows_ptr", lambda t: (0x1000, 0))
    monkeypatch.setattr(L, "_state_ptr", lambda t: (0x2000, 0))
    t = torch.zeros(4)
    ws = torch.zeros(16, dtype=torch.uint8)
    weights = [torch.zeros((8, 64)), torch.zeros((8, 128), dtype=torch.bfloat16)]
    bucket = dict(bal_offsets=t, shard_keys=t, shard_bm=t, splits=t, shard_offsets=t)
    uq = dict(unique=t, unique_offsets=t, seg_offsets=t, occ_bm=t, occ_uid=t, cls=t, counts=t)
    calls = [
        L.prepare_balance("fbs", 4, (3, 2), t, t, t, t, ws),
        L.prepare_balance("vbs", 4, (3, 2), t, t, t, t, ws),
        L.prepare_bucketize([8, 8], t, t, 4, bucket, t, ws),
        L.prepare_unique(bucket, [8, 8], 4, uq, None, None, ws),
        L.prepare_unique(bucket, [8, 8], 4, uq, uq, t, ws),
        L.prepare_lookup(weights, 4, uq, [t, t]),
        L.prepare_lookup(weights, 4, uq, [t, t], L.FS_COLLISION, t),
        L.prepare_update(weights, [t, t], 4, uq, "rw_adagrad", 0.1, 1e-8, L.FS_ALL, None, ws),
        L.prepare_collision(uq, 2, 4, None, None, ws),
        L.prepare_collision(uq, 2, 4, uq, t, ws),
        L.prepare_balance_shares(4, (3, 2), t, t, t, t, t, ws),
        L.prepare_rank_cost(t, torch.zeros(5), (1, 64, 0), t),
        L.prepare_autotune(t, t, (1, 16), (1, 50), t),
    ]
    for p in calls:
        assert len(p.args) == len(p.fn.argtypes), p.name
        for name, i in p.pos.items():
            assert 0 <= i < len(p.args), (p.name, name)
            if name == "rows":  # defaults to every row, right after the class filter
                assert p.args[i] == L.FS_ROWS_ALL and p.args[i - 1] == L.FS_ALL, p.name
            else:
                assert p.args[i] in (None, 0), (p.name, name)
        assert p.pos["stream"] == len(p.args) - 1, p.name


def test_combine_rejects_bad_rows_and_strides(L):
    cb = L._c_combine
    outs = (C.c_void_p * 2)(FAKE, FAKE)

    def call(dims, stride, src=FAKE, T=None):
        tab = _tables(L, [(1000, d, L.FS_F32, False) for d in dims])
        return cb(src, stride, FAKE, FAKE, FAKE, 4, tab, T if T is not None else len(dims), outs,
                  10, None)
    assert call([48], 256) == L.FS_ERR_UNSUPPORTED      # 192-byte rows
    assert call([64, 128], 256) == L.FS_ERR_INVALID_ARG  # stride below the 512-byte row
    assert call([64], 264) == L.FS_ERR_INVALID_ARG       # stride not a multiple of 16
    assert call([64], 256, src=FAKE + 8) == L.FS_ERR_INVALID_ARG  # src not 16-byte aligned
    assert call([64], 256, T=0) == L.FS_ERR_INVALID_ARG


def test_keyed_transpose_rejects(L):
    kt = L._c_kt
    ws_n = L.keyed_transpose_workspace_size(4, 6)
    assert ws_n >= 8 * 24 and L.keyed_transpose_workspace_size(40, 600) > ws_n
    assert L.keyed_transpose_workspace_size(-1, 3) == 0

    def call(n=100, eb=8, F=4, B=6, vals=FAKE, outv=FAKE, lens=FAKE, offs=FAKE, ws=FAKE,
             ws_bytes=ws_n):
        return kt(vals, n, eb, lens, F, B, outv, offs, None, ws, ws_bytes, None)
    assert call(eb=2) == L.FS_ERR_UNSUPPORTED
    assert call(eb=16) == L.FS_ERR_UNSUPPORTED
    assert call(F=-1) == L.FS_ERR_INVALID_ARG
    assert call(F=1 << 16, B=1 << 15) == L.FS_ERR_INVALID_ARG  # F * B >= 2^31
    assert call(n=-1) == L.FS_ERR_INVALID_ARG
    assert call(offs=None) == L.FS_ERR_INVALID_ARG
    assert call(lens=None) == L.FS_ERR_INVALID_ARG
    assert call(vals=None) == L.FS_ERR_INVALID_ARG
    assert call(vals=FAKE + 4) == L.FS_ERR_INVALID_ARG       # 8-byte elements, 4-aligned
    assert call(outv=FAKE + 2, eb=4) == L.FS_ERR_INVALID_ARG
    assert call(ws_bytes=ws_n - 1) == L.FS_ERR_WORKSPACE
    assert call(ws=None) == L.FS_ERR_WORKSPACE


def test_autotune_calls_reject(L):
    ws_n = L.balance_workspace_size(100, 8)
    sh = L._c_balance_shares

    def cut(shares=FAKE, a=(3, 2), ws_bytes=ws_n, W=8):
        return sh(FAKE, 100, W, a[0], a[1], shares, FAKE, FAKE, None, None, FAKE, ws_bytes, None)
    assert cut(shares=None) == L.FS_ERR_INVALID_ARG
    assert cut(a=(1, 3)) == L.FS_ERR_UNSUPPORTED
    assert cut(W=0) == L.FS_ERR_INVALID_ARG
    assert cut(ws_bytes=ws_n - 1) == L.FS_ERR_WORKSPACE
    rc = L._c_rank_cost

    def cost(c=(1, 0, 0), n=100, W=8, perm=FAKE):
        return rc(FAKE, n, perm, FAKE, W, c[0], c[1], c[2], FAKE, None)
    assert cost(c=(-1, 0, 0)) == L.FS_ERR_INVALID_ARG
    assert cost(c=(1, 1 << 17, 0)) == L.FS_ERR_INVALID_ARG
    assert cost(n=L.FS_MAX_SAMPLES + 1) == L.FS_ERR_INVALID_ARG
    assert cost(W=L.FS_MAX_RANKS + 1) == L.FS_ERR_INVALID_ARG
    assert cost(perm=None) == L.FS_ERR_INVALID_ARG
    at = L._c_autotune

    def tune(step=(1, 16), tol=(1, 20), W=8, shares=FAKE):
        return at(FAKE, W, step[0], step[1], tol[0], tol[1], shares, None, None)
    assert tune(step=(2, 1)) == L.FS_ERR_INVALID_ARG
    assert tune(step=(1, 0)) == L.FS_ERR_INVALID_ARG
    assert tune(step=(1, (1 << 20) + 1)) == L.FS_ERR_INVALID_ARG
    assert tune(tol=(3, 2)) == L.FS_ERR_INVALID_ARG
    assert tune(tol=(-1, 2)) == L.FS_ERR_INVALID_ARG
    assert tune(W=0) == L.FS_ERR_INVALID_ARG
    assert tune(shares=None) == L.FS_ERR_INVALID_ARG
