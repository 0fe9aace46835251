"""Per-call parity of the HIP path against the CPU oracle on seeded inputs.

Index outputs are compared bit for bit; reduced gradients and updated rows
to the tolerance the fp32 / bf16 arithmetic leaves (1e-5 fp32, 1e-2 bf16,
relative to the size of the combined values). Sizes span several tiles and
a ragged tail; edge cases cover empty and tiny batches, W > N, zero-token
samples, dropped IDs, and hot rows long enough to cross many chunks.
"""

import numpy as np
import pytest
import torch

from harness import host, snapshot_stores, store_vals_f32, rel_err_rows
from jagged_embedding_sparse_amd import lib, synth
from oracle import oracle as O

pytestmark = pytest.mark.gpu


def cu(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def say(*a):
    print("[case]", *a, flush=True)


# ----------------------------------------------------------------------------- balance

# batches of at most 1024 samples take the one-workgroup balance, larger ones
# the multi-workgroup sort: both sides of the limit, at the largest W too
BAL_CASES = [(64, 4), (512, 16), (1024, 64), (2048, 256), (4096, 512), (0, 3), (1, 1), (7, 8),
             (10, 4), (6, 4), (100, 1024), (16384, 1024), (4097, 512), (1025, 3),
             (1024, 1024), (1000, 7)]


def _lengths(N, seed, kind):
    rng = np.random.default_rng(seed)
    if kind == "ties":
        return rng.integers(1, 40, size=N).astype(np.int32)
    if kind == "zero":
        return rng.integers(0, 3, size=N).astype(np.int32)
    return np.minimum(np.ceil(rng.lognormal(6.5, 1.3, size=N)), 32768).astype(np.int32)


@pytest.mark.parametrize("kind", ["ties", "skew", "zero"])
@pytest.mark.parametrize("N,W", BAL_CASES)
def test_fbs_parity(N, W, kind):
    say("fbs", N, W, kind)
    L = _lengths(N, N + W, kind)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    perm, ro = lib.fs_balance_fbs(cu(L), W, err=err)
    operm, oro = O.balance_fbs(L, W)
    torch.cuda.synchronize()
    assert np.array_equal(host(ro), oro)
    assert np.array_equal(host(perm), operm)
    assert int(err.item()) == 0


@pytest.mark.parametrize("alpha", [(3, 2), (2, 1), (1, 1), (0, 1), (1, 2)])
@pytest.mark.parametrize("N,W", BAL_CASES)
def test_vbs_parity(N, W, alpha):
    say("vbs", N, W, alpha)
    L = _lengths(N, 3 * N + W, "skew")
    perm, ro, rw = lib.fs_balance_vbs(cu(L), W, alpha)
    operm, oro, orw = O.balance_vbs(L, W, alpha)
    torch.cuda.synchronize()
    assert np.array_equal(host(perm), operm)
    assert np.array_equal(host(ro), oro)
    assert np.array_equal(host(rw), orw)


@pytest.mark.parametrize("N", [6, 2000])  # the one-workgroup balance and the larger sort
def test_balance_length_range_is_clamped_and_flagged(N):
    say("len-range", N)
    L = np.random.default_rng(N).integers(0, 3000, N).astype(np.int32)
    L[:6] = [5, -3, 70000, 12, 0, 65535]
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    perm, ro, rw = lib.fs_balance_vbs(cu(L), 2, (2, 1), err=err)
    operm, oro, orw = O.balance_vbs(np.clip(L, 0, 65535), 2, (2, 1))
    torch.cuda.synchronize()
    assert int(err.item()) & lib.FS_EF_LEN_RANGE
    assert np.array_equal(host(perm), operm) and np.array_equal(host(rw), orw)
    err.zero_()
    perm, ro = lib.fs_balance_fbs(cu(L), 2, err=err)
    operm, oro = O.balance_fbs(np.clip(L, 0, 65535), 2)
    torch.cuda.synchronize()
    assert int(err.item()) & lib.FS_EF_LEN_RANGE
    assert np.array_equal(host(perm), operm) and np.array_equal(host(ro), oro)


@pytest.mark.parametrize("k", [1, 2, 3, 4, 5])
def test_balance_workload_lengths(k):
    w = synth.WORKLOADS[k]
    for it in range(3):
        say("bal-workload", k, it)
        L = synth.draw_lengths(w, k, it)
        perm, ro = lib.fs_balance_fbs(cu(L), w.world)
        operm, oro = O.balance_fbs(L, w.world)
        vperm, vro, vrw = lib.fs_balance_vbs(cu(L), w.world, w.alpha)
        ovp, ovro, ovrw = O.balance_vbs(L, w.world, w.alpha)
        torch.cuda.synchronize()
        assert np.array_equal(host(perm), operm) and np.array_equal(host(ro), oro)
        assert np.array_equal(host(vperm), ovp) and np.array_equal(host(vro), ovro)
        assert np.array_equal(host(vrw), ovrw)


# ----------------------------------------------------------------------------- VBS AutoTune

SHARE_CASES = [(64, 4), (1024, 64), (4096, 512), (16384, 1024), (0, 3), (1, 1), (7, 8), (100, 1024),
               (4097, 512)]


def _shares(rng, W, kind):
    if kind == "equal":
        return np.full(W, 1 << 16, np.int64)
    if kind == "wide":  # a few ranks with huge shares, many with tiny ones
        x = rng.integers(1, 50, W).astype(np.int64)
        x[rng.random(W) < 0.1] = 1 << 40
        return x
    return rng.integers(1, 1 << 20, W).astype(np.int64)


@pytest.mark.parametrize("kind", ["equal", "random", "wide"])
@pytest.mark.parametrize("alpha", [(3, 2), (1, 1), (2, 1)])
@pytest.mark.parametrize("N,W", SHARE_CASES)
def test_vbs_shares_parity(N, W, alpha, kind):
    say("vbs shares", N, W, alpha, kind)
    rng = np.random.default_rng(N + 3 * W)
    L = _lengths(N, N + W, "skew")
    sh = _shares(rng, W, kind)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    perm, ro, rw = lib.fs_balance_vbs_shares(cu(L), W, cu(sh), alpha, err=err)
    operm, oro, orw = O.balance_vbs_shares(L, W, sh, alpha)
    torch.cuda.synchronize()
    assert np.array_equal(host(ro), oro)
    assert np.array_equal(host(perm), operm)
    assert np.array_equal(host(rw), orw)
    assert int(err.item()) == 0
    if kind == "equal":  # the same cuts as the plain VBS call
        _, ro2, rw2 = lib.fs_balance_vbs(cu(L), W, alpha)
        torch.cuda.synchronize()
        assert np.array_equal(host(ro2), oro) and np.array_equal(host(rw2), orw)


def test_vbs_shares_out_of_range_are_clamped_and_flagged():
    L = _lengths(3000, 9, "skew")
    sh = np.array([0, -5, 1, 7, (1 << 40) + 1, 1 << 62, 3, 1], np.int64)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    perm, ro, rw = lib.fs_balance_vbs_shares(cu(L), 8, cu(sh), (3, 2), err=err)
    clamped = np.clip(sh, 1, 1 << 40)
    operm, oro, orw = O.balance_vbs_shares(L, 8, clamped, (3, 2))
    torch.cuda.synchronize()
    assert int(err.item()) == lib.FS_EF_SHAPE
    assert np.array_equal(host(ro), oro) and np.array_equal(host(rw), orw)


@pytest.mark.parametrize("coef", [(1, 0, 0), (3, 700, 50000), (0, 1, 0), (65536, 65536, 65536)])
@pytest.mark.parametrize("N,W", [(4096, 512), (16384, 1024), (1000, 7), (0, 5), (5, 64)])
def test_rank_cost_parity(N, W, coef):
    say("rank cost", N, W, coef)
    L = _lengths(N, N * 5 + W, "skew")
    perm, ro, _ = lib.fs_balance_vbs(cu(L), W, (1, 1))
    cost = lib.fs_rank_cost(cu(L), perm, ro, coef)
    torch.cuda.synchronize()
    ref = O.rank_cost(L, host(perm), host(ro), coef)
    assert np.array_equal(host(cost), ref)


@pytest.mark.parametrize("step,tol", [((1, 16), (1, 20)), ((1, 2), (0, 1)), ((0, 1), (1, 1)),
                                      ((1, 1), (1, 1000)), ((3, 1 << 20), (1 << 19, 1 << 20))])
@pytest.mark.parametrize("W", [1, 2, 64, 513, 1024])
def test_vbs_autotune_parity(W, step, tol):
    say("autotune", W, step, tol)
    rng = np.random.default_rng(W * 31 + step[1])
    times = rng.integers(0, 1 << 40, W).astype(np.int64)
    times[rng.random(W) < 0.2] = int(np.median(times))  # exact ties with other ranks
    sh = rng.integers(1, 1 << 40, W).astype(np.int64)
    sh[rng.random(W) < 0.1] = 1
    d_sh = cu(sh)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    lib.fs_vbs_autotune(cu(times), d_sh, step, tol, err=err)
    torch.cuda.synchronize()
    assert np.array_equal(host(d_sh), O.vbs_autotune(times, sh, step, tol))
    assert int(err.item()) == 0


def test_vbs_autotune_clamps_and_flags():
    times = np.array([-4, 10, (1 << 52) + 9, 30], np.int64)
    sh = np.array([0, 1 << 41, 100, 100], np.int64)
    d_sh = cu(sh)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    lib.fs_vbs_autotune(cu(times), d_sh, (1, 10), (1, 20), err=err)
    torch.cuda.synchronize()
    ref = O.vbs_autotune(np.clip(times, 0, 1 << 52), np.clip(sh, 1, 1 << 40), (1, 10), (1, 20))
    assert np.array_equal(host(d_sh), ref)
    assert int(err.item()) == lib.FS_EF_SHAPE


@pytest.mark.parametrize("k", [3, 4])
def test_autotune_loop_on_device(k):
    """Forty iterations of cut -> modelled cost -> AutoTune on the device,
    with no host synchronisation between them, replayed by the oracle: every
    iteration's cuts and shares bit-exact. On workload 3 the cost spread
    shrinks; workload 4's (weights L^2, 256 ranks for 2048 samples) is set
    by single samples, which no share can split."""
    w = synth.workload(k)
    bat = synth.Batches(w, k)
    W = w.world
    alpha = w.alpha
    sh = torch.full((W,), 1 << 16, dtype=torch.int64, device="cuda")
    osh = np.full(W, 1 << 16, np.int64)
    lens = [bat.batch(i)["uih_len"] for i in range(4)]
    d_lens = [cu(x) for x in lens]
    got = []
    for it in range(40):
        perm, ro, _ = lib.fs_balance_vbs_shares(d_lens[it % 4], W, sh, alpha)
        cost = lib.fs_rank_cost(d_lens[it % 4], perm, ro, (1, 64, 0))
        got.append((ro.clone(), sh.clone()))
        lib.fs_vbs_autotune(cost, sh, (1, 16), (1, 50))
    torch.cuda.synchronize()
    spreads = []
    for it in range(40):
        L = lens[it % 4]
        operm, oro, _ = O.balance_vbs_shares(L, W, osh, alpha)
        assert np.array_equal(host(got[it][0]), oro), it
        assert np.array_equal(host(got[it][1]), osh), it
        c = O.rank_cost(L, operm, oro, (1, 64, 0))
        spreads.append(c.max() / c.mean())
        osh = O.vbs_autotune(c, osh, (1, 16), (1, 50))
    assert np.array_equal(host(sh), osh)
    if k == 3:
        assert min(spreads[-5:]) < 0.9 * spreads[0]


# ----------------------------------------------------------------------------- bucketize


def _tiny_batch(seed, N, rows, maxlen=40, bad=0, zero_tok=0):
    rng = np.random.default_rng(seed)
    n_s = rng.integers(1, maxlen + 1, size=N)
    if zero_tok:
        n_s[rng.choice(N, size=min(zero_tok, N), replace=False)] = 0
    so = np.concatenate([[0], np.cumsum(n_s)]).astype(np.int64)
    n = int(so[-1])
    ids = np.stack([rng.zipf(1.2, size=n) % r for r in rows]).astype(np.int64)
    if bad and n:
        pos = rng.choice(n, size=min(bad, n), replace=False)
        ids[0, pos[::2]] = -1
        ids[-1, pos[1::2]] = rows[-1] + 7
    L = np.maximum(n_s - rng.integers(0, 2, size=N), 0).astype(np.int32)
    return dict(uih_len=L, sample_offsets=so, ids=ids, n_tok=n)


def _gpu_bucketize(b, rows, W, balancer="fbs", alpha=(3, 2)):
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    if balancer == "fbs":
        perm, ro = lib.fs_balance_fbs(cu(b["uih_len"]), W, err=err)
    else:
        perm, ro, _ = lib.fs_balance_vbs(cu(b["uih_len"]), W, alpha, err=err)
    bk = lib.fs_bucketize_permute(cu(b["ids"]), cu(b["sample_offsets"]), rows, perm, ro, W,
                                  err=err)
    return perm, ro, bk, err


def _oracle_bucketize(b, rows, W, balancer="fbs", alpha=(3, 2)):
    if balancer == "fbs":
        perm, ro = O.balance_fbs(b["uih_len"], W)
    else:
        perm, ro, _ = O.balance_vbs(b["uih_len"], W, alpha)
    return perm, ro, O.bucketize(b["ids"], b["sample_offsets"], rows, perm, ro, W)


def _cmp_bucket(bk, obk):
    nv = int(obk["shard_offsets"][-1])
    assert np.array_equal(host(bk["bal_offsets"]), obk["bal_offsets"])
    assert np.array_equal(host(bk["shard_offsets"]), obk["shard_offsets"])
    assert np.array_equal(host(bk["splits"]).reshape(obk["splits"].shape), obk["splits"])
    assert np.array_equal(host(bk["shard_keys"])[:nv], obk["shard_keys"])
    assert np.array_equal(host(bk["shard_bm"])[:nv], obk["shard_bm"])


BKT_CASES = [
    # (seed, N, rows, W, maxlen, bad, zero_tok, balancer)
    (1, 64, [100_000], 4, 60, 0, 0, "fbs"),
    (2, 512, [10_000_000], 16, 200, 0, 0, "fbs"),
    (3, 300, [5000, 70, 900_000], 7, 90, 0, 0, "vbs"),
    (4, 50, [1000], 64, 30, 9, 3, "fbs"),          # W > N, dropped IDs, empty samples
    (5, 2048, [20_000_000, 20_000_000, 20_000_000, 5_000_000], 256, 50, 0, 0, "vbs"),
    (6, 1, [10], 3, 9000, 0, 0, "fbs"),            # one long sample, many tiles
    (7, 40, [3], 8, 20, 0, 0, "fbs"),              # table smaller than W
    (8, 4096, [200_000_000], 512, 120, 4, 0, "fbs"),
    (9, 9, [1 << 20], 1024, 800, 0, 2, "vbs"),
]


@pytest.mark.parametrize("case", BKT_CASES, ids=lambda c: f"s{c[0]}")
def test_bucketize_parity(case):
    seed, N, rows, W, maxlen, bad, zt, bal = case
    say("bucketize", case)
    b = _tiny_batch(seed, N, rows, maxlen, bad, zt)
    perm, ro, bk, err = _gpu_bucketize(b, rows, W, bal)
    operm, oro, obk = _oracle_bucketize(b, rows, W, bal)
    torch.cuda.synchronize()
    assert np.array_equal(host(perm), operm)
    _cmp_bucket(bk, obk)
    assert (int(err.item()) & lib.FS_EF_ID_RANGE) == (obk["err"] & 1)


@pytest.mark.parametrize("k", [1, 2, 3, 4])
def test_bucketize_workload_batch(k):
    w = synth.WORKLOADS[k]
    bt = synth.Batches(w, k)
    rows = [t.rows for t in w.tables]
    for it in range(2):
        b = bt.batch(it)
        for bal in ("fbs", "vbs"):
            say("bucketize-workload", k, it, bal)
            _, _, bk, err = _gpu_bucketize(b, rows, w.world, bal, w.alpha)
            _, _, obk = _oracle_bucketize(b, rows, w.world, bal, w.alpha)
            torch.cuda.synchronize()
            _cmp_bucket(bk, obk)
            assert int(err.item()) == 0


def test_bucketize_bad_offsets_flag_shape():
    say("bucketize-shape")
    b = _tiny_batch(3, 20, [100], 10)
    so = b["sample_offsets"].copy()
    so[-1] += 5  # disagrees with n_tok
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    perm, ro = lib.fs_balance_fbs(cu(b["uih_len"]), 4)
    bk = lib.fs_bucketize_permute(cu(b["ids"]), cu(so), [100], perm, ro, 4, err=err)
    torch.cuda.synchronize()
    assert int(err.item()) & lib.FS_EF_SHAPE
    assert np.all(host(bk["shard_offsets"]) == 0) and np.all(host(bk["splits"]) == 0)


# ----------------------------------------------------------------------------- combine

# (seed, N, rows, dims, dtypes, W, bad IDs): one table and several, row sizes
# 64 B .. 2 KB, W above N, dropped IDs
COMBINE_CASES = [
    (41, 300, [5000], [64], ["f32"], 4, 0),
    (42, 500, [3000, 700, 90000], [64, 128, 256], ["f32", "bf16", "f32"], 16, 9),
    (43, 40, [1500, 20000], [512, 1024], ["bf16", "bf16"], 64, 3),
    (44, 200, [100000], [512], ["f32"], 7, 0),
]


@pytest.mark.parametrize("case", COMBINE_CASES)
def test_ranged_combine_parity(case):
    """GPU combine vs the oracle's on the same shard-major rows (random bytes,
    a stride wider than every row): every slot bit-exact, untouched slots
    keep their fill."""
    seed, N, rows, dims, dts, W, bad = case
    say("combine", case)
    b = _tiny_batch(seed, N, rows, 40, bad)
    _, _, bk, err = _gpu_bucketize(b, rows, W)
    torch.cuda.synchronize()
    nv = int(host(bk["shard_offsets"])[-1])
    torch_dt = [torch.float32 if d == "f32" else torch.bfloat16 for d in dts]
    row_bytes = [d * (4 if dt == "f32" else 2) for d, dt in zip(dims, dts)]
    stride = max(row_bytes) + 32
    rng = np.random.default_rng(seed)
    src_h = rng.integers(0, 256, size=(max(nv, 1), stride), dtype=np.uint8)
    src = torch.from_numpy(src_h).cuda()
    n_tok = b["n_tok"]
    fill = [torch.full((n_tok, d), 3, dtype=dt, device="cuda") for d, dt in zip(dims, torch_dt)]
    out = lib.fs_ranged_combine(src, bk, W, dims, torch_dt, rows, n_tok, out=fill)
    torch.cuda.synchronize()
    keys = host(bk["shard_keys"])[:nv]
    bm = host(bk["shard_bm"])[:nv]
    ref = O.ranged_combine(src_h[:nv], keys, bm, rows, row_bytes, n_tok)
    for t in range(len(rows)):
        got = host(out[t].view(torch.uint8) if out[t].dtype == torch.float32 else
                   out[t].view(torch.int16)).view(np.uint8).reshape(n_tok, row_bytes[t])
        hit = np.zeros(n_tok, bool)
        hit[bm[(keys >= sum(rows[:t])) & (keys < sum(rows[:t + 1]))]] = True
        assert np.array_equal(got[hit], ref[t][hit])
        three = np.full((1, dims[t]), 3, dtype=np.float32)
        pattern = (three.view(np.uint8) if dts[t] == "f32" else
                   torch.full((1, dims[t]), 3, dtype=torch.bfloat16).view(torch.int16)
                   .numpy().view(np.uint8))
        assert np.array_equal(got[~hit], np.repeat(pattern, int((~hit).sum()), axis=0))
    assert int(err.item()) == (lib.FS_EF_ID_RANGE if bad else 0)


# ----------------------------------------------------------------------------- keyed transpose

# (seed, F, B, length mix, element bytes)
KT_CASES = [
    (51, 3, 5, "short", 8),
    (52, 7, 1000, "short", 8),      # four offset tiles and a ragged tail
    (53, 8, 300, "long", 4),        # lists of up to 3000 values
    (54, 40, 300, "sparse", 8),     # four lists in five empty
    (55, 1, 1, "one", 8),           # one list of 10000 values
    (56, 1, 5000, "short", 4),      # one feature: a plain copy
    (57, 3000, 1, "short", 8),      # one sample
    (58, 6, 7, "empty", 8),         # every list empty
    (59, 0, 9, "empty", 8),         # no features at all
    (60, 16, 4096, "mixed", 8),     # 2^16 lists, lognormal lengths, a third empty
    (61, 5, 2048, "mixed", 4),
    (62, 32, 256, "short", 8),      # 8192 lists: the largest one-workgroup offsets
    (63, 1, 8193, "short", 4),      # one more: tiled offsets, a one-list tail tile
    (64, 2048, 2, "short", 8),      # two samples: rows padded to three in LDS
    (65, 4096, 2, "sparse", 8),     # padded rows too long for LDS: tiled offsets
    (66, 1, 32769, "short", 8),     # seventeen offset tiles
]


def _kt_lengths(rng, F, B, kind):
    if kind == "long":
        x = rng.integers(0, 3000, (F, B))
    elif kind == "sparse":
        x = np.where(rng.random((F, B)) < 0.8, 0, rng.integers(1, 5, (F, B)))
    elif kind == "one":
        x = np.full((F, B), 10000)
    elif kind == "empty":
        x = np.zeros((F, B))
    elif kind == "mixed":
        x = np.minimum(np.floor(rng.lognormal(3.0, 1.5, (F, B))), 20000)
        x[rng.random((F, B)) < 0.33] = 0
    else:
        x = rng.integers(0, 7, (F, B))
    return x.astype(np.int32)


def _kt_values(rng, n, eb):
    if eb == 8:
        return rng.integers(-2 ** 62, 2 ** 62, n, dtype=np.int64)
    return rng.integers(-2 ** 31, 2 ** 31, n, dtype=np.int32)


@pytest.mark.parametrize("shift", [0, 1])
@pytest.mark.parametrize("case", KT_CASES)
def test_keyed_transpose_parity(case, shift):
    """Batch-major values and offsets bit-exact against the oracle; the
    elements around the output are not touched. 4-byte values are compared
    widened to int64 (the transpose only moves them). shift = 1 puts values
    and output one element past a 16-byte boundary (the element-wise copy);
    shift = 0 keeps them aligned (the 16-byte copy)."""
    seed, F, B, kind, eb = case
    say("keyed transpose", case, shift)
    rng = np.random.default_rng(seed)
    lengths = _kt_lengths(rng, F, B, kind)
    n = int(lengths.sum())
    vals = _kt_values(rng, n, eb)
    dt = torch.int64 if eb == 8 else torch.int32
    vbuf = torch.zeros(n + 8, dtype=dt, device="cuda")
    vbuf[shift:shift + n] = cu(vals)
    out = torch.full((n + 64,), 77, dtype=dt, device="cuda")
    offs = torch.full((F * B + 1,), -5, dtype=torch.int64, device="cuda")
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    lib.fs_keyed_transpose(vbuf[shift:shift + n], cu(lengths), out=out[shift:shift + n],
                           out_offsets=offs, err=err)
    ref, ro = O.keyed_transpose(vals.astype(np.int64), lengths)
    torch.cuda.synchronize()
    assert np.array_equal(host(offs), ro)
    got = host(out)
    assert np.array_equal(got[shift:shift + n].astype(np.int64), ref)
    assert (got[:shift] == 77).all() and (got[shift + n:] == 77).all()
    assert int(err.item()) == 0


@pytest.mark.parametrize("k", [4, 5])
def test_keyed_transpose_workload(k):
    """The jagged IDs of a workload batch as F features keyed by sample: F
    sequence features of each sample's token count (workload 4's four tables,
    eight features for workload 5: 51M int64 values, every one compared)."""
    w = synth.workload(k)
    b = synth.Batches(w, k).batch(0)
    so = b["sample_offsets"]
    F = 4 if k == 4 else 8
    say("keyed transpose workload", k, F)
    lengths = np.tile(np.diff(so).astype(np.int32), (F, 1))
    n = int(lengths.sum())
    vals = (np.ascontiguousarray(b["ids"]).ravel() if k == 4 else
            np.random.default_rng(k).integers(0, 2 ** 40, n, dtype=np.int64))
    assert len(vals) == n
    got, go = lib.fs_keyed_transpose(cu(vals), cu(lengths))
    ref, ro = O.keyed_transpose(vals, lengths)
    torch.cuda.synchronize()
    assert np.array_equal(host(go), ro)
    assert np.array_equal(host(got), ref)


def test_keyed_transpose_bad_lengths_flag_shape():
    """Negative lengths count as zero; a value count other than the lengths'
    sum flags FS_EF_SHAPE and copies only what lies inside both arrays."""
    rng = np.random.default_rng(70)
    F, B = 6, 900
    lengths = rng.integers(0, 40, (F, B)).astype(np.int32)
    lengths[rng.random((F, B)) < 0.05] = -3
    clean = np.maximum(lengths, 0)
    total = int(clean.sum())
    ref_idx, ro = O.keyed_transpose(np.arange(total, dtype=np.int64), clean)
    for n_vals in (total, total - 1000, total + 500):
        say("keyed transpose bad", n_vals)
        err = torch.zeros(1, dtype=torch.int32, device="cuda")
        out = torch.full((n_vals + 64,), -1, dtype=torch.int64, device="cuda")
        offs = torch.empty(F * B + 1, dtype=torch.int64, device="cuda")
        vals = torch.arange(n_vals, dtype=torch.int64, device="cuda")
        lib.fs_keyed_transpose(vals, cu(lengths), out=out[:n_vals], out_offsets=offs, err=err)
        torch.cuda.synchronize()
        assert int(err.item()) == lib.FS_EF_SHAPE
        assert np.array_equal(host(offs), ro)
        got = host(out)
        p = np.arange(n_vals)
        want = np.full(n_vals, -1, np.int64)
        inside = p < total
        src = np.full(n_vals, -1, np.int64)
        src[inside] = ref_idx[p[inside]]
        ok = inside & (src < n_vals)
        want[ok] = src[ok]
        assert np.array_equal(got[:n_vals], want)
        assert (got[n_vals:] == -1).all()


# ----------------------------------------------------------------------------- unique


def _gpu_unique(bk, rows, W, n_cap, prev=None, prev_cap=0):
    return lib.fs_unique_collision_split(
        bk["shard_keys"], bk["shard_bm"], bk["shard_offsets"], n_cap, rows, W,
        prev_unique=prev["unique"] if prev else None, prev_counts=prev["counts"] if prev else None,
        prev_cap=prev_cap, prev_unique_offsets=prev["unique_offsets"] if prev else None)


def _cmp_unique(uq, ouq, cls, pcls, counts):
    U = len(ouq["unique"])
    assert int(host(uq["counts"])[0]) == U
    assert np.array_equal(host(uq["counts"]), counts)
    assert np.array_equal(host(uq["unique"])[:U], ouq["unique"])
    assert np.array_equal(host(uq["unique_offsets"]), ouq["unique_offsets"])
    assert np.array_equal(host(uq["seg_offsets"])[:U + 1], ouq["seg_offsets"])
    n = len(ouq["occ_bm"])
    assert np.array_equal(host(uq["occ_bm"])[:n], ouq["occ_bm"])
    assert np.array_equal(host(uq["occ_uid"])[:n], ouq["occ_uid"])
    assert np.array_equal(host(uq["cls"])[:U], cls)
    if pcls is not None and len(pcls):
        assert np.array_equal(host(uq["prev_cls"])[:len(pcls)], pcls)


# s11-s16 sort all items as one segment; s17-s19 are sized so that sorting
# inside the shards saves a pass (2^21 rows: 21-bit global keys, 3 passes;
# 20-bit shard-local keys, 2 passes; ~100-150 tiles against 2-3 shards), with
# one, two and three tables (the (table, shard) group moves)
UQ_CASES = [(11, 64, [100_000], 4, 60), (12, 512, [300, 5000], 16, 200),
            (13, 2048, [20_000, 20_000, 9000, 500], 256, 40), (14, 37, [50], 8, 30),
            (15, 4096, [200_000_000], 512, 60), (16, 3, [7], 2, 3),
            (17, 2048, [1 << 21], 2, 400), (18, 2048, [1 << 20, 1 << 20], 2, 200),
            (19, 2048, [1 << 20, 700_000, 300_000], 3, 100),
            # at most 4096 items: the one-workgroup path, with 3 and 2 tables
            (20, 64, [50, 5000, 300], 8, 20), (21, 100, [1 << 20, 1 << 20], 2, 40),
            # the call limits on the one-workgroup path: 8 tables over 1024 shards
            (22, 16, [1 << 20] * 7 + [3000], 1024, 20),
            # a few thousand items above the one-workgroup path's limit
            (23, 256, [5000, 1 << 20], 16, 40), (24, 600, [1 << 22], 64, 50)]


@pytest.mark.parametrize("case", UQ_CASES, ids=lambda c: f"s{c[0]}")
def test_unique_collision_parity(case):
    seed, N, rows, W, maxlen = case
    T = len(rows)
    prev, oprev, prev_cap = None, None, 0
    for it in range(3):
        say("unique", case, it)
        b = _tiny_batch(seed * 10 + it, N, rows, maxlen, bad=2 if it == 1 else 0)
        if it == 2:  # identical to the previous batch: every row collides
            b = _tiny_batch(seed * 10 + 1, N, rows, maxlen, bad=2)
        _, _, bk, _ = _gpu_bucketize(b, rows, W)
        _, _, obk = _oracle_bucketize(b, rows, W)
        n_cap = T * b["n_tok"]
        uq = _gpu_unique(bk, rows, W, n_cap, prev, prev_cap)
        ouq = O.unique(obk["shard_keys"], obk["shard_bm"], rows, W)
        cls, pcls, counts = O.collision(ouq["unique"], oprev["unique"] if oprev else None)
        torch.cuda.synchronize()
        _cmp_unique(uq, ouq, cls, pcls if prev else None, counts)
        if it == 2:
            assert counts[1] == counts[0]
        prev, oprev, prev_cap = uq, ouq, n_cap


@pytest.mark.parametrize("case", UQ_CASES, ids=lambda c: f"s{c[0]}")
def test_dedup_then_collision_split_equals_one_call(case):
    """A dedup call without previous rows followed by fs_collision_split
    gives every output of one fs_unique_collision_split call with the
    previous rows, bit for bit (three consecutive batches, the last
    identical to the one before)."""
    seed, N, rows, W, maxlen = case
    T = len(rows)
    prev_one, prev_two, prev_cap = None, None, 0
    for it in range(3):
        say("dedup + split", case, it)
        b = _tiny_batch(seed * 10 + (1 if it == 2 else it), N, rows, maxlen,
                        bad=2 if it >= 1 else 0)
        _, _, bk, _ = _gpu_bucketize(b, rows, W)
        n_cap = T * b["n_tok"]
        one = _gpu_unique(bk, rows, W, n_cap, prev_one, prev_cap)
        two = _gpu_unique(bk, rows, W, n_cap)  # every row exclusive
        pcls = lib.fs_collision_split(
            two, n_cap, T, W, prev_unique=prev_two["unique"] if prev_two else None,
            prev_unique_offsets=prev_two["unique_offsets"] if prev_two else None,
            prev_counts=prev_two["counts"] if prev_two else None, prev_cap=prev_cap)
        torch.cuda.synchronize()
        U = int(host(one["counts"])[0])
        n = int(host(bk["shard_offsets"])[-1])
        assert np.array_equal(host(one["counts"]), host(two["counts"]))
        for k, m in (("unique", U), ("unique_offsets", T * W + 1), ("seg_offsets", U + 1),
                     ("occ_bm", n), ("occ_uid", n), ("cls", U)):
            assert np.array_equal(host(one[k])[:m], host(two[k])[:m]), k
        if prev_one is not None:
            pu = int(host(prev_one["counts"])[0])
            assert np.array_equal(host(one["prev_cls"])[:pu], host(pcls)[:pu])
        prev_one, prev_two, prev_cap = one, two, n_cap


@pytest.mark.parametrize("W,rows", [(1, [2_000_000]), (3, [300_000, 1_000_000])],
                         ids=["W1", "W3-2tables"])
def test_collision_uneven_batches(W, rows):
    """Consecutive batches of very different sizes (big, small, big, big): a
    group's rows cut into many chunks and spread over several workgroups,
    and one chunk's previous rows spanning many LDS pieces; classes and
    counts equal the oracle's."""
    T = len(rows)
    prev, oprev, prev_cap = None, None, 0
    for it, (N, maxlen) in enumerate([(4096, 120), (16, 20), (4096, 120), (2048, 60)]):
        say("collision-uneven", W, rows, it)
        b = _tiny_batch(7000 + it, N, rows, maxlen)
        _, _, bk, _ = _gpu_bucketize(b, rows, W)
        _, _, obk = _oracle_bucketize(b, rows, W)
        n_cap = T * b["n_tok"]
        uq = _gpu_unique(bk, rows, W, n_cap, prev, prev_cap)
        ouq = O.unique(obk["shard_keys"], obk["shard_bm"], rows, W)
        cls, pcls, counts = O.collision(ouq["unique"], oprev["unique"] if oprev else None)
        torch.cuda.synchronize()
        _cmp_unique(uq, ouq, cls, pcls if prev else None, counts)
        prev, oprev, prev_cap = uq, ouq, n_cap


def _shard_major(rng, sizes, rows, W, kinds):
    """Shard-major keys of one table with exactly sizes[d] items in shard d;
    kinds[d] picks the key mix: "dup" (few distinct rows), "one" (one row),
    "edge" (the shard's first and last rows among random ones), else random
    rows of the shard. bm values are distinct and rise within each shard, as
    in a bucketize call's output (the dedup keeps that order per row)."""
    block = -(-rows // W)
    parts = []
    for d, (n, kind) in enumerate(zip(sizes, kinds)):
        lo, hi = d * block, min(rows, (d + 1) * block)
        if kind == "dup":
            pool = rng.integers(lo, hi, size=37)
            k = pool[rng.integers(0, len(pool), size=n)]
        elif kind == "one":
            k = np.full(n, lo + (hi - lo) // 2)
        else:
            k = rng.integers(lo, hi, size=n)
            if kind == "edge" and n >= 2:
                k[rng.choice(n, size=2, replace=False)] = [lo, hi - 1]
        parts.append(k.astype(np.int64))
    keys = np.concatenate(parts)
    pool = rng.permutation(len(keys) * 3)[:len(keys)]
    bm = np.concatenate([np.sort(x) for x in np.split(pool, np.cumsum(sizes)[:-1])])
    bm = bm.astype(np.int32)
    so = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int64)
    return keys, bm, so


# One table sorted inside the shards, shards of exact sizes: empty shards,
# partial waves and tiles (63/64/65, 2047/2048 items), sizes around 2^14,
# shards of few distinct rows or of one row, the shard's first and last rows,
# a short last shard; shard-local keys of 20 bits (two radix passes) and of
# 8 bits (one pass).
SS_CASES = [
    ("wide", 16 << 20, [0, 1, 63, 64, 65, 2047, 2048, 16383, 16384, 16385, 40000, 5000, 0, 777,
                        30000, 12],
     ["rand", "rand", "edge", "dup", "rand", "one", "edge", "dup", "edge", "rand", "dup", "rand",
      "rand", "one", "edge", "rand"]),
    ("narrow", 16 * 200 - 3, [20000, 16384, 100, 0, 16383, 1, 9000, 16385, 64, 3, 0, 0, 4096, 5,
                              700, 16384],
     ["dup", "edge", "rand", "rand", "rand", "one", "edge", "dup", "rand", "rand", "rand", "rand",
      "edge", "one", "dup", "rand"]),
    ("all-small", 16 << 20, [16384, 9000, 1, 0] * 4, ["edge", "dup", "rand", "rand"] * 4),
    # the one-workgroup dedup takes calls of up to 4096 items, the radix passes
    # one more (and the 32768-item pair: a one-workgroup path staged in global
    # memory up to that size was built and measured slower, so the radix
    # passes take both)
    ("4096-items", 16 << 20, [1000, 0, 63, 1, 2047, 985] + [0] * 10,
     ["dup", "rand", "edge", "one", "rand", "edge"] + ["rand"] * 10),
    ("4097-items", 16 << 20, [1000, 0, 63, 1, 2047, 986] + [0] * 10,
     ["dup", "rand", "edge", "one", "rand", "edge"] + ["rand"] * 10),
    ("32768-items", 16 << 20, [16384, 0, 63, 1, 2047, 14273] + [0] * 10,
     ["dup", "rand", "edge", "one", "rand", "edge"] + ["rand"] * 10),
    ("32769-items", 16 << 20, [16384, 0, 63, 1, 2047, 14274] + [0] * 10,
     ["dup", "rand", "edge", "one", "rand", "edge"] + ["rand"] * 10),
    # calls of up to 2^20 items (512 tiles) compact with the tile scan in the
    # compaction's own launch, larger ones with a scan launch before it
    ("1048576-items", 16 << 20, [65536] * 16, ["rand", "dup", "edge", "one"] * 4),
    ("1048577-items", 16 << 20, [65536] * 15 + [65537], ["rand", "dup", "edge", "one"] * 4),
]


@pytest.mark.parametrize("name,rows,sizes,kinds", SS_CASES, ids=[c[0] for c in SS_CASES])
def test_unique_shard_sizes(name, rows, sizes, kinds):
    """Unique outputs equal the oracle's, element by element, for shards of
    exact sizes; each row's occurrences keep their order (occ_bm rising)."""
    W = len(sizes)
    rng = np.random.default_rng(sum(sizes) % 1000 + W)
    keys, bm, so = _shard_major(rng, sizes, rows, W, kinds)
    n = len(keys)
    say("unique shard sizes", name, n)
    # spare capacity, kept on the same side of each path's limit (the
    # one-workgroup dedup's 4096 items, the compaction's own scan's 2^20)
    lims = [t for t in (4096, 1 << 20) if n <= t]
    caps = (n, n + 5000) if not lims else ((n, lims[0]) if n < lims[0] else (n,))
    for n_cap in caps:
        uq = lib.fs_unique_collision_split(cu(keys), cu(bm), cu(so), n_cap, [rows], W)
        ouq = O.unique(keys, bm, [rows], W)
        cls, _, counts = O.collision(ouq["unique"], None)
        torch.cuda.synchronize()
        _cmp_unique(uq, ouq, cls, None, counts)


def test_unique_empty_batch():
    say("unique-empty")
    rows = [100]
    b = dict(uih_len=np.zeros(4, np.int32), sample_offsets=np.zeros(5, np.int64),
             ids=np.zeros((1, 0), np.int64), n_tok=0)
    _, _, bk, _ = _gpu_bucketize(b, rows, 4)
    uq = _gpu_unique(bk, rows, 4, 0)
    torch.cuda.synchronize()
    assert host(uq["counts"]).tolist() == [0, 0, 0, 0]
    assert np.all(host(uq["unique_offsets"]) == 0)


def test_lookup_and_update_of_an_empty_batch():
    """After an empty batch's dedup, the lookup and the update (SGD and
    row-wise Adagrad, each row part, with a workspace and without) succeed
    and leave the table and its state as they were."""
    say("lookup-update-empty")
    rows = [100]
    b = dict(uih_len=np.zeros(4, np.int32), sample_offsets=np.zeros(5, np.int64),
             ids=np.zeros((1, 0), np.int64), n_tok=0)
    _, _, bk, _ = _gpu_bucketize(b, rows, 4)
    uq = _gpu_unique(bk, rows, 4, 0)
    w = _table(100, 64, "f32", 3)
    st = torch.rand(100, dtype=torch.float32, device="cuda")
    w0, s0 = w.clone(), st.clone()
    out = lib.fs_jagged_lookup([w], 4, uq, 0)
    assert tuple(out[0].shape) == (0, 64)
    g = torch.empty((0, 64), dtype=torch.float32, device="cuda")
    for optim in ("sgd", "rw_adagrad"):
        for part in (lib.FS_ROWS_ALL, lib.FS_ROWS_FEW, lib.FS_ROWS_MANY):
            lib.fs_grad_reduce_update([w], [st], 4, [g], 0, uq, optim, 0.05, 1e-8, rows=part)
            lib.fs_grad_reduce_update_noalloc([w], [st], 4, [g], 0, uq, optim, 0.05, 1e-8,
                                              rows=part)
    torch.cuda.synchronize()
    assert torch.equal(w, w0) and torch.equal(st, s0)


# ----------------------------------------------------------------------------- lookup + update


def _csr_to_dev(ouq):
    return {k: cu(v) for k, v in ouq.items()}


def _table(rows, dim, dtype, seed):
    return synth.init_table(rows, dim, dtype, seed, "cuda")


def _table_rowstate(rows, dim, dtype, seed, align=16):
    """The same values in rows of a wider buffer, each row's state in its own
    padding (slots rounded up to `align` bytes); returns (weights view, state
    view, the whole buffer as bytes)."""
    tdt = torch.float32 if dtype == "f32" else torch.bfloat16
    w, st = lib.alloc_table(rows, dim, tdt, True, device="cuda", align=align)
    synth.init_table(rows, dim, dtype, seed, "cuda", out=w)
    st.zero_()
    buf = torch.empty(0, dtype=torch.uint8, device="cuda").set_(w.untyped_storage())
    return w, st, buf


LK_CASES = [([100_000], [64], ["f32"], 4), ([5000, 300], [128, 256], ["bf16", "f32"], 16),
            ([4000, 4000, 9000, 20], [64, 128, 256, 64], ["f32"] * 4, 8),
            ([777], [512], ["f32"], 2), ([3000], [1024], ["bf16"], 3), ([100], [32], ["f32"], 4),
            ([200], [16], ["f32"], 4), ([1000], [512], ["bf16"], 5)]


@pytest.mark.parametrize("layout", ["dense", "rowstate", "rowstate256"])
@pytest.mark.parametrize("case", LK_CASES, ids=lambda c: f"D{c[1]}")
def test_lookup_parity(case, layout):
    rows, dims, dts, W = case
    say("lookup", case, layout)
    b0 = _tiny_batch(21, 300, rows, 50)
    b1 = _tiny_batch(22, 300, rows, 50)
    if layout == "dense":
        ws = [_table(r, d, dt, 5 + t) for t, (r, d, dt) in enumerate(zip(rows, dims, dts))]
    else:  # rows spaced wider than they are (the state's padding)
        al = 256 if layout == "rowstate256" else 16
        ws = [_table_rowstate(r, d, dt, 5 + t, al)[0]
              for t, (r, d, dt) in enumerate(zip(rows, dims, dts))]
    stores = snapshot_stores(ws, [None] * len(ws), [np.arange(r) for r in rows])
    outs = {}
    oq = []
    for b in (b0, b1):
        _, _, obk = _oracle_bucketize(b, rows, W)
        oq.append(O.unique(obk["shard_keys"], obk["shard_bm"], rows, W))
    cls1, _, _ = O.collision(oq[1]["unique"], oq[0]["unique"])
    oq[1]["cls"] = cls1
    n = b1["n_tok"]
    for which in (lib.FS_ALL, lib.FS_COLLISION, lib.FS_EXCLUSIVE):
        dq = _csr_to_dev(oq[1])
        fill = [torch.full((n, d), 7, dtype=w.dtype, device="cuda") for d, w in zip(dims, ws)]
        outs[which] = lib.fs_jagged_lookup(ws, W, dq, n, which=which, cls=dq["cls"], out=fill)
    torch.cuda.synchronize()
    rb = np.concatenate([[0], np.cumsum(rows)[:-1]])
    for t, st in enumerate(stores):
        lo, hi = int(oq[1]["unique_offsets"][t * W]), int(oq[1]["unique_offsets"][(t + 1) * W])
        for which in (lib.FS_ALL, lib.FS_COLLISION, lib.FS_EXCLUSIVE):
            sentinel = torch.full((1, dims[t]), 7, dtype=ws[t].dtype)
            sentinel = (sentinel.view(torch.int16).numpy().view(np.uint16) if st.bf16
                        else sentinel.numpy())
            exp = np.broadcast_to(sentinel, (n, dims[t])).copy()
            O.lookup(st, int(rb[t]), lo, hi, oq[1], n, which=which, out=exp)
            got = outs[which][t]
            got = host(got.view(torch.int16)).view(np.uint16) if st.bf16 else host(got)
            assert np.array_equal(got, exp), (t, which)


def _hot_batch(seed, rows, n_tok, hot):
    """One sample per token; `hot` = [(row, count)] forced occurrences."""
    rng = np.random.default_rng(seed)
    ids = rng.integers(0, rows, size=n_tok).astype(np.int64)
    pos = rng.permutation(n_tok)
    k = 0
    for r, c in hot:
        ids[pos[k:k + c]] = r
        k += c
    so = np.arange(n_tok + 1, dtype=np.int64)
    return dict(uih_len=np.ones(n_tok, np.int32), sample_offsets=so, ids=ids[None, :],
                n_tok=n_tok)


RU_CASES = [
    # (dim, dtype, optim, hot, n_tok, W, rows)
    (128, "f32", "sgd", [(3, 5000), (9, 700), (11, 65), (12, 64), (13, 513)], 16384, 8, 2000),
    (128, "bf16", "rw_adagrad", [(3, 5000), (9, 700), (11, 65), (12, 64)], 16384, 8, 2000),
    (64, "f32", "rw_adagrad", [(1, 3000), (2, 1025)], 12000, 4, 50_000),
    (256, "f32", "sgd", [(5, 2000), (6, 600)], 9000, 16, 30_000),
    (512, "bf16", "rw_adagrad", [(5, 1500)], 6000, 2, 3000),
    (1024, "f32", "rw_adagrad", [(7, 900)], 4000, 3, 5000),
    (128, "f32", "rw_adagrad", [], 10000, 4, 10_000_000),  # all rows short
    (128, "f32", "sgd", [(0, 30000)], 30000, 4, 100),       # one row owns every token
    # ~0.6M unique rows: the short-row kernel takes 32-row units per wave
    (64, "f32", "sgd", [(7, 20_000)], 600_000, 8, 50_000_000),
    # 2.7M tokens: 256-occurrence long-row chunks, one row split over ~1560 of them
    (64, "bf16", "rw_adagrad", [(5, 400_000), (6, 3000)], 2_700_000, 16, 5_000_000),
    # a row of every medium length (5 .. 64 occurrences) at the widths whose
    # own medium-row kernel streams 16 gradient rows at a time (calls above
    # 2^17 occurrences: smaller ones run the one-launch kernel): batches end
    # ragged
    (64, "bf16", "rw_adagrad", [(10 + k, 5 + k) for k in range(60)] + [(90, 200)], 150_000, 8,
     1_000_000),
    (256, "f32", "sgd", [(10 + k, 5 + k) for k in range(60)], 140_000, 4, 2_000_000),
]


@pytest.mark.parametrize("layout", ["dense", "rowstate", "rowstate256"])
@pytest.mark.parametrize("case", RU_CASES, ids=lambda c: f"D{c[0]}-{c[1]}-{c[2]}-{c[4]}")
def test_reduce_update_parity(case, layout):
    """Reduced gradients bit-exact, rows and states to the fp32 / bf16
    tolerance; with each row's state in its own padding, every byte outside
    the touched rows' weights and states is left as it was."""
    dim, dt, optim, hot, n_tok, W, rows = case
    if layout != "dense" and rows * dim > 2e9:
        pytest.skip("table too large for a second layout")
    say("reduce-update", case, layout)
    b = _hot_batch(dim + n_tok, rows, n_tok, hot)
    _, _, obk = _oracle_bucketize(b, [rows], W)
    ouq = O.unique(obk["shard_keys"], obk["shard_bm"], [rows], W)
    U = len(ouq["unique"])
    cls = (np.random.default_rng(1).random(U) < 0.5).astype(np.uint8)
    grad = synth.gradient_rows(7, 0, 0, np.arange(n_tok), dim)
    if layout == "dense":
        wt = _table(rows, dim, dt, 9)
        st = torch.zeros(rows, dtype=torch.float32, device="cuda") if optim == "rw_adagrad" \
            else None
    else:
        wt, st, buf = _table_rowstate(rows, dim, dt, 9, 256 if layout == "rowstate256" else 16)
        before = buf.clone()
        st = st if optim == "rw_adagrad" else None
    stores = snapshot_stores([wt], [st], [np.unique(b["ids"][0])])
    dq = _csr_to_dev(ouq)
    dcls = cu(cls)
    red = torch.full((U, dim), np.nan, dtype=torch.float32, device="cuda")
    # collision rows first, then exclusive rows (two calls, as the schedule does)
    for which in (lib.FS_COLLISION, lib.FS_EXCLUSIVE):
        lib.fs_grad_reduce_update([wt], [st], W, [cu(grad)], n_tok, dq, optim, 0.05, 1e-8,
                                  which=which, cls=dcls, reduced_out=[red])
    g = O.reduce(dim, 0, U, ouq, grad)
    prev = store_vals_f32(stores[0]).copy()
    O.update(stores[0], 0, 0, U, ouq["unique"], g, optim, 0.05, 1e-8)
    torch.cuda.synchronize()
    gr = host(red)
    assert np.array_equal(gr, g), float(np.nanmax(np.abs(gr - g)))  # exact fp64 sums
    rid = stores[0].row_ids
    got = host(wt.index_select(0, cu(rid)).float())
    ref = store_vals_f32(stores[0])
    tol = 1e-2 if dt == "bf16" else 1e-5
    assert rel_err_rows(got, ref, prev) <= tol
    if dt == "f32" and optim == "sgd":
        assert np.array_equal(got, ref)
    if optim == "rw_adagrad":
        np.testing.assert_allclose(host(st.index_select(0, cu(rid))), stores[0].state, rtol=1e-6)
    if layout != "dense":
        e = 4 if dt == "f32" else 2
        stride = wt.stride(0) * e
        mine = torch.zeros(rows, stride, dtype=torch.bool, device="cuda")
        touched = cu(rid.astype(np.int64))
        mine[touched, :dim * e] = True
        if optim == "rw_adagrad":
            mine[touched, dim * e:dim * e + 4] = True
        b2, b1 = buf.view(rows, stride), before.view(rows, stride)
        assert torch.equal(b2.masked_fill(mine, 0), b1.masked_fill(mine, 0))


@pytest.mark.parametrize("mode", ["concurrent", "many-first", "noalloc"])
@pytest.mark.parametrize("case", [RU_CASES[i] for i in (0, 1, 2, 4, 7, 9)],
                         ids=lambda c: f"D{c[0]}-{c[1]}-{c[2]}-{c[4]}")
def test_update_row_parts_equal_whole(case, mode):
    """The update in two parts -- rows of at most 64 occurrences
    (FS_ROWS_FEW) and longer rows (FS_ROWS_MANY) -- gives the one-call
    result bit for bit: rows, states and reduced sums, for every class
    filter. "concurrent": the parts on two streams at once with one
    workspace; "many-first": one stream, long rows first; "noalloc": the
    allocation-free call, parts concurrent."""
    dim, dt, optim, hot, n_tok, W, rows = case
    say("update parts", case, mode)
    b = _hot_batch(dim + n_tok, rows, n_tok, hot)
    _, _, obk = _oracle_bucketize(b, [rows], W)
    ouq = O.unique(obk["shard_keys"], obk["shard_bm"], [rows], W)
    U = len(ouq["unique"])
    dq = _csr_to_dev(ouq)
    touched = cu(np.unique(b["ids"][0]))
    dcls = cu((np.random.default_rng(2).random(U) < 0.5).astype(np.uint8))
    grad = cu(synth.gradient_rows(8, 0, 0, np.arange(n_tok), dim))
    ada = optim == "rw_adagrad"
    outs = []
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    for split in (False, True):
        wt = _table(rows, dim, dt, 9)
        st = torch.full((rows,), 0.25, dtype=torch.float32, device="cuda") if ada else None
        red = torch.full((U, dim), np.nan, dtype=torch.float32, device="cuda")
        ws = torch.empty(lib.reduce_workspace_size(n_tok, dim), dtype=torch.uint8,
                         device="cuda")
        for which in (lib.FS_COLLISION, lib.FS_EXCLUSIVE, lib.FS_ALL):
            kw = dict(which=which, cls=dcls if which != lib.FS_ALL else None, reduced_out=[red])

            def call(rows_, stream):
                if mode == "noalloc":
                    lib.fs_grad_reduce_update_noalloc([wt], [st], W, [grad], n_tok, dq, optim,
                                                      0.05, 1e-8, rows=rows_, stream=stream, **kw)
                else:
                    lib.fs_grad_reduce_update([wt], [st], W, [grad], n_tok, dq, optim, 0.05,
                                              1e-8, ws=ws, rows=rows_, stream=stream, **kw)
            torch.cuda.synchronize()
            if not split:
                call(lib.FS_ROWS_ALL, None)
            elif mode == "many-first":
                call(lib.FS_ROWS_MANY, None)
                call(lib.FS_ROWS_FEW, None)
            else:
                call(lib.FS_ROWS_MANY, s2)
                call(lib.FS_ROWS_FEW, s1)
            torch.cuda.synchronize()
        w_t = wt.index_select(0, touched)
        outs.append((host(w_t.view(torch.int16)) if dt == "bf16" else host(w_t).view(np.uint32),
                     host(st.index_select(0, touched)).view(np.uint32) if ada else None,
                     host(red).view(np.uint32)))
    (w0, s0, r0), (w1, s1_, r1) = outs
    assert np.array_equal(w0, w1)
    assert np.array_equal(r0, r1)  # bit patterns (rows of other classes hold NaN in both)
    if ada:
        assert np.array_equal(s0, s1_)


def test_bucketize_repeated_sample_flags_shape():
    # perm holds in-range entries but repeats the longest sample: the
    # lengths under perm overrun n_tok, so the call must write no items
    say("bucketize-perm-repeat")
    b = _tiny_batch(3, 20, [100], 10)
    so = b["sample_offsets"]
    lens = np.diff(so)
    perm_h = np.full(len(lens), int(np.argmax(lens)), np.int32)
    ro_h = np.array([0, len(lens) // 2, len(lens)], np.int32)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    bk = lib.fs_bucketize_permute(cu(b["ids"]), cu(so), [100], cu(perm_h), cu(ro_h), 2, err=err)
    torch.cuda.synchronize()
    assert int(err.item()) & lib.FS_EF_SHAPE
    assert np.all(host(bk["shard_offsets"]) == 0) and np.all(host(bk["splits"]) == 0)
