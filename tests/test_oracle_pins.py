"""Pins of the CPU oracle against what the pages and the mathematics fix.

Every check here is independent of the oracle's own code: hand-derived deals
from the FreeScale paper (section 4.1), closed forms, invariants, brute force
on tiny inputs in pure Python, and library routines (numpy.unique, math.fsum,
torch.optim, torch's bfloat16 cast) on cases where the method reduces to them.
"""

import math
import os
from decimal import Decimal, getcontext

import numpy as np
import pytest

from oracle import oracle as O


def _read_golden(path):
    with open(path) as f:
        return [ln.strip() for ln in f if ln.strip() and not ln.startswith("#")]


# ----------------------------------------------------------------------------
# FBS


def _ranks_positions(perm, ro, order):
    """Sorted positions held by each rank, from (perm, rank_offsets)."""
    pos_of = {s: p for p, s in enumerate(order)}
    return [sorted(pos_of[s] for s in perm[ro[r]:ro[r + 1]]) for r in range(len(ro) - 1)]


def _py_order(L):
    return [s for _, s in sorted((int(l), s) for s, l in enumerate(L))]


def test_fbs_hand_deals(golden_dir):
    rng = np.random.default_rng(0)
    for ln in _read_golden(os.path.join(golden_dir, "fbs_deals.txt")):
        head, pos = ln.split(":")
        N, W, r = map(int, head.split())
        L = rng.permutation(N).astype(np.int32) + 1  # distinct lengths
        perm, ro = O.balance_fbs(L, W)
        got = _ranks_positions(perm, ro, _py_order(L))[r]
        assert got == [int(x) for x in pos.split()], ln


def test_fbs_printed_pattern_is_not_a_partition():
    # The literal "i, 2n-i, 2n+i, 4n-i" assigns some position twice and skips
    # another (0-based and 1-based alike); the snake reading is a partition.
    n, rounds = 4, 4
    for base in (0, 1):
        taken = []
        for i in range(base, n + base):
            for k in range(rounds // 2):
                taken += [2 * k * n + i, 2 * (k + 1) * n - i]
        assert len(set(taken)) < len(taken)
    snake = [O.fbs_rank_of_position(p, n) for p in range(n * rounds)]
    assert all(snake.count(r) == rounds for r in range(n))


@pytest.mark.parametrize("N,W", [(64, 4), (512, 16), (1024, 64), (4096, 512), (10, 4), (7, 8),
                                 (1, 1), (0, 3)])
def test_fbs_counts_and_order(N, W):
    rng = np.random.default_rng(N * 7 + W)
    L = rng.integers(1, 50, size=N).astype(np.int32)  # many ties
    perm, ro = O.balance_fbs(L, W)
    counts = np.diff(ro)
    assert counts.sum() == N and counts.max() - counts.min() <= 1
    if N % W == 0:
        assert np.all(counts == N // W)
    assert sorted(perm.tolist()) == list(range(N))
    # each rank's samples are in dealing order: ascending (length, index)
    for r in range(W):
        seg = perm[ro[r]:ro[r + 1]]
        keys = [(int(L[s]), int(s)) for s in seg]
        assert keys == sorted(keys)


@pytest.mark.parametrize("N,W", [(16, 4), (48, 6), (4096, 512)])
def test_fbs_position_sums_equal_when_2W_divides_N(N, W):
    # each pair of rounds hands every rank positions summing to 4kW + 2W - 1
    L = np.arange(N, dtype=np.int32)[::-1].copy()
    perm, ro = O.balance_fbs(L, W)
    pos = _ranks_positions(perm, ro, _py_order(L))
    sums = {sum(p) for p in pos}
    assert len(sums) == 1
    assert sums.pop() == sum(4 * k * W + 2 * W - 1 for k in range(N // (2 * W)))


# ----------------------------------------------------------------------------
# VBS


def _decimal_round_pow(L, num, den):
    getcontext().prec = 60
    if num == 0:
        return 1  # L**0 = 1, also for L = 0
    x = Decimal(L) ** (Decimal(num) / Decimal(den))
    return int((x + Decimal("0.5")).to_integral_value(rounding="ROUND_FLOOR"))


def test_vbs_weights_exact():
    for L in list(range(0, 300)) + [1024, 4095, 8191, 16384, 32767, 32768, 65535]:
        for a in [(3, 2), (2, 1), (1, 1), (0, 1), (1, 2), (4, 2)]:
            assert O.vbs_weight(L, a) == _decimal_round_pow(L, *a), (L, a)
    assert O.vbs_weight(3, (1, 3)) == -1  # unsupported exponent


def test_vbs_hand_example(golden_dir):
    g = dict(ln.split(":", 1) for ln in _read_golden(os.path.join(golden_dir,
                                                                  "vbs_example.txt")))
    L = np.array(g["lengths"].split(), np.int32)
    a = tuple(map(int, g["alpha"].split()))
    perm, ro, rw = O.balance_vbs(L, int(g["ranks"]), a)
    assert perm.tolist() == [int(x) for x in g["perm"].split()]
    assert ro.tolist() == [int(x) for x in g["rank_offsets"].split()]
    assert rw.tolist() == [int(x) for x in g["rank_weight"].split()]


@pytest.mark.parametrize("N,W,alpha", [(64, 4, (3, 2)), (1024, 64, (3, 2)), (2048, 256, (2, 1)),
                                       (4096, 512, (3, 2)), (9, 4, (1, 1)), (5, 8, (2, 1))])
def test_vbs_cut_property(N, W, alpha):
    rng = np.random.default_rng(N + W)
    L = np.minimum(np.ceil(rng.lognormal(5, 1.3, size=N)), 32768).astype(np.int32)
    perm, ro, rw = O.balance_vbs(L, W, alpha)
    order = _py_order(L)
    assert perm.tolist() == order
    w = [_decimal_round_pow(int(L[s]), *alpha) for s in order]
    T = sum(w)
    assert ro[0] == 0 and ro[-1] == N and np.all(np.diff(ro) >= 0)
    assert rw.sum() == T
    for r in range(W):
        seg = sum(w[ro[r]:ro[r + 1]])
        assert seg == rw[r]
        # within one boundary sample's weight of T/W
        bnd = [w[c - 1] for c in (ro[r], ro[r + 1]) if 0 < c <= N]
        assert abs(seg * W - T) < W * max(bnd + [0]) or seg * W == T
    # brute force: no cut can move one sample and get closer to its ideal
    S = np.concatenate([[0], np.cumsum(w)])
    for r in range(1, W):
        c = ro[r]
        assert S[c] * W >= r * T
        assert c == 0 or S[c - 1] * W < r * T


def test_vbs_equal_lengths_equal_blocks():
    L = np.full(64, 37, np.int32)
    perm, ro, rw = O.balance_vbs(L, 8, (3, 2))
    assert ro.tolist() == list(range(0, 65, 8))
    assert len(set(rw.tolist())) == 1


def test_vbs_alpha_zero_is_equal_counts():
    L = np.random.default_rng(3).integers(1, 9000, size=100).astype(np.int32)
    perm, ro, _ = O.balance_vbs(L, 7, (0, 1))
    c = np.diff(ro)
    assert set(c.tolist()) <= {100 // 7, 100 // 7 + 1}


# ---- VBS AutoTune ([FS] 4.1 autotune, Figure 4; Algorithm 1's input R)

@pytest.mark.parametrize("alpha", [(0, 1), (1, 2), (1, 1), (3, 2), (2, 1)])
@pytest.mark.parametrize("N,W", [(0, 3), (9, 4), (1024, 64), (4096, 512), (5, 8)])
def test_vbs_equal_shares_is_plain_vbs(N, W, alpha):
    """Equal shares (of any size) reduce to the plain VBS cut."""
    rng = np.random.default_rng(N * 7 + W)
    L = np.minimum(np.ceil(rng.lognormal(5, 1.3, size=N)), 32768).astype(np.int32)
    ref = O.balance_vbs(L, W, alpha)
    for c in (1, 7, 1 << 40):
        got = O.balance_vbs_shares(L, W, np.full(W, c), alpha)
        for a, b in zip(got, ref):
            assert np.array_equal(a, b)


def test_vbs_shares_hand_examples():
    # four unit weights (alpha = 1, L = 1): shares 1:3 and 3:1
    assert O.balance_vbs_shares([1, 1, 1, 1], 2, [1, 3], (1, 1))[1].tolist() == [0, 1, 4]
    assert O.balance_vbs_shares([1, 1, 1, 1], 2, [3, 1], (1, 1))[1].tolist() == [0, 3, 4]
    # eight samples of weight 5, shares 1:1:2 -> 2, 2 and 4 samples
    perm, ro, rw = O.balance_vbs_shares([5] * 8, 3, [1, 1, 2], (1, 1))
    assert ro.tolist() == [0, 2, 4, 8] and rw.tolist() == [10, 10, 20]
    # a share of 1 against 2^40: the first rank's ideal cut is below one sample
    assert O.balance_vbs_shares([3] * 6, 2, [1, 1 << 40], (1, 1))[1].tolist() == [0, 1, 6]
    with pytest.raises(ValueError):
        O.balance_vbs_shares([1, 2], 2, [0, 1], (1, 1))


@pytest.mark.parametrize("W", [2, 7, 64, 300])
def test_vbs_shares_segments_track_their_targets(W):
    """Every cut is the lower bound of its ideal point T * Q_r / Q, so each
    segment differs from T * s_r / Q by less than one boundary sample."""
    rng = np.random.default_rng(W)
    N = 3000
    L = np.minimum(np.ceil(rng.lognormal(5, 1.3, size=N)), 32768).astype(np.int32)
    shares = rng.integers(1, 1000, size=W)
    perm, ro, rw = O.balance_vbs_shares(L, W, shares, (3, 2))
    w = [_decimal_round_pow(int(L[s]), 3, 2) for s in _py_order(L)]
    S = np.concatenate([[0], np.cumsum(w)]).astype(object)
    T, Q = int(S[-1]), int(shares.sum())
    Qr = np.concatenate([[0], np.cumsum(shares)]).astype(object)
    assert ro[0] == 0 and ro[-1] == N
    for r in range(1, W):
        c = int(ro[r])
        assert S[c] * Q >= Qr[r] * T
        assert c == 0 or S[c - 1] * Q < Qr[r] * T
    for r in range(W):
        seg = int(S[ro[r + 1]] - S[ro[r]])
        assert seg == rw[r]
        assert abs(seg * Q - T * int(shares[r])) < Q * max(w)


def test_rank_cost_hand_example_and_total():
    L = np.array([3, 1, 4, 1, 5], np.int32)
    perm = np.array([1, 3, 0, 2, 4], np.int32)
    ro = np.array([0, 2, 5], np.int32)
    # rank 0: L = 1, 1 -> 2 (2*1 + 3*1 + 7); rank 1: L = 3, 4, 5
    got = O.rank_cost(L, perm, ro, (2, 3, 7))
    assert got.tolist() == [24, (18 + 9 + 7) + (32 + 12 + 7) + (50 + 15 + 7)]
    rng = np.random.default_rng(5)
    L = rng.integers(0, 20000, 4000).astype(np.int32)
    perm, ro, _ = O.balance_vbs(L, 37, (1, 1))
    c = O.rank_cost(L, perm, ro, (1, 0, 0))
    assert c.sum() == int((L.astype(np.int64) ** 2).sum())


def test_autotune_hand_examples():
    assert O.vbs_autotune([10, 20, 30], [100, 100, 100], (1, 10), (0, 1)).tolist() == \
        [110, 100, 90]
    # inside the tolerance band: nothing moves
    assert O.vbs_autotune([19, 20, 21], [100, 100, 100], (1, 10), (1, 10)).tolist() == \
        [100, 100, 100]
    # just outside it (mean 20, band 18 .. 22)
    assert O.vbs_autotune([17, 20, 23], [100, 100, 100], (1, 10), (1, 10)).tolist() == \
        [110, 100, 90]
    # the step is at least one, shares never drop below one or exceed 2^40
    assert O.vbs_autotune([1, 9], [3, 1], (1, 16), (0, 1)).tolist() == [4, 1]
    assert O.vbs_autotune([0, 5], [1 << 40, 5], (1, 2), (0, 1)).tolist() == [1 << 40, 3]
    # equal times: no change
    assert O.vbs_autotune([7] * 5, [1, 2, 3, 4, 5], (1, 2), (0, 1)).tolist() == [1, 2, 3, 4, 5]


def test_autotune_closes_the_cost_gap():
    """Weights L^1 under-count a quadratic cost: with shares fed back from the
    modelled time the ranks' costs converge (the purpose of the mechanism) to
    near the floor that the single costliest sample sets."""
    rng = np.random.default_rng(11)
    L = np.minimum(np.ceil(rng.lognormal(6.5, 1.3, size=4096)), 32768).astype(np.int32)
    W = 64
    shares = np.full(W, 1 << 16, np.int64)

    def spread(sh):
        perm, ro, _ = O.balance_vbs_shares(L, W, sh, (1, 1))
        t = O.rank_cost(L, perm, ro, (1, 0, 0))
        return t, t.max() / t.mean()
    t, first = spread(shares)
    for _ in range(60):
        shares = O.vbs_autotune(t, shares, (1, 16), (1, 50))
        t, last = spread(shares)
    c = L.astype(np.int64) ** 2
    floor = c.max() / (c.sum() / W)  # one sample's cost over the mean rank's
    assert first > 3 * last and last < 1.3 * floor


# ----------------------------------------------------------------------------
# bucketize (indexed permute + ranged dispatch)


def _tiny_batch(rng, N, T, R, maxlen=6):
    n_s = rng.integers(1, maxlen + 1, size=N)
    so = np.concatenate([[0], np.cumsum(n_s)]).astype(np.int64)
    ids = np.stack([rng.integers(0, R[t], size=int(so[-1])) for t in range(T)])
    return n_s, so, ids


def _brute_shard_major(ids, so, rows, perm, ro, W):
    """Shard-major items by explicit sort of (d, r, t, q, j) tuples."""
    T = len(rows)
    rb = np.concatenate([[0], np.cumsum(rows)[:-1]])
    bal = [0]
    for s in perm:
        bal.append(bal[-1] + int(so[s + 1] - so[s]))
    rank_of_q = {}
    for r in range(W):
        for q in range(ro[r], ro[r + 1]):
            rank_of_q[q] = r
    items = []
    for q, s in enumerate(perm):
        for j in range(int(so[s + 1] - so[s])):
            for t in range(T):
                idv = int(ids[t][so[s] + j])
                block = -(-int(rows[t]) // W)
                d = idv // block
                items.append(((d, rank_of_q[q], t, q, j), int(rb[t]) + idv, bal[q] + j))
    items.sort()
    return items, bal


@pytest.mark.parametrize("W,T", [(1, 1), (3, 1), (4, 2), (5, 3)])
def test_bucketize_brute_force(W, T):
    rng = np.random.default_rng(W * 10 + T)
    R = [int(x) for x in rng.integers(5, 40, size=T)]
    N = 9
    _, so, ids = _tiny_batch(rng, N, T, R)
    L = rng.integers(1, 5, size=N).astype(np.int32)
    perm, ro = O.balance_fbs(L, W)
    bk = O.bucketize(ids, so, R, perm, ro, W)
    items, bal = _brute_shard_major(ids, so, R, perm, ro, W)
    assert bk["bal_offsets"].tolist() == bal
    assert bk["shard_keys"].tolist() == [k for _, k, _ in items]
    assert bk["shard_bm"].tolist() == [b for _, _, b in items]
    d_of = [t[0] for t, _, _ in items]
    assert bk["shard_offsets"].tolist() == [sum(1 for d in d_of if d < x) for x in range(W + 1)]
    sp = bk["splits"]
    for d in range(W):
        for r in range(W):
            assert sp[d, r] == sum(1 for t, _, _ in items if t[0] == d and t[1] == r)
    assert bk["err"] == 0


def test_bucketize_single_shard_is_identity():
    rng = np.random.default_rng(5)
    _, so, ids = _tiny_batch(rng, 20, 1, [1000])
    L = rng.integers(1, 9, size=20).astype(np.int32)
    perm, ro = O.balance_fbs(L, 1)
    bk = O.bucketize(ids, so, [1000], perm, ro, 1)
    n = ids.shape[1]
    assert bk["splits"].tolist() == [[n]]
    assert bk["shard_bm"].tolist() == list(range(n))  # shard-major = batch-major
    src = np.concatenate([ids[0][so[s]:so[s + 1]] for s in perm])
    assert np.array_equal(bk["shard_keys"], src)


def test_bucketize_drops_out_of_range_ids():
    so = np.array([0, 3, 5], np.int64)
    ids = np.array([[1, 50, 2, -1, 3]], np.int64)
    perm, ro = O.balance_fbs(np.array([3, 2], np.int32), 2)
    bk = O.bucketize(ids, so, [10], perm, ro, 2)
    assert bk["err"] & 1
    assert sorted(bk["shard_keys"].tolist()) == [1, 2, 3]
    assert bk["shard_offsets"][-1] == 3


def test_keyed_transpose_hand_example():
    """Two features, three samples; feature 0 has lengths 2, 0, 1 and feature 1
    has 1, 2, 0. Feature-major input: f0 = [10 11 | - | 12], f1 = [20 | 21 22 | -].
    Batch-major output: sample 0 = 10 11 20, sample 1 = 21 22, sample 2 = 12."""
    lengths = np.array([[2, 0, 1], [1, 2, 0]])
    values = np.array([10, 11, 12, 20, 21, 22])
    out, off = O.keyed_transpose(values, lengths)
    assert out.tolist() == [10, 11, 20, 21, 22, 12]
    # (b, f) starts: (0,0)=0 (0,1)=2 (1,0)=3 (1,1)=3 (2,0)=5 (2,1)=6, total 6
    assert off.tolist() == [0, 2, 3, 3, 5, 6, 6]


@pytest.mark.parametrize("F,B", [(1, 7), (3, 5), (6, 1), (4, 9)])
def test_keyed_transpose_twice_is_identity(F, B):
    """The batch-major output is a feature-major jagged tensor of B
    "features" over F "samples" (lengths transposed); transposing it back
    returns the input, and both offset lists agree with cumulative sums."""
    rng = np.random.default_rng(F * 31 + B)
    lengths = rng.integers(0, 5, size=(F, B))
    values = rng.integers(-10**12, 10**12, size=int(lengths.sum()))
    out, off = O.keyed_transpose(values, lengths)
    assert np.array_equal(off, np.concatenate([[0], np.cumsum(lengths.T.reshape(-1))]))
    back, off2 = O.keyed_transpose(out, lengths.T)
    assert np.array_equal(back, values)
    assert np.array_equal(off2, np.concatenate([[0], np.cumsum(lengths.reshape(-1))]))


@pytest.mark.parametrize("W,T", [(1, 1), (3, 2), (5, 3)])
def test_ranged_combine_inverts_the_dispatch(W, T):
    """Combine after dispatch is the identity: a row that carries an item's
    key lands in the batch-major slot of the token that holds that ID. The
    slot's token is found from the balanced order directly (sample perm[q],
    token j), not through the dispatch; dropped IDs leave their slot empty."""
    rng = np.random.default_rng(100 + W * 10 + T)
    R = [int(x) for x in rng.integers(4, 30, size=T)]
    N = 11
    _, so, ids = _tiny_batch(rng, N, T, R)
    ids[0, 0] = R[0] + 3  # one dropped ID
    L = rng.integers(1, 6, size=N).astype(np.int32)
    perm, ro = O.balance_fbs(L, W)
    bk = O.bucketize(ids, so, R, perm, ro, W)
    n_tok = ids.shape[1]
    nv = len(bk["shard_keys"])
    # row k: the item's key as 8 little-endian int64 copies (64 bytes), then
    # bytes (31 key + c) % 251 + 1 at column c, so a short or long copy shows
    row_bytes = [64 * (t + 1) for t in range(T)]  # row sizes differ per table
    stride = max(row_bytes) + 16
    src = np.zeros((nv, stride), np.uint8)
    src[:, :64] = np.repeat(bk["shard_keys"][:, None], 8, axis=1).view(np.uint8)
    cols = np.arange(64, stride)
    src[:, 64:] = ((31 * bk["shard_keys"][:, None] + cols[None, :]) % 251 + 1).astype(np.uint8)
    outs = O.ranged_combine(src, bk["shard_keys"], bk["shard_bm"], R, row_bytes, n_tok)
    row_base = np.concatenate([[0], np.cumsum(R)[:-1]])
    bm = 0
    for q in range(N):
        s_ = perm[q]
        for j in range(int(so[s_ + 1] - so[s_])):
            for t in range(T):
                id_ = int(ids[t, so[s_] + j])
                got = outs[t][bm]
                if 0 <= id_ < R[t]:
                    keys = got[:64].view(np.int64)
                    key = row_base[t] + id_
                    assert keys.tolist() == [key] * 8
                    c = np.arange(64, row_bytes[t])
                    assert np.array_equal(got[64:], ((31 * key + c) % 251 + 1).astype(np.uint8))
                else:
                    assert not got.any()
            bm += 1
    assert bm == n_tok


# ----------------------------------------------------------------------------
# dedup / CSR and collision


def test_unique_against_numpy():
    rng = np.random.default_rng(11)
    rows = [300, 50]
    W = 4
    _, so, ids = _tiny_batch(rng, 40, 2, rows, maxlen=30)
    L = rng.integers(1, 9, size=40).astype(np.int32)
    perm, ro = O.balance_fbs(L, W)
    bk = O.bucketize(ids, so, rows, perm, ro, W)
    uq = O.unique(bk["shard_keys"], bk["shard_bm"], rows, W)
    keys, bm = bk["shard_keys"], bk["shard_bm"]
    u_np, inv, cnt = np.unique(keys, return_inverse=True, return_counts=True)
    assert np.array_equal(uq["unique"], u_np)
    assert np.array_equal(np.diff(uq["seg_offsets"]), cnt)
    for u in range(len(u_np)):
        occ = uq["occ_bm"][uq["seg_offsets"][u]:uq["seg_offsets"][u + 1]]
        assert occ.tolist() == sorted(bm[inv == u].tolist())
        assert np.all(uq["occ_uid"][uq["seg_offsets"][u]:uq["seg_offsets"][u + 1]] == u)
    # every item exactly once
    assert sorted(uq["occ_bm"].tolist() + []) == sorted(bm.tolist())
    # (table, shard) groups
    rb = [0, 300]
    for t in range(2):
        block = -(-rows[t] // W)
        for d in range(W):
            lo, hi = uq["unique_offsets"][t * W + d], uq["unique_offsets"][t * W + d + 1]
            for k in uq["unique"][lo:hi]:
                assert (k - rb[t]) // block == d and rb[t] <= k < rb[t] + rows[t]


def test_collision_brute_force():
    rng = np.random.default_rng(2)
    for _ in range(20):
        a = np.unique(rng.integers(0, 40, size=rng.integers(0, 30)))
        b = np.unique(rng.integers(0, 40, size=rng.integers(0, 30)))
        cls, pcls, counts = O.collision(a, b)
        sa, sb = set(a.tolist()), set(b.tolist())
        assert cls.tolist() == [int(x in sb) for x in a.tolist()]
        assert pcls.tolist() == [int(x in sa) for x in b.tolist()]
        C = len(sa & sb)
        assert counts.tolist() == [len(a), C, len(a) - C, len(b) - C]
    a = np.arange(10)
    assert O.collision(a, a)[2][1] == 10
    assert O.collision(a, a + 100)[2][1] == 0
    assert O.collision(a, None)[2].tolist() == [10, 0, 10, 0]


# ----------------------------------------------------------------------------
# lookup, reduce, update


def _csr_from(keys, bm):
    return O.unique(np.asarray(keys, np.int64), np.asarray(bm, np.int32), [10_000], 1)


def test_lookup_decodes_row_and_column():
    # table value = row*1024 + col is exact in fp32: the output names its row
    R, D = 4000, 16
    vals = (np.arange(R)[:, None] * 1024 + np.arange(D)[None, :]).astype(np.float32)
    st = O.RowStore(np.arange(R), vals)
    rng = np.random.default_rng(4)
    n = 500
    keys = rng.integers(0, R, size=n)
    uq = _csr_from(keys, np.arange(n))
    out = O.lookup(st, 0, 0, len(uq["unique"]), uq, n)
    assert np.array_equal(out[:, 0] // 1024, keys.astype(np.float32))
    assert np.array_equal(out - out[:, :1], np.broadcast_to(np.arange(D, dtype=np.float32), out.shape))


def test_lookup_class_filter_and_bf16():
    R, D = 50, 8
    vals = np.arange(R * D, dtype=np.uint16).reshape(R, D)
    st = O.RowStore(np.arange(R), vals, bf16=True)
    keys = [3, 3, 7, 9, 7, 3]
    uq = _csr_from(keys, range(6))
    uq["cls"] = np.array([1, 0, 1], np.uint8)  # rows 3 and 9 collide
    out = np.full((6, D), 0xFFFF, np.uint16)
    O.lookup(st, 0, 0, 3, uq, 6, which=1, out=out)
    for i, k in enumerate(keys):
        exp = vals[k] if k in (3, 9) else np.full(D, 0xFFFF, np.uint16)
        assert np.array_equal(out[i], exp)


def test_reduce_counts_and_one_hot():
    rng = np.random.default_rng(8)
    n, D = 3000, 8
    keys = rng.zipf(1.3, size=n) % 200
    uq = _csr_from(keys, np.arange(n))
    U = len(uq["unique"])
    ones = np.ones((n, D), np.float32)
    g = O.reduce(D, 0, U, uq, ones)
    assert np.array_equal(g[:, 0], np.diff(uq["seg_offsets"]).astype(np.float32))
    # one-hot in the column = bm % D, value = bm: each row's sum lists its bms
    oh = np.zeros((n, D), np.float32)
    oh[np.arange(n), np.arange(n) % D] = np.arange(n)
    g = O.reduce(D, 0, U, uq, oh)
    for u in range(U):
        bms = np.nonzero(keys == uq["unique"][u])[0]
        exp = np.zeros(D)
        np.add.at(exp, bms % D, bms)
        assert np.array_equal(g[u], exp.astype(np.float32))


def test_reduce_is_exactly_rounded_sum():
    rng = np.random.default_rng(9)
    n, D = 4000, 4
    keys = rng.integers(0, 3, size=n)
    grad = (rng.standard_normal((n, D)) * np.exp(rng.uniform(-20, 20, (n, D)))).astype(np.float32)
    uq = _csr_from(keys, np.arange(n))
    g = O.reduce(D, 0, 3, uq, grad)
    for u in range(3):
        for d in range(D):
            exact = math.fsum(float(x) for x in grad[keys == uq["unique"][u], d])
            # fp64 accumulation of 1300 terms: within 1e-13 of the exact sum's scale
            assert abs(float(g[u, d]) - exact) <= abs(exact) * 2 ** -23 + 1e-12 * np.abs(
                grad[keys == uq["unique"][u], d]).astype(np.float64).sum()


def test_sgd_matches_torch():
    import torch
    rng = np.random.default_rng(1)
    R, D = 30, 16
    w0 = rng.standard_normal((R, D)).astype(np.float32) * 0.01
    keys = rng.integers(0, R, size=200)
    grad = rng.standard_normal((200, D)).astype(np.float32)
    uq = _csr_from(keys, np.arange(200))
    U = len(uq["unique"])
    g = O.reduce(D, 0, U, uq, grad)
    st = O.RowStore(np.arange(R), w0.copy())
    O.update(st, 0, 0, U, uq["unique"], g, "sgd", 0.01, 0.0)
    p = torch.nn.Parameter(torch.from_numpy(w0.copy()))
    opt = torch.optim.SGD([p], lr=0.01)
    gt = torch.zeros(R, D)
    gt[torch.from_numpy(uq["unique"])] = torch.from_numpy(g)
    p.grad = gt
    opt.step()
    # torch may fuse the multiply-add (one rounding); ours rounds lr*g first
    # (two roundings of the operands' scale apart at most, even under cancellation)
    ref = p.detach().numpy()
    scale = np.maximum(np.abs(w0), np.abs(ref - w0)).astype(np.float32)
    assert np.all(np.abs(st.vals - ref) <= 2 * np.spacing(scale))


def test_rowwise_adagrad_dim1_matches_torch_adagrad():
    # with one column, row-wise Adagrad is torch's element-wise Adagrad
    import torch
    rng = np.random.default_rng(2)
    R = 64
    w0 = rng.standard_normal((R, 1)).astype(np.float32)
    st = O.RowStore(np.arange(R), w0.copy())
    p = torch.nn.Parameter(torch.from_numpy(w0.copy()))
    opt = torch.optim.Adagrad([p], lr=0.05, eps=1e-8, initial_accumulator_value=0.0)
    for it in range(3):
        g = rng.standard_normal((R, 1)).astype(np.float32)
        O.update(st, 0, 0, R, np.arange(R), g, "rw_adagrad", 0.05, 1e-8)
        p.grad = torch.from_numpy(g.copy())
        opt.step()
        # torch divides g by the root first; ours scales lr first: ulp-level apart
        np.testing.assert_allclose(st.vals, p.detach().numpy(), rtol=4e-7, atol=1e-9)
    np.testing.assert_allclose(st.state, opt.state[p]["sum"].numpy().ravel(), rtol=2.5e-7)


def test_rowwise_adagrad_closed_form():
    # |g_d| = c on every column: state = c^2 after one step, step = lr*g/(c+eps)
    R, D, c = 5, 64, 0.375  # exact binary fraction
    w0 = np.zeros((R, D), np.float32)
    st = O.RowStore(np.arange(R), w0.copy())
    signs = np.where(np.random.default_rng(0).random((R, D)) < 0.5, -1.0, 1.0)
    g = (signs * c).astype(np.float32)
    O.update(st, 0, 0, R, np.arange(R), g, "rw_adagrad", 0.05, 1e-8)
    assert np.all(st.state == np.float32(c * c))
    np.testing.assert_allclose(st.vals, -0.05 * g / (c + 1e-8), rtol=1e-6)
    # a single non-zero column: the accumulator is the MEAN over columns
    st2 = O.RowStore(np.arange(1), np.zeros((1, D), np.float32))
    g1 = np.zeros((1, D), np.float32)
    g1[0, 3] = 2.0
    O.update(st2, 0, 0, 1, np.arange(1), g1, "rw_adagrad", 1.0, 0.0)
    assert st2.state[0] == np.float32(4.0 / D)
    assert st2.vals[0, 3] == np.float32(-2.0 / math.sqrt(4.0 / D))


def test_bf16_rounding_matches_torch():
    import torch
    rng = np.random.default_rng(3)
    x = np.concatenate([rng.standard_normal(5000).astype(np.float32) * 0.01,
                        np.array([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 1.0 + 2 ** -9, -1.0 - 2 ** -8,
                                  3.4e38, -3.4e38, np.inf, -np.inf, 0.0, -0.0, 1e-40],
                                 np.float32)])
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().astype(np.uint16)
    got = np.array([O.f32_to_bf16(float(v)) for v in x], np.uint16)
    assert np.array_equal(got, ref)
    nan = O.f32_to_bf16(float("nan"))
    assert (nan & 0x7F80) == 0x7F80 and (nan & 0x7F)
    for h in [0x3F80, 0xBF81, 0x0001, 0x7F7F]:
        ref = torch.from_numpy(np.array([h], np.uint16).view(np.int16)).view(torch.bfloat16)
        assert np.float32(O.bf16_to_f32(h)) == ref.float().item()


def test_bf16_update_rounds_once():
    # bf16 rows widen exactly, update in fp32, round-to-nearest-even on store
    import torch
    D = 32
    w0 = torch.randn(1, D).mul(0.01).to(torch.bfloat16)
    g = np.random.default_rng(0).standard_normal((1, D)).astype(np.float32)
    st = O.RowStore([0], w0.view(torch.int16).numpy().astype(np.uint16), bf16=True)
    O.update(st, 0, 0, 1, np.arange(1), g, "sgd", 0.01, 0.0)
    ref = (w0.float() - torch.from_numpy(g) * np.float32(0.01)).to(torch.bfloat16)
    assert np.array_equal(st.vals, ref.view(torch.int16).numpy().astype(np.uint16))


# ----------------------------------------------------------------------------
# the synchronous loop (FreeScale section 3.2: the synchronized baseline that a
# strict write-then-read order on collision rows reproduces)


def _loop_workload(optim="sgd", lr=0.25, eps=0.0, rows=16, dim=4, W=2):
    from jagged_embedding_sparse_amd import synth
    return synth.Workload("loop-pin", 4, W, (synth.TableSpec(rows, dim, "f32", 1.0),), optim,
                          lr, eps, "fbs", (1, 1), 2, ("lognormal", 1.0, 1.0), 8, 0)


def _hand_batch(samples):
    """One table; sample s holds the IDs samples[s] (all UIH tokens)."""
    lens = np.array([len(x) for x in samples], np.int32)
    so = np.zeros(len(samples) + 1, np.int64)
    so[1:] = np.cumsum(lens)
    ids = np.array([[i for x in samples for i in x]], np.int64)
    return dict(uih_len=lens, num_cand=np.zeros(len(samples), np.int32), sample_offsets=so,
                ids=ids, n_tok=int(so[-1]))


def _row_grid(rows, dim):
    # row r, column c holds r + c/16: every value and every SGD step below is exact
    return (np.arange(rows, dtype=np.float32)[:, None]
            + np.arange(dim, dtype=np.float32)[None, :] / 16).astype(np.float32)


def _ids_by_bm(batch, out):
    """Row ID at every balanced batch-major slot of one iteration's outputs."""
    perm, bal = out["perm"], out["bucket"]["bal_offsets"]
    so = batch["sample_offsets"]
    tok = np.concatenate([np.arange(so[s], so[s + 1]) for s in perm]) if len(perm) else []
    assert len(tok) == bal[-1]
    return batch["ids"][0][np.asarray(tok, np.int64)]


def _run_loop(w, batches, grad_value=1.0):
    rows, dim = w.tables[0].rows, w.tables[0].dim
    w0 = _row_grid(rows, dim)
    store = O.RowStore(np.arange(rows), w0.copy())
    run = O.SyncRun(w, [store])
    outs = []
    for b in batches:
        outs.append(run.step(b, lambda o, b=b: [np.full((b["n_tok"], dim), grad_value,
                                                        np.float32)]))
    return w0, store, outs


def _occ(batch):
    ids, cnt = np.unique(batch["ids"][0], return_counts=True)
    return dict(zip(ids.tolist(), cnt.tolist()))


def test_sync_loop_sgd_two_iterations():
    """Iteration 1 reads the rows as iteration 0 updated them (w0 - lr*k for
    a row iteration 0 touched k times with all-ones gradients, w0 otherwise);
    iteration 0 reads the initial rows; the split is against iteration 0's
    rows; the final rows carry both updates."""
    w = _loop_workload()
    b0 = _hand_batch([[1, 3, 3], [5], [1, 7], [9, 9, 9, 1]])
    b1 = _hand_batch([[1, 2], [3, 11], [9], [12, 1]])
    w0, store, outs = _run_loop(w, [b0, b1])
    k0, k1 = _occ(b0), _occ(b1)
    # iteration 0: the initial rows, at every slot
    ids0 = _ids_by_bm(b0, outs[0])
    assert np.array_equal(outs[0]["emb"][0], w0[ids0])
    # iteration 1: rows seen in iteration 0 moved by lr * k, the others did not
    ids1 = _ids_by_bm(b1, outs[1])
    exp1 = np.stack([w0[r] - np.float32(0.25 * k0.get(int(r), 0)) for r in ids1])
    assert np.array_equal(outs[1]["emb"][0], exp1)
    # the split: U1 = {1, 2, 3, 9, 11, 12}, C = {1, 3, 9}, U0 = {1, 3, 5, 7, 9}
    assert outs[0]["counts"].tolist() == [5, 0, 5, 0]
    assert outs[1]["counts"].tolist() == [6, 3, 3, 2]
    assert outs[1]["uniq"]["cls"].tolist() == [1, 0, 1, 1, 0, 0]  # rows 1 2 3 9 11 12
    assert outs[1]["prev_cls"].tolist() == [1, 1, 0, 0, 1]  # rows 1 3 5 7 9
    # the reduced gradient of each row is its occurrence count
    assert outs[1]["reduced"][0][:, 0].tolist() == [k1[r] for r in (1, 2, 3, 9, 11, 12)]
    # final rows: both updates
    for r in range(16):
        k = k0.get(r, 0) + k1.get(r, 0)
        assert np.array_equal(store.vals[r], w0[r] - np.float32(0.25 * k)), r


def test_sync_loop_identical_and_disjoint_batches():
    """Identical consecutive batches give C = U (every row of both iterations
    collides); disjoint ones give C = 0."""
    w = _loop_workload()
    b = _hand_batch([[4, 4], [6], [8, 4], [6, 10, 15]])
    _, _, outs = _run_loop(w, [b, _hand_batch([[4, 4], [6], [8, 4], [6, 10, 15]])])
    U = len(np.unique(b["ids"][0]))
    assert outs[1]["counts"].tolist() == [U, U, 0, 0]
    assert np.all(outs[1]["uniq"]["cls"] == 1) and np.all(outs[1]["prev_cls"] == 1)
    _, _, outs = _run_loop(w, [b, _hand_batch([[0, 1], [2], [3, 5], [7, 9, 11]])])
    assert outs[1]["counts"].tolist() == [8, 0, 8, U]
    assert np.all(outs[1]["uniq"]["cls"] == 0) and np.all(outs[1]["prev_cls"] == 0)


def test_sync_loop_rowwise_adagrad_closed_form():
    """Row-wise Adagrad with all-ones gradients (eps = 0): a row touched k
    times gets g = k on every column, so s = k^2 and w - lr * g / sqrt(s) =
    w - lr; iteration 1 reads that, and a row touched k0 then k1 times ends at
    s = k0^2 + k1^2."""
    w = _loop_workload(optim="rw_adagrad", lr=0.25, eps=0.0)
    b0 = _hand_batch([[1, 3, 3], [5], [1, 7], [9, 9, 9, 1]])
    b1 = _hand_batch([[1, 2], [3, 11], [9], [12, 1]])
    w0, store, outs = _run_loop(w, [b0, b1])
    k0, k1 = _occ(b0), _occ(b1)
    ids1 = _ids_by_bm(b1, outs[1])
    exp1 = np.stack([w0[r] - np.float32(0.25 if r in k0 else 0.0) for r in ids1])
    np.testing.assert_allclose(outs[1]["emb"][0], exp1, rtol=0, atol=1e-6)
    for r in range(16):
        s = k0.get(r, 0) ** 2 + k1.get(r, 0) ** 2
        assert store.state[r] == np.float32(s), r
        exp = w0[r] - (0.25 if r in k0 else 0) - (0.25 * k1[r] / math.sqrt(s) if r in k1 else 0)
        np.testing.assert_allclose(store.vals[r], exp, rtol=0, atol=1e-6)
