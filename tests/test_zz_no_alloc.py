"""The allocation-free update against the workspace-taking one.

fs_grad_reduce_update_noalloc keeps the long rows' fp64 partial sums in the
library's fixed per-GPU scratch instead of a caller workspace. Both entry
points run on identical copies of the tables with the same gradients and
CSR, two calls in a row (the second on a smaller batch, so it runs over what
the first left in the scratch), with rows long enough to be split over many
chunks; reduced gradients, rows and Adagrad state must agree bit for bit.
"""

import numpy as np
import pytest
import torch

from jagged_embedding_sparse_amd import lib

pytestmark = pytest.mark.gpu


def say(*a):
    print("[case]", *a, flush=True)


def _csr(ids, rows, W):
    """Unique keys, (table, shard) offsets and the occurrence CSR of int64
    ids [T, n_tok], with bm = token index (plain numpy: a valid input for
    both entry points)."""
    T, n = ids.shape
    rb = np.concatenate([[0], np.cumsum(rows)[:-1]]).astype(np.int64)
    keys = (ids + rb[:, None]).ravel()
    bm = np.tile(np.arange(n, dtype=np.int32), T)
    order = np.argsort(keys, kind="stable")
    ks, occ_bm = keys[order], bm[order]
    uq, first, cnt = np.unique(ks, return_index=True, return_counts=True)
    seg = np.append(first, len(ks)).astype(np.int32)
    occ_uid = np.repeat(np.arange(len(uq), dtype=np.int32), cnt)
    t_of = np.searchsorted(rb, uq, side="right") - 1
    block = np.array([-(-r // W) for r in rows], np.int64)
    gid = t_of * W + (uq - rb[t_of]) // block[t_of]
    uo = np.searchsorted(gid, np.arange(T * W + 1), side="left").astype(np.int64)
    c = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()  # noqa: E731
    return dict(unique=c(uq), unique_offsets=c(uo), seg_offsets=c(seg), occ_bm=c(occ_bm),
                occ_uid=c(occ_uid)), len(uq)


def _ids(rng, rows, n_tok, hot):
    """Uniform IDs per table plus forced hot rows [(row, count)] in table 0."""
    ids = np.stack([rng.integers(0, r, size=n_tok) for r in rows]).astype(np.int64)
    pos = rng.permutation(n_tok)
    k = 0
    for r, cnt in hot:
        ids[0, pos[k:k + cnt]] = r
        k += cnt
    return ids


CASES = [
    # tables (rows, dim, dtype), optimizer, W, [(n_tok, hot rows)] of the two calls
    ([(200_000, 128, torch.bfloat16), (50_000, 64, torch.float32)], "rw_adagrad", 16,
     [(300_000, [(3, 60_000), (9, 5_000), (11, 700)]), (120_000, [(3, 20_000), (5, 900)])]),
    ([(30_000, 256, torch.float32)], "sgd", 4,
     [(200_000, [(1, 90_000), (2, 513)]), (50_000, [(7, 10_000)])]),
    ([(4_000, 1024, torch.float32)], "rw_adagrad", 8,
     [(60_000, [(0, 30_000)]), (20_000, [(0, 5_000), (1, 4_000)])]),
]


@pytest.mark.parametrize("case", CASES, ids=["2tables-bf16-adagrad", "D256-sgd", "D1024-adagrad"])
def test_noalloc_matches_workspace_update(case):
    specs, optim, W, calls = case
    rows = [r for r, _, _ in specs]
    say("noalloc", [(r, d, str(dt)) for r, d, dt in specs], optim, W, [n for n, _ in calls])
    g = torch.Generator(device="cuda").manual_seed(5)
    wa = [(torch.randn(r, d, device="cuda", generator=g) * 0.01).to(dt) for r, d, dt in specs]
    wb = [x.clone() for x in wa]
    ada = optim == "rw_adagrad"
    sa = [torch.zeros(r, device="cuda") if ada else None for r in rows]
    sb = [x.clone() if x is not None else None for x in sa]
    rng = np.random.default_rng(11)
    for call, (n_tok, hot) in enumerate(calls):
        ids = _ids(rng, rows, n_tok, hot)
        uq, U = _csr(ids, rows, W)
        grads = [torch.randn(n_tok, d, device="cuda", generator=g) for _, d, _ in specs]
        cls = torch.from_numpy((rng.random(U) < 0.4).astype(np.uint8)).cuda()
        # the first call splits the update by class (collision rows, then the
        # rest), the second updates every row at once
        whichs = (lib.FS_COLLISION, lib.FS_EXCLUSIVE) if call == 0 else (lib.FS_ALL,)
        for which in whichs:
            ra = [torch.full((U, d), float("nan"), device="cuda") for _, d, _ in specs]
            rb = [x.clone() for x in ra]
            lib.fs_grad_reduce_update(wa, sa, W, grads, n_tok, uq, optim, 0.05, 1e-8,
                                      which=which, cls=cls, reduced_out=ra)
            lib.fs_grad_reduce_update_noalloc(wb, sb, W, grads, n_tok, uq, optim, 0.05, 1e-8,
                                              which=which, cls=cls, reduced_out=rb)
            torch.cuda.synchronize()
            for t in range(len(specs)):
                assert torch.equal(ra[t].isnan(), rb[t].isnan()), (call, which, t)
                assert torch.equal(ra[t].nan_to_num(0.0), rb[t].nan_to_num(0.0)), (call, which, t)
        for t in range(len(specs)):
            a = wa[t].view(torch.int16) if wa[t].dtype == torch.bfloat16 else wa[t]
            b = wb[t].view(torch.int16) if wb[t].dtype == torch.bfloat16 else wb[t]
            assert torch.equal(a, b), (call, t)
            if ada:
                assert torch.equal(sa[t], sb[t]), (call, t)
        say("call", call, "n_tok", n_tok, "U", U, "equal")
