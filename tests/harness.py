"""Shared helpers of the GPU parity tests: uploads, gradient layout, and the
oracle's synchronous run over the same seeded batches.

Every expected value comes from oracle/ (or from the pages via the pins);
nothing here reads a GPU result back into an oracle input.
"""

from __future__ import annotations

import numpy as np
import torch

from jagged_embedding_sparse_amd import lib, synth
from oracle import oracle as O


def to_dev(batch):
    return dict(uih_len=torch.from_numpy(np.ascontiguousarray(batch["uih_len"])).cuda(),
                sample_offsets=torch.from_numpy(batch["sample_offsets"]).cuda(),
                ids=torch.from_numpy(np.ascontiguousarray(batch["ids"])).cuda(),
                n_tok=batch["n_tok"])


def host(t):
    return t.detach().cpu().numpy()


def orig_token_of_bm(so, perm, bal):
    """Original token index of every balanced batch-major slot."""
    lens = np.diff(bal)
    starts = so[perm]
    return np.repeat(starts - bal[:-1], lens) + np.arange(bal[-1])


def balanced_grads(w, seed, it, batch, perm, bal):
    """fp32 gradient rows of iteration `it` in the balanced batch-major order.

    Keyed by the original (sample, token) through synth's counter hash, so the
    same token has the same gradient whatever the balancer does."""
    tok = orig_token_of_bm(batch["sample_offsets"], perm, bal)
    return [synth.gradient_rows(seed, it, t, tok, spec.dim) for t, spec in enumerate(w.tables)]


def touched_rows(batches, w):
    """Ascending table-local row ids each table touches over all batches."""
    out = []
    for t, spec in enumerate(w.tables):
        ids = np.concatenate([b["ids"][t] for b in batches])
        ids = ids[(ids >= 0) & (ids < spec.rows)]
        out.append(np.unique(ids))
    return out


def gpu_tables(w, seed, align=0):
    """Device tables of workload w: dense (align 0), or each row's state in
    the row's own slot of `align`-rounded bytes (lib.alloc_table)."""
    weights, states = [], []
    ada = w.optim == "rw_adagrad"
    for t, spec in enumerate(w.tables):
        if align:
            tdt = torch.float32 if spec.dtype == "f32" else torch.bfloat16
            wv, st = lib.alloc_table(spec.rows, spec.dim, tdt, ada, device="cuda", align=align)
            weights.append(synth.init_table(spec.rows, spec.dim, spec.dtype, seed, "cuda",
                                            table=t, out=wv))
            states.append(st.zero_() if st is not None else None)
        else:
            weights.append(synth.init_table(spec.rows, spec.dim, spec.dtype, seed, "cuda",
                                            table=t))
            states.append(torch.zeros(spec.rows, dtype=torch.float32, device="cuda")
                          if ada else None)
    return weights, states


def snapshot_stores(weights, states, rows_per_table):
    """Oracle row stores holding the initial value of every touched row."""
    stores = []
    for t, (wt, rid) in enumerate(zip(weights, rows_per_table)):
        idx = torch.from_numpy(rid).cuda()
        vals = wt.index_select(0, idx)
        if wt.dtype == torch.bfloat16:
            v = host(vals.view(torch.int16)).view(np.uint16)
        else:
            v = host(vals)
        st = host(states[t].index_select(0, idx)) if states[t] is not None else None
        stores.append(O.RowStore(rid, v, st, bf16=wt.dtype == torch.bfloat16))
    return stores


def rows_now(weights, states, t, rid):
    idx = torch.from_numpy(rid).cuda()
    vals = weights[t].index_select(0, idx)
    if weights[t].dtype == torch.bfloat16:
        v = host(vals.float())
    else:
        v = host(vals)
    st = host(states[t].index_select(0, idx)) if states[t] is not None else None
    return v, st


def store_vals_f32(store):
    if store.bf16:
        return (store.vals.astype(np.uint32) << 16).view(np.float32)
    return store.vals


def rel_err_rows(got, ref, prev):
    """|got - ref| / (|prev| + |ref - prev|): the error relative to the size of
    the values the update combined, meaningful under cancellation."""
    den = np.abs(prev) + np.abs(ref - prev)
    den = np.where(den == 0, 1.0, den)
    return float(np.max(np.abs(got.astype(np.float64) - ref) / den)) if got.size else 0.0
