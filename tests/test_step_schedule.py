"""The step's own control flow on the CPU, with the launches replaced by a log.

The three-ahead schedules (joined, and Algorithm 2's prioritized order) run
their prologue, steps, join and epilogue over stand-in streams and events:
every iteration's index stages are issued once and in order, on the two
index streams in turn, each against the iteration before it, and each
iteration is looked up only after its own index stages and those of the
iteration before it (whose unique rows its collision split reads) were
issued; the update of iteration i comes after the lookup of i.
"""

from collections import deque

import pytest
import torch

from jagged_embedding_sparse_amd.step import IterState, SparseStep


class _FakeEvent:
    def record(self, stream=None):
        pass

    def wait(self, stream=None):
        pass

    def query(self):
        return False


class _FakeStream:
    cuda_stream = 0

    def wait_event(self, ev):
        ev.wait(self)

    def wait_stream(self, s):
        pass


@pytest.mark.timeout(60)
@pytest.mark.parametrize("schedule", ["joined", "prioritized"])
def test_three_ahead_schedule_order_on_stubs(monkeypatch, schedule):
    log = []
    cs = _FakeStream()
    monkeypatch.setattr(torch.cuda, "current_stream", lambda *a, **k: cs)
    s = object.__new__(SparseStep)
    s.schedule, s.lookahead, s.graph = schedule, 3, False
    s._capture, s._dry, s.timer = None, False, None
    s.autotune, s.split_update = None, "auto"
    s.states_buf = [IterState(slot=i) for i in range(4)]
    for st in s.states_buf:
        st.ev_uq, st.ev_done, st.ev_bal = _FakeEvent(), _FakeEvent(), _FakeEvent()
    s.s_idx = [_FakeStream(), _FakeStream()]
    s.sA, s.sB = s.s_idx[0], _FakeStream()
    s.sC = _FakeStream() if schedule == "prioritized" else None
    s._ahead, s._n_indexed, s.cur, s.slot = deque(), 0, None, 0
    s._ev_idx = [_FakeEvent(), _FakeEvent()]
    s._ev_fork, s._ev_join, s._cs_ev = _FakeEvent(), _FakeEvent(), None
    s.ws_red = [None, None]
    s._forked = []

    def index_stages(batch, st, prev, stream, x=0):
        # the bookkeeping the real stages do, then the log
        st.idx_x, st.n_tok, st.it = x, int(batch["ids"].shape[1]), batch["it"]
        s._n_indexed += 1
        log.append(("index", batch["it"], x, None if prev is None else prev.it))

    monkeypatch.setattr(s, "_index_stages", index_stages)
    monkeypatch.setattr(s, "_lookup", lambda st, which, stream: log.append(("lookup", st.it)))
    monkeypatch.setattr(s, "_run_update", lambda st, *a, **k: log.append(("update", st.it)))
    K = 12
    batches = [dict(it=i, ids=torch.zeros((1, 10 + i))) for i in range(K)]
    s.prologue(batches[0], batch_after=batches[1:3])
    for i in range(1, K):
        s.step(batches[i], [], batch_after=batches[i + 2] if i + 2 < K else None)
    s.join()
    s.epilogue([])
    idx = [e for e in log if e[0] == "index"]
    assert [e[1] for e in idx] == list(range(K))
    assert [e[2] for e in idx] == [i % 2 for i in range(K)]
    assert [e[3] for e in idx] == [None] + list(range(K - 1))
    seen, looked, updated = set(), [], []
    for e in log:
        if e[0] == "index":
            seen.add(e[1])
        elif e[0] == "lookup":  # the prioritized schedule looks up twice (by class)
            j = e[1]
            assert j in seen and (j == 0 or j - 1 in seen)
            if not looked or looked[-1] != j:
                looked.append(j)
        else:
            j = e[1]
            assert j in looked
            if not updated or updated[-1] != j:
                updated.append(j)
    assert looked == list(range(K))
    assert updated == list(range(K))
