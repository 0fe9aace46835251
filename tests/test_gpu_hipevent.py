"""HipEvent (events without the system-scope fence) orders streams of one GPU
and times work like torch's events.

Stream A writes a buffer with a chain of kernels long enough to still run
when stream B is told to wait; B waits for A's event and then copies the
buffer: the copy must see every write. The elapsed time of a span around A's
chain must be positive and agree with torch's events around the same chain.
"""

import pytest
import torch

from jagged_embedding_sparse_amd.hipevent import HipEvent

pytestmark = pytest.mark.gpu


def test_never_recorded_event_is_a_no_op():
    ev = HipEvent()
    assert ev.query()
    ev.wait(torch.cuda.current_stream())  # nothing recorded: nothing to wait for
    ev.synchronize()


def test_wait_orders_streams_and_query_completes():
    torch.cuda.set_device(0)
    sa, sb = torch.cuda.Stream(), torch.cuda.Stream()
    n = 1 << 24
    x = torch.zeros(n, dtype=torch.float32, device="cuda")
    out = torch.empty_like(x)
    torch.cuda.synchronize()
    for trial in range(3):
        ev = HipEvent()
        with torch.cuda.stream(sa):
            for k in range(1, 41):  # 40 dependent passes over 64 MB
                x.add_(1.0)
            ev.record(sa)
        sb.wait_event(ev)  # torch's wait_event calls ev.wait(sb)
        with torch.cuda.stream(sb):
            out.copy_(x)
        torch.cuda.synchronize()
        assert ev.query()
        expect = 40.0 * (trial + 1)
        assert torch.all(out == expect).item(), (trial, out.min().item(), out.max().item())


def test_elapsed_time_matches_torch_events():
    torch.cuda.set_device(0)
    s = torch.cuda.current_stream()
    x = torch.zeros(1 << 24, dtype=torch.float32, device="cuda")
    h0, h1 = HipEvent(enable_timing=True), HipEvent(enable_timing=True)
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record(s)
    h0.record(s)
    for _ in range(50):
        x.add_(1.0)
    h1.record(s)
    t1.record(s)
    torch.cuda.synchronize()
    hip_ms, torch_ms = h0.elapsed_time(h1), t0.elapsed_time(t1)
    assert hip_ms > 0
    # the torch pair brackets the HipEvent pair
    assert hip_ms <= torch_ms * 1.01 + 0.01, (hip_ms, torch_ms)
    assert hip_ms >= 0.5 * torch_ms, (hip_ms, torch_ms)
