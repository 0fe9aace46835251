"""HIP events without a system-scope fence, for ordering streams of one GPU.

An event recorded the default way ends with a system-scope release: the GPU
writes back and invalidates its caches so that the host and other devices see
the work before the event. Events that only order streams of the same GPU, or
only time its work, need none of that. HIP's hipEventDisableSystemFence flag
drops it (measured on the sparse step, same GPU, two runs each: the
four-table workload 0.436 -> 0.431 ms per step, the others within 1%); a
wait on such an event also costs the host less than one on torch's (4.9
against 6.4 us). torch's events cannot set the flag, so this module creates
them through the HIP runtime torch has already loaded (one runtime per
process: torch's copy and the one the library links share their soname).

`HipEvent` has the methods the step and its timers use from torch.cuda.Event:
record(stream), wait(stream) (so that torch's Stream.wait_event accepts it),
query(), synchronize() and elapsed_time(end). The HIP event is created at the
first record, like torch's, so constructing one needs no GPU.
"""

from __future__ import annotations

import ctypes as C
import os

import torch

hipEventDisableTiming = 0x2
hipEventDisableSystemFence = 0x20000000
hipSuccess, hipErrorNotReady = 0, 600

_hip = None


def _runtime():
    global _hip
    if _hip is None:
        torch.cuda.init()  # loads and initialises the runtime torch uses
        mode = getattr(os, "RTLD_NOLOAD", 0) | getattr(os, "RTLD_LAZY", 1)
        h = C.CDLL("libamdhip64.so.7", mode=mode)
        P = C.c_void_p
        for name, res, args in (
                ("hipEventCreateWithFlags", C.c_int, [C.POINTER(P), C.c_uint]),
                ("hipEventRecord", C.c_int, [P, P]),
                ("hipStreamWaitEvent", C.c_int, [P, P, C.c_uint]),
                ("hipEventQuery", C.c_int, [P]),
                ("hipEventSynchronize", C.c_int, [P]),
                ("hipEventElapsedTime", C.c_int, [C.POINTER(C.c_float), P, P]),
                ("hipEventDestroy", C.c_int, [P])):
            fn = getattr(h, name)
            fn.restype, fn.argtypes = res, args
        _hip = h
    return _hip


def _check(name, rc):
    if rc != hipSuccess:
        raise RuntimeError(f"{name} failed: HIP error {rc}")


class HipEvent:
    """A HIP event recorded without the system-scope fence (see module doc)."""

    __slots__ = ("timing", "_ev", "_recorded")

    def __init__(self, enable_timing: bool = False):
        self.timing = bool(enable_timing)
        self._ev = None
        self._recorded = False

    def _create(self):
        h = _runtime()
        ev = C.c_void_p()
        flags = hipEventDisableSystemFence | (0 if self.timing else hipEventDisableTiming)
        _check("hipEventCreateWithFlags", h.hipEventCreateWithFlags(C.byref(ev), flags))
        self._ev = ev

    def record(self, stream=None):
        if self._ev is None:
            self._create()
        s = stream if stream is not None else torch.cuda.current_stream()
        _check("hipEventRecord", _hip.hipEventRecord(self._ev, s.cuda_stream))
        self._recorded = True

    def wait(self, stream=None):
        """`stream` waits for the work before the last record (none if never
        recorded)."""
        if not self._recorded:
            return
        s = stream if stream is not None else torch.cuda.current_stream()
        _check("hipStreamWaitEvent", _hip.hipStreamWaitEvent(s.cuda_stream, self._ev, 0))

    def query(self) -> bool:
        if not self._recorded:
            return True
        rc = _hip.hipEventQuery(self._ev)
        if rc == hipErrorNotReady:
            return False
        _check("hipEventQuery", rc)
        return True

    def synchronize(self):
        if self._recorded:
            _check("hipEventSynchronize", _hip.hipEventSynchronize(self._ev))

    def elapsed_time(self, end: "HipEvent") -> float:
        """Milliseconds from this event's record to `end`'s."""
        ms = C.c_float()
        _check("hipEventElapsedTime", _hip.hipEventElapsedTime(C.byref(ms), self._ev, end._ev))
        return float(ms.value)

    def __del__(self):
        if self._ev is not None and _hip is not None:
            try:
                _hip.hipEventDestroy(self._ev)
            except Exception:
                pass
