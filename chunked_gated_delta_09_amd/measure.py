"""Binding of the library's measurement extension (``include/kda_measure.h``): HIP events
recorded around each kernel launch of a call, for per-kernel timing. Not needed to use the
library; bench.py uses it."""
from __future__ import annotations

import ctypes

from . import load

_fn = None


def set_kernel_events(events, count):
    """Record events[2i] / events[2i+1] around the i-th kernel launch of each later call on
    this thread (``events`` a ctypes array of hipEvent_t, or None to stop)."""
    global _fn
    if _fn is None:
        _fn = load().kda_set_kernel_events
        _fn.restype = None
        _fn.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_int]
    _fn(events, count)


def bwd_state_grads(dims, workspace, stream=None):
    """The per-chunk state gradients (dS_out of every chunk, [NT, HV, K, V] fp32) that the
    reverse scan of the last kda_chunk_bwd call made with ``workspace`` left in it."""
    import torch

    from . import Dims, _check, _stream, num_chunks
    lib = load()
    fn = lib.kda_bwd_state_grads
    fn.restype = ctypes.c_int
    fn.argtypes = [ctypes.POINTER(Dims), ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_void_p]
    nt = num_chunks(dims)
    out = torch.empty(nt, dims.HV, dims.K, dims.V, dtype=torch.float32, device=workspace.device)
    st = _stream() if stream is None else ctypes.c_void_p(stream)
    _check(fn(ctypes.byref(dims), ctypes.c_void_p(workspace.data_ptr()), workspace.numel(),
              ctypes.c_void_p(out.data_ptr()), st))
    return out
