"""MI355X (gfx950) KDA chunk library: Python binding of the C ABI in ``include/kda.h``.

Only argument marshalling lives here: checking tensors, allocating outputs and workspace
through torch's caching allocator, and passing raw device pointers and the current HIP
stream to ``libkda.so``. Every step of the computation runs in the library's HIP kernels.
The binding raises if the library has not been built; there is no fallback path.
"""
from __future__ import annotations

import ctypes
import math
import os

__all__ = ["load", "fwd_states", "chunk_bwd", "chunk_bwd_into", "chunk_bwd_noalloc_into", "make_dims", "num_chunks",
           "fwd_workspace_bytes", "bwd_workspace_bytes", "saved_bytes", "KdaError", "LIB_PATH"]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libkda.so")

KDA_F32, KDA_BF16 = 0, 1
_STATUS = {0: "KDA_OK", -1: "KDA_EINVAL", -2: "KDA_EUNSUPPORTED", -3: "KDA_EHIP"}


class KdaError(RuntimeError):
    def __init__(self, status, msg):
        super().__init__(f"{_STATUS.get(status, status)}: {msg}")
        self.status = status


class Dims(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("T", ctypes.c_int32), ("H", ctypes.c_int32), ("HV", ctypes.c_int32),
                ("K", ctypes.c_int32), ("V", ctypes.c_int32), ("C", ctypes.c_int32), ("N", ctypes.c_int32),
                ("cu_seqlens_dev", ctypes.c_void_p), ("cu_seqlens_host", ctypes.POINTER(ctypes.c_int32)),
                ("scale", ctypes.c_float), ("dtype", ctypes.c_int32), ("beta_logits", ctypes.c_int32)]


_lib = None


def load():
    """Load libkda.so (built by ``chunked_gated_delta_09_amd.build``)."""
    global _lib
    if _lib is None:
        # torch first: its bundled HIP runtime (soname libamdhip64.so.7) is then the one
        # libkda.so binds to, so torch's streams and allocations are valid in the library.
        import torch  # noqa: F401
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m chunked_gated_delta_09_amd.build`")
        lib = ctypes.CDLL(LIB_PATH)
        vp, sz = ctypes.c_void_p, ctypes.c_size_t
        dp = ctypes.POINTER(Dims)
        lib.kda_num_chunks.restype = ctypes.c_int64
        lib.kda_num_chunks.argtypes = [dp]
        lib.kda_fwd_workspace_bytes.restype = sz
        lib.kda_fwd_workspace_bytes.argtypes = [dp]
        lib.kda_bwd_workspace_bytes.restype = sz
        lib.kda_bwd_workspace_bytes.argtypes = [dp]
        lib.kda_last_error.restype = ctypes.c_char_p
        lib.kda_last_error.argtypes = []
        lib.kda_fwd_states.restype = ctypes.c_int
        lib.kda_fwd_states.argtypes = [dp] + [vp] * 10 + [vp, sz, vp]
        lib.kda_chunk_bwd.restype = ctypes.c_int
        lib.kda_chunk_bwd.argtypes = [dp] + [vp] * 15 + [vp, sz, vp]
        lib.kda_chunk_bwd_noalloc.restype = ctypes.c_int
        lib.kda_chunk_bwd_noalloc.argtypes = [dp] + [vp] * 15 + [vp]
        lib.kda_saved_bytes.restype = sz
        lib.kda_saved_bytes.argtypes = [dp]
        lib.kda_fwd_states_save.restype = ctypes.c_int
        lib.kda_fwd_states_save.argtypes = [dp] + [vp] * 10 + [vp, sz] + [vp, sz, vp]
        lib.kda_chunk_bwd_saved.restype = ctypes.c_int
        lib.kda_chunk_bwd_saved.argtypes = [dp] + [vp] * 8 + [sz] + [vp] * 8 + [vp, sz, vp]
        _lib = lib
    return _lib


def _check(status):
    if status != 0:
        raise KdaError(status, load().kda_last_error().decode())


def make_dims(B, T, H, HV, K, V, C, scale=None, dtype="bf16", cu_seqlens=None, cu_seqlens_dev=None,
              beta_logits=False):
    """Build a kda_dims. ``cu_seqlens`` (host list/tensor) selects packed sequences; the
    matching device copy must be passed as ``cu_seqlens_dev`` (int32 tensor on the GPU).
    ``beta_logits``: beta holds logits (sigmoid applied in the kernels, dbeta w.r.t. the
    logits). Returns (dims, keepalive)."""
    dt = KDA_F32 if dtype in ("f32", "fp32", "float32") else KDA_BF16
    if scale is None:
        scale = 1.0 / math.sqrt(K)
    if cu_seqlens is not None:
        cu = [int(x) for x in (cu_seqlens.tolist() if hasattr(cu_seqlens, "tolist") else cu_seqlens)]
        host = (ctypes.c_int32 * len(cu))(*cu)
        N = len(cu) - 1
        dev = ctypes.c_void_p(cu_seqlens_dev.data_ptr()) if cu_seqlens_dev is not None else None
        d = Dims(B, T, H, HV, K, V, C, N, dev, ctypes.cast(host, ctypes.POINTER(ctypes.c_int32)), scale, dt,
                 int(bool(beta_logits)))
        return d, (host, cu_seqlens_dev)
    d = Dims(B, T, H, HV, K, V, C, B, None, None, scale, dt, int(bool(beta_logits)))
    return d, None


def num_chunks(dims):
    return int(load().kda_num_chunks(ctypes.byref(dims)))


def fwd_workspace_bytes(dims):
    return int(load().kda_fwd_workspace_bytes(ctypes.byref(dims)))


def bwd_workspace_bytes(dims):
    return int(load().kda_bwd_workspace_bytes(ctypes.byref(dims)))


def saved_bytes(dims):
    """Bytes of the forward's save for the saved-operand backward (kda_saved_bytes)."""
    return int(load().kda_saved_bytes(ctypes.byref(dims)))


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _check_tensor(t, name, dtype, shape):
    import torch
    if t is None:
        return
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    del torch


def _geometry(q_or_k, v, C, cu_seqlens, scale, beta_logits=False):
    import torch
    B, T, H, K = q_or_k.shape
    HV, V = v.shape[2], v.shape[3]
    dtype = "f32" if q_or_k.dtype == torch.float32 else "bf16"
    cu_dev = None
    if cu_seqlens is not None:
        if B != 1:
            raise ValueError("packed sequences need batch size 1")
        cu_dev = torch.tensor([int(x) for x in cu_seqlens], dtype=torch.int32, device=q_or_k.device)
    dims, keep = make_dims(B, T, H, HV, K, V, C, scale, dtype, cu_seqlens, cu_dev, beta_logits)
    return dims, keep, (B, T, H, HV, K, V, dims.N)


def fwd_states(q, k, v, g, beta, h0=None, cu_seqlens=None, C=64, scale=None, output_o=False,
               output_final_state=True, beta_logits=False, save=False):
    """Forward chunk states. Returns dict(states [NT,HV,K,V], inv [NT,HV,C,C],
    final_state [N,HV,K,V] fp32 or None, o [B,T,HV,V] or None, saved uint8 or None).
    ``beta_logits``: beta holds logits (the kernels apply a sigmoid). ``save``: also keep the
    backward's chunk operands (kda_fwd_states_save; implies output_o) for
    ``chunk_bwd(..., saved=...)``."""
    import torch
    dims, keep, (B, T, H, HV, K, V, N) = _geometry(k, v, C, cu_seqlens, scale, beta_logits)
    tdt = k.dtype
    for t, nm, sh in [(q, "q", (B, T, H, K)), (k, "k", (B, T, H, K)), (v, "v", (B, T, HV, V))]:
        _check_tensor(t, nm, tdt, sh)
    _check_tensor(g, "g", torch.float32, (B, T, HV, K))
    _check_tensor(beta, "beta", torch.float32, (B, T, HV))
    _check_tensor(h0, "h0", tdt, (N, HV, K, V))
    NT = num_chunks(dims)
    if NT < 0:
        raise KdaError(-1, load().kda_last_error().decode())
    dev = k.device
    states = torch.empty(NT, HV, K, V, dtype=tdt, device=dev)
    inv = torch.empty(NT, HV, C, C, dtype=tdt, device=dev)
    final = torch.empty(N, HV, K, V, dtype=torch.float32, device=dev) if output_final_state else None
    o = torch.empty(B, T, HV, V, dtype=tdt, device=dev) if (output_o or save) else None
    wsb = fwd_workspace_bytes(dims)
    ws = torch.empty(max(wsb, 1), dtype=torch.uint8, device=dev)
    saved = None
    if save:
        svb = saved_bytes(dims)
        saved = torch.empty(max(svb, 1), dtype=torch.uint8, device=dev)
        _check(load().kda_fwd_states_save(ctypes.byref(dims), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                                          _ptr(h0), _ptr(states), _ptr(inv), _ptr(final), _ptr(o), _ptr(saved), svb,
                                          _ptr(ws), wsb, _stream()))
    else:
        _check(load().kda_fwd_states(ctypes.byref(dims), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(h0),
                                     _ptr(states), _ptr(inv), _ptr(final), _ptr(o), _ptr(ws), wsb, _stream()))
    del keep
    return dict(states=states, inv=inv, final_state=final, o=o, saved=saved)


def chunk_bwd_into(dims, q, k, v, g, beta, states, inv, dO, dS_final, dq, dk, dv, dg, dbeta, dh0, workspace,
                   stream=None, saved=None):
    """Raw call with caller-owned outputs and workspace (no allocation, no checks beyond
    the library's own). ``saved``: the forward's save (kda_chunk_bwd_saved)."""
    st = _stream() if stream is None else ctypes.c_void_p(stream)
    if saved is not None:
        _check(load().kda_chunk_bwd_saved(ctypes.byref(dims), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                                          _ptr(states), _ptr(inv), _ptr(saved), saved.numel(), _ptr(dO),
                                          _ptr(dS_final), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dg), _ptr(dbeta),
                                          _ptr(dh0), _ptr(workspace), workspace.numel(), st))
        return
    _check(load().kda_chunk_bwd(ctypes.byref(dims), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(states),
                                _ptr(inv), _ptr(dO), _ptr(dS_final), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dg),
                                _ptr(dbeta), _ptr(dh0), _ptr(workspace), workspace.numel(), st))


def chunk_bwd_noalloc_into(dims, q, k, v, g, beta, states, inv, dO, dS_final, dq, dk, dv, dg, dbeta, dh0,
                           stream=None):
    """kda_chunk_bwd_noalloc: as chunk_bwd_into with the library's own static workspace (at
    most KDA_NOALLOC_MAX_WORKSPACE bytes; calls on one GPU must not overlap)."""
    st = _stream() if stream is None else ctypes.c_void_p(stream)
    _check(load().kda_chunk_bwd_noalloc(ctypes.byref(dims), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                                        _ptr(states), _ptr(inv), _ptr(dO), _ptr(dS_final), _ptr(dq), _ptr(dk),
                                        _ptr(dv), _ptr(dg), _ptr(dbeta), _ptr(dh0), st))


def chunk_bwd(q, k, v, g, beta, states, inv, dO, dS_final=None, cu_seqlens=None, C=64, scale=None,
              output_dh0=True, beta_logits=False, saved=None):
    """Chunkwise backward. Returns dict(dq, dk [B,T,H,K], dv [B,T,HV,V], dg [B,T,HV,K] fp32,
    dbeta [B,T,HV] fp32, dh0 [N,HV,K,V] fp32 or None). ``beta_logits``: beta holds logits
    and dbeta is the gradient w.r.t. them. ``saved``: the ``saved`` tensor of
    ``fwd_states(..., save=True)`` on the same inputs (kda_chunk_bwd_saved)."""
    import torch
    dims, keep, (B, T, H, HV, K, V, N) = _geometry(q, v, C, cu_seqlens, scale, beta_logits)
    tdt = q.dtype
    NT = num_chunks(dims)
    if NT < 0:
        raise KdaError(-1, load().kda_last_error().decode())
    for t, nm, sh in [(q, "q", (B, T, H, K)), (k, "k", (B, T, H, K)), (v, "v", (B, T, HV, V)),
                      (dO, "dO", (B, T, HV, V)), (states, "states", (NT, HV, K, V)), (inv, "inv", (NT, HV, C, C)),
                      (dS_final, "dS_final", (N, HV, K, V))]:
        _check_tensor(t, nm, tdt, sh)
    _check_tensor(g, "g", torch.float32, (B, T, HV, K))
    _check_tensor(beta, "beta", torch.float32, (B, T, HV))
    dev = q.device
    dq = torch.empty_like(q)
    dk = torch.empty_like(k)
    dv = torch.empty_like(v)
    dg = torch.empty(B, T, HV, K, dtype=torch.float32, device=dev)
    dbeta = torch.empty(B, T, HV, dtype=torch.float32, device=dev)
    dh0 = torch.empty(N, HV, K, V, dtype=torch.float32, device=dev) if output_dh0 else None
    wsb = bwd_workspace_bytes(dims)
    ws = torch.empty(max(wsb, 1), dtype=torch.uint8, device=dev)
    if saved is not None:
        _check_tensor(saved, "saved", torch.uint8, (max(saved_bytes(dims), 1),))
    chunk_bwd_into(dims, q, k, v, g, beta, states, inv, dO, dS_final, dq, dk, dv, dg, dbeta, dh0, ws, saved=saved)
    del keep
    return dict(dq=dq, dk=dk, dv=dv, dg=dg, dbeta=dbeta, dh0=dh0)
