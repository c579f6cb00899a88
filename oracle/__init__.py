"""KDA oracle: plain fp64 CPU definitions of what the KDA chunk backward computes.

TEST INFRASTRUCTURE ONLY. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call anything in this package. The
GPU library never links, loads or calls it, and it shares no code with the GPU library.

Two independent functions live here:

* ``run`` -- the token-by-token fp64 recurrence with its hand-derived backward
  (``kda_oracle.c``). This is the definition the GPU results are compared against.
* ``chunked.chunked_fwd_bwd`` -- the fp64 chunkwise form of the same map (chunk
  equations of the FlashKDA backward page, steps 1-3, and of the FLA ``chunk_kda_bwd``
  page). It exists to pin the chunk algebra against the recurrence and to expose
  per-chunk intermediates (states, state gradients, the WY/UT inverse).

Layouts (fp64, row-major, batch folded into the token axis of packed sequences):
q, k [T, H, K]; v, dO [T, HV, V]; g [T, HV, K]; beta [T, HV]; h0, dS_final [N, HV, K, V].
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "kda_oracle.c")
_LIB = os.path.join(_HERE, "libkda_oracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile the C oracle with gcc (plain C, -O2, pthreads)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-std=c99", "-D_POSIX_C_SOURCE=200809L", "-shared", "-fPIC",
                               "-pthread", _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        build(force=False)
        lib = ctypes.CDLL(_LIB)
        dp = ctypes.POINTER(ctypes.c_double)
        lib.kda_oracle_run.restype = ctypes.c_int
        lib.kda_oracle_run.argtypes = [ctypes.c_int, ctypes.POINTER(ctypes.c_int64), ctypes.c_int, ctypes.c_int,
                                       ctypes.c_int, ctypes.c_int, ctypes.c_double] + [dp] * 16 + [ctypes.c_int]
        _lib = lib
    return _lib


def _ptr(a):
    if a is None:
        return ctypes.POINTER(ctypes.c_double)()
    assert a.dtype == np.float64 and a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def _f64(a):
    if a is None:
        return None
    if hasattr(a, "detach"):  # torch tensor
        a = a.detach().to("cpu").double().numpy()
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def run(q, k, v, g, beta, cu_seqlens, scale, h0=None, dO=None, dS_final=None, backward=True, nthreads=0,
        beta_logits=False):
    """Forward (o, S_T) and, if ``backward``, the VJP (dq, dk, dv, dg, dbeta, dh0) of
    L = sum_t <dO_t, o_t> + <dS_final, S_T>. Returns a dict of fp64 numpy arrays and the
    number of threads used under key ``threads``.

    ``beta_logits``: ``beta`` holds logits x and the write strength is sigmoid(x) (the
    FlashKDA backward page applies a sigmoid to the raw beta it loads); dbeta is then the
    gradient w.r.t. x, the strength's gradient times sigmoid(x)(1 - sigmoid(x))."""
    q, k, v, g, beta = map(_f64, (q, k, v, g, beta))
    logit = None
    if beta_logits:
        logit = beta
        beta = 1.0 / (1.0 + np.exp(-logit))
    h0, dO, dS_final = _f64(h0), _f64(dO), _f64(dS_final)
    T, H, K = q.shape
    HV, V = v.shape[1], v.shape[2]
    cu = np.ascontiguousarray(np.asarray(cu_seqlens, dtype=np.int64))
    N = cu.shape[0] - 1
    assert k.shape == (T, H, K) and v.shape == (T, HV, V) and g.shape == (T, HV, K) and beta.shape == (T, HV)
    assert cu[0] == 0 and cu[-1] == T
    out = {"o": np.zeros((T, HV, V)), "S_T": np.zeros((N, HV, K, V))}
    if backward:
        assert dO is not None and dO.shape == (T, HV, V)
        out.update(dq=np.zeros((T, H, K)), dk=np.zeros((T, H, K)), dv=np.zeros((T, HV, V)),
                   dg=np.zeros((T, HV, K)), dbeta=np.zeros((T, HV)), dh0=np.zeros((N, HV, K, V)))
    lib = _load()
    nt = lib.kda_oracle_run(N, cu.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)), H, HV, K, V, float(scale),
                            _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(h0), _ptr(dO), _ptr(dS_final),
                            _ptr(out["o"]), _ptr(out["S_T"]),
                            _ptr(out.get("dq")), _ptr(out.get("dk")), _ptr(out.get("dv")), _ptr(out.get("dg")),
                            _ptr(out.get("dbeta")), _ptr(out.get("dh0")), int(nthreads))
    if nt < 0:
        raise ValueError("kda_oracle_run rejected its arguments")
    if backward and beta_logits:
        out["dbeta"] = out["dbeta"] * beta * (1.0 - beta)
    out["threads"] = nt
    return out


def loss(out, dO, dS_final=None):
    """L = sum <dO, o> + <dS_final, S_T> for a forward result ``out``."""
    val = float(np.sum(_f64(dO) * out["o"]))
    if dS_final is not None:
        val += float(np.sum(_f64(dS_final) * out["S_T"]))
    return val
