"""Shared helpers of the GPU tests: run the HIP library on a workload and the fp64 oracle
on the same (optionally head-sampled) inputs, and compare with relative L2 errors."""
from __future__ import annotations

import dataclasses

import numpy as np
import torch

from chunked_gated_delta_09_amd import inputs as kin

# Tolerances (max relative L2 error per tensor) for the two precisions.
TOL = {"f32": 1e-4, "bf16": 2e-2}
GRADS = ["dq", "dk", "dv", "dg", "dbeta", "dh0"]


def rel_l2(x, ref):
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = np.linalg.norm(ref)
    num = np.linalg.norm(x - ref)
    return float(num / den) if den > 0 else float(num)


def small_workload(name, **kw):
    base = dict(H=1, HV=1, K=128, V=128, C=64, dtype="bf16")
    base.update(kw)
    return kin.Workload(name, **base)


def to_dev(t):
    return None if t is None else t.contiguous().cuda()


def run_gpu(inp, C=None, output_o=True, beta_logits=False, saved=False):
    """kda_fwd_states + kda_chunk_bwd on the GPU; ``saved``: the saved-operand pair
    kda_fwd_states_save + kda_chunk_bwd_saved instead."""
    import chunked_gated_delta_09_amd as kda
    w = inp["workload"]
    C = w.C if C is None else C
    q, k, v, g, beta, h0, dsf, dO = (to_dev(inp[n]) for n in ("q", "k", "v", "g", "beta", "h0", "dS_final", "dO"))
    f = kda.fwd_states(q, k, v, g, beta, h0=h0, cu_seqlens=inp["cu_seqlens"], C=C, scale=inp["scale"],
                       output_o=output_o, beta_logits=beta_logits, save=saved)
    b = kda.chunk_bwd(q, k, v, g, beta, f["states"], f["inv"], dO, dS_final=dsf, cu_seqlens=inp["cu_seqlens"], C=C,
                      scale=inp["scale"], beta_logits=beta_logits, saved=f["saved"])
    torch.cuda.synchronize()
    out = {key: (val.float().cpu().numpy() if val is not None else None) for key, val in {**f, **b}.items()
           if key != "saved"}
    return out


def _np(t):
    return None if t is None else t.float().numpy().astype(np.float64)


def head_slices(inp, qk_heads=None):
    """Index arrays of the q/k heads and value heads to compare (None = all)."""
    w = inp["workload"]
    G = w.HV // w.H
    if qk_heads is None:
        qk_heads = list(range(w.H))
    v_heads = [hq * G + e for hq in qk_heads for e in range(G)]
    return list(qk_heads), v_heads


def run_oracle(oracle_mod, inp, qk_heads=None, beta_logits=False, nthreads=0):
    """fp64 oracle on the given q/k heads (and their value heads), all sequences."""
    w = inp["workload"]
    qh, vh = head_slices(inp, qk_heads)
    B, T = inp["B"], inp["T"]
    flat = lambda t, heads: None if t is None else _np(t).reshape(B * T, *t.shape[2:])[:, heads]
    q, k = flat(inp["q"], qh), flat(inp["k"], qh)
    v, g, dO = flat(inp["v"], vh), flat(inp["g"], vh), flat(inp["dO"], vh)
    beta = _np(inp["beta"]).reshape(B * T, w.HV)[:, vh]
    h0 = None if inp["h0"] is None else _np(inp["h0"])[:, vh]
    dsf = None if inp["dS_final"] is None else _np(inp["dS_final"])[:, vh]
    cont = lambda a: None if a is None else np.ascontiguousarray(a)
    return oracle_mod.run(cont(q), cont(k), cont(v), cont(g), cont(beta), kin.flat_cu(inp), inp["scale"],
                          h0=cont(h0), dO=cont(dO), dS_final=cont(dsf), beta_logits=beta_logits,
                          nthreads=nthreads)


def gpu_on_heads(inp, out, qk_heads=None):
    """The GPU outputs restricted to the sampled heads, in the oracle's flat layout."""
    qh, vh = head_slices(inp, qk_heads)
    B, T = inp["B"], inp["T"]
    res = {}
    for key in ("dq", "dk"):
        res[key] = out[key].reshape(B * T, -1, out[key].shape[-1])[:, qh]
    for key in ("dv", "dg", "o"):
        if out.get(key) is not None:
            res[key] = out[key].reshape(B * T, -1, out[key].shape[-1])[:, vh]
    res["dbeta"] = out["dbeta"].reshape(B * T, -1)[:, vh]
    for key in ("dh0", "final_state"):
        if out.get(key) is not None:
            res[key] = out[key][:, vh]
    return res


# Floor of a chunk's reference norm in the per-chunk error, as a fraction of a full chunk's
# share of the whole tensor's norm (sqrt(C / rows of the tensor) of it): a chunk whose
# gradient is genuinely tiny, or a partial chunk of a token or two (whose "tensor" is a
# handful of values, where bf16 rounding alone reaches ~2e-2), is then judged against the
# scale of a chunk of this tensor instead of its own, while a wrong row (about 1/8 of a
# 64-row chunk's norm) or a wrong partial tail still counts against the chunk it sits in.
CHUNK_FLOOR = 0.25
TOKEN_KEYS = ("dq", "dk", "dv", "dg", "dbeta", "o")


def chunk_errors(x, ref, cu, C):
    """Per-(chunk, head) relative L2 errors of a token-major tensor [T, heads, ...] (fp64),
    chunks of C tokens within each sequence of cu, with the chunk reference norm floored as
    described at CHUNK_FLOOR. Returns an array [chunks, heads]."""
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    T = ref.shape[0]
    heads = ref.shape[1]
    x = x.reshape(T, heads, -1)
    ref = ref.reshape(T, heads, -1)
    full = np.sqrt(np.sum(ref ** 2, axis=(0, 2)))  # per head
    out = []
    for a, b in zip(cu[:-1], cu[1:]):
        for s in range(a, b, C):
            e = min(s + C, b)
            num = np.sqrt(np.sum((x[s:e] - ref[s:e]) ** 2, axis=(0, 2)))
            den = np.sqrt(np.sum(ref[s:e] ** 2, axis=(0, 2)))
            floor = CHUNK_FLOOR * full * np.sqrt(min(C, T) / max(T, 1))
            den = np.maximum(den, floor)
            out.append(np.where(den > 0, num / np.where(den > 0, den, 1.0), num))
    return np.array(out).reshape(-1, heads)


def compare(inp, out, ref, qk_heads=None, keys=None, tol=None, per_chunk=True):
    """Relative L2 error of each compared tensor, and (per_chunk) the largest per-(chunk,
    head) relative L2 error of each token-major tensor under the key '<name>@chunk'.
    Returns (errors, failures): every error is held to the same tolerance."""
    w = inp["workload"]
    tol = TOL[w.dtype] if tol is None else tol
    got = gpu_on_heads(inp, out, qk_heads)
    pairs = {"dq": "dq", "dk": "dk", "dv": "dv", "dg": "dg", "dbeta": "dbeta", "dh0": "dh0", "o": "o",
             "final_state": "S_T"}
    errs = {}
    cu = kin.flat_cu(inp)
    for key, rkey in pairs.items():
        if keys is not None and key not in keys:
            continue
        if key not in got or got[key] is None:
            continue
        errs[key] = rel_l2(got[key], ref[rkey])
        if per_chunk and key in TOKEN_KEYS and np.asarray(ref[rkey]).shape[0] > 0:
            ce = chunk_errors(got[key], ref[rkey], cu, w.C)
            if ce.size:
                errs[key + "@chunk"] = float(ce.max())
    bad = {k: v for k, v in errs.items() if not v <= tol}
    return errs, bad
