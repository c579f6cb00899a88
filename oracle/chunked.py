"""fp64 chunkwise form of KDA forward and backward (TEST INFRASTRUCTURE ONLY).

Follows the chunk algebra of the FlashKDA backward page (step 1: recompute U; step 2:
the gradient products; step 3: the adjoint of the triangular solve; the chunk forward it
differentiates, written below as O, S_out and Lm in this module's notation) and of the FLA
chunk_kda_bwd page (kernel chunk_kda_bwd_kernel_wy_dqkg_fused: the inter terms and the dg
formula; driver chunk_kda_bwd: GVA reduction and the reverse chunk-local cumsum of dg).
Notation, per sequence n, v-head h and chunk c with L valid rows:

  G = chunk-local inclusive cumsum of g; gam = G[L-1]
  qd = scale*q*e^G; kd = k*e^G; ki = k*e^-G; kr = k*e^(gam-G)
  Lm = strict_tril(diag(beta) kd ki^T); INV = (I + Lm)^-1; Mqk = tril(qd ki^T)
  vc0 = v - kd S_in; U = INV diag(beta) vc0
  O = qd S_in + Mqk U;  S_out = diag(e^gam) S_in + kr^T U

Backward, given dO and dS (gradient w.r.t. S_out):
  dU = Mqk^T dO + kr dS;  dvc = INV^T dU;  dv = diag(beta) dvc
  dS_in = diag(e^gam) dS + qd^T dO - kd^T diag(beta) dvc
  dMqk = tril(dO U^T);  dL = -strict_tril(dvc U^T)
  dqd = dO S_in^T + dMqk ki;  dkd = -diag(beta) dvc S_in^T + diag(beta) dL ki
  dki = dMqk^T qd + (diag(beta) dL)^T kd;  dkr = U dS^T
  dbeta = rowsum(dvc o vc0) + rowsum(kd o (dL ki))
  dq = scale e^G o dqd;  dk = e^G o dkd + e^-G o dki + e^(gam-G) o dkr
  dG = qd o dqd + kd o dkd - ki o dki - kr o dkr
  dG[L-1] += e^gam o rowsum(dS o S_in) + sum_j kr_j o dkr_j
  dg = reverse cumsum of dG within the chunk

Plain numpy; no blocking beyond the chunking the method itself defines.

``bf16_operands=True`` is an error model of a bf16 implementation, not a definition: every
operand of a matrix product above, every per-chunk tensor kept between the passes (S_in,
INV, the state gradient of each chunk) and the outputs dq, dk, dv are rounded to bf16
(round to nearest even); products, sums and the elementwise gate algebra stay in fp64 (the
FlashKDA backward page keeps its workspace in bf16 and does its math in fp32). Its
per-tensor error against the fp64 definition predicts the error a bf16 kernel can expect.
``f32_operands=True`` is the same model with fp32 rounding, for the fp32 path.
"""
from __future__ import annotations

import numpy as np


def _f64(a):
    if a is None:
        return None
    if hasattr(a, "detach"):
        a = a.detach().to("cpu").double().numpy()
    return np.asarray(a, dtype=np.float64)


def chunk_table(cu_seqlens, C):
    """Global chunk numbering: sequence 0's chunks first, then sequence 1's, ...
    Returns a list of (n, bos, length) per global chunk."""
    cu = [int(x) for x in cu_seqlens]
    out = []
    for n in range(len(cu) - 1):
        for s in range(cu[n], cu[n + 1], C):
            out.append((n, s, min(C, cu[n + 1] - s)))
    return out


def _bf16(a):
    """Round to the nearest bf16 value (ties to even), returned as fp64."""
    import torch
    return torch.from_numpy(np.asarray(a, dtype=np.float64)).to(torch.bfloat16).to(torch.float64).numpy()


def _f32(a):
    """Round to the nearest fp32 value, returned as fp64."""
    return np.asarray(a, dtype=np.float64).astype(np.float32).astype(np.float64)


def chunked_fwd_bwd(q, k, v, g, beta, cu_seqlens, scale, C, h0=None, dO=None, dS_final=None, backward=True,
                    bf16_operands=False, f32_operands=False):
    """Returns o, S_T and (if backward) dq, dk, dv, dg, dbeta, dh0, plus the per-chunk
    intermediates ``states`` (S_in, [NT, HV, K, V]), ``dstates`` (gradient w.r.t. each
    chunk's S_out, [NT, HV, K, V]) and ``inv`` ([NT, HV, C, C], identity on padded rows).
    ``bf16_operands``, ``f32_operands``: the error models described in the module docstring."""
    r = _bf16 if bf16_operands else (_f32 if f32_operands else (lambda a: a))
    q, k, v, g, beta = map(_f64, (q, k, v, g, beta))
    h0, dO, dS_final = _f64(h0), _f64(dO), _f64(dS_final)
    T, H, K = q.shape
    HV, V = v.shape[1], v.shape[2]
    Gs = HV // H
    cu = [int(x) for x in cu_seqlens]
    N = len(cu) - 1
    table = chunk_table(cu, C)
    NT = len(table)
    first = {}
    for c, (n, s, ln) in enumerate(table):
        first.setdefault(n, c)
    o = np.zeros((T, HV, V))
    S_T = np.zeros((N, HV, K, V))
    states = np.zeros((NT, HV, K, V))
    dstates = np.zeros((NT, HV, K, V))
    inv = np.zeros((NT, HV, C, C))
    res = {}
    if backward:
        dq_h = np.zeros((T, HV, K))
        dk_h = np.zeros((T, HV, K))
        dv = np.zeros((T, HV, V))
        dg = np.zeros((T, HV, K))
        dbeta = np.zeros((T, HV))
        dh0 = np.zeros((N, HV, K, V))
    for n in range(N):
        chunks = [c for c in range(NT) if table[c][0] == n]
        for h in range(HV):
            hq = h // Gs
            S = h0[n, h].copy() if h0 is not None else np.zeros((K, V))
            saved = []
            for c in chunks:
                _, s, L = table[c]
                sl = slice(s, s + L)
                qc, kc, vc = q[sl, hq], k[sl, hq], v[sl, h]
                b = beta[sl, h]
                G = np.cumsum(g[sl, h], axis=0)
                gam = G[L - 1]
                qd = scale * qc * np.exp(G)
                kd = kc * np.exp(G)
                ki = kc * np.exp(-G)
                kr = kc * np.exp(gam[None, :] - G)
                Lm = np.tril(b[:, None] * (r(kd) @ r(ki).T), -1)
                INV = r(np.linalg.inv(np.eye(L) + Lm))
                Mqk = np.tril(r(qd) @ r(ki).T)
                S_in = r(S)
                vc0 = vc - r(kd) @ S_in
                U = INV @ r(b[:, None] * vc0)
                o[sl, h] = r(qd) @ S_in + r(Mqk) @ r(U)
                states[c, h] = S_in
                inv[c, h] = np.eye(C)
                inv[c, h, :L, :L] = INV
                saved.append((c, sl, L, qc, kc, b, G, gam, qd, kd, ki, kr, INV, Mqk, vc0, U, S_in))
                S = np.exp(gam)[:, None] * S + r(kr).T @ r(U)
            S_T[n, h] = S
            if not backward:
                continue
            dS = dS_final[n, h].copy() if dS_final is not None else np.zeros((K, V))
            for (c, sl, L, qc, kc, b, G, gam, qd, kd, ki, kr, INV, Mqk, vc0, U, S_in) in reversed(saved):
                dstates[c, h] = dS
                dOc = dO[sl, h]
                dSr = r(dS)
                dU = r(Mqk).T @ dOc + r(kr) @ dSr
                dvc = INV.T @ r(dU)
                dv[sl, h] = b[:, None] * dvc
                dS_in = np.exp(gam)[:, None] * dS + r(qd).T @ dOc - r(kd).T @ r(b[:, None] * dvc)
                dMqk = np.tril(dOc @ r(U).T)
                dL = -np.tril(r(dvc) @ r(U).T, -1)
                dLki = r(dL) @ r(ki)
                dqd = dOc @ S_in.T + r(dMqk) @ r(ki)
                dkd = -b[:, None] * (r(dvc) @ S_in.T) + b[:, None] * dLki
                dki = r(dMqk).T @ r(qd) + r(b[:, None] * dL).T @ r(kd)
                dkr = r(U) @ dSr.T
                dbeta[sl, h] = np.sum(dvc * vc0, axis=1) + np.sum(kd * dLki, axis=1)
                dq_h[sl, h] = scale * np.exp(G) * dqd
                dk_h[sl, h] = np.exp(G) * dkd + np.exp(-G) * dki + np.exp(gam[None, :] - G) * dkr
                dG = qd * dqd + kd * dkd - ki * dki - kr * dkr
                dG[L - 1] += np.exp(gam) * np.sum(dSr * S_in, axis=1) + np.sum(kr * dkr, axis=0)
                dg[sl, h] = np.cumsum(dG[::-1], axis=0)[::-1]
                dS = dS_in
            dh0[n, h] = dS
    res.update(o=o, S_T=S_T, states=states, inv=inv)
    if backward:
        res.update(dq=r(dq_h.reshape(T, H, Gs, K).sum(axis=2)), dk=r(dk_h.reshape(T, H, Gs, K).sum(axis=2)),
                   dv=r(dv), dg=dg, dbeta=dbeta, dh0=dh0, dstates=dstates)
    return res
