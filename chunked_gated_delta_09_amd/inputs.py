"""Seeded synthetic inputs for the KDA chunk backward.

This module only draws random tensors; it holds none of the method's arithmetic. Both the
GPU tests / benchmark and the oracle-side tests take their inputs from here.

Distributions (the five workloads of the KDA chunk-backward study):
  q, k ~ N(0, 1), then L2-normalised per (token, head) over K (input preparation)
  v, dO ~ N(0, 1)
  g = logsigmoid(N(3, 1)) per (token, v-head, channel), kept in fp32
  beta = sigmoid(N(0, 1)) per (token, v-head), kept in fp32
  h0, dS_final ~ N(0, 0.1) (standard deviation 0.1) where the workload has them
All values are drawn in fp32 from one ``torch.Generator('cpu')`` seeded with
``1000 + workload id`` (or an explicit seed), in the fixed order
[varlen lengths], q, k, v, g-logits, beta-logits, h0, dS_final, dO,
and then rounded to the workload dtype (g and beta stay fp32).
"""
from __future__ import annotations

import dataclasses
import math

import torch


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    H: int
    HV: int
    K: int
    V: int
    C: int
    dtype: str            # "f32" or "bf16"
    B: int = 1            # dense batch (ignored when varlen > 0)
    T: int = 0            # dense sequence length
    varlen: int = 0       # number of packed sequences (0 = dense)
    total: int = 0        # total tokens when varlen > 0
    len_lo: int = 256
    len_hi: int = 4096
    has_h0: bool = False
    has_dsf: bool = False

    @property
    def torch_dtype(self):
        return torch.float32 if self.dtype == "f32" else torch.bfloat16


WORKLOADS = {
    0: Workload("tiny_fp32_t64_k16_c16", H=1, HV=1, K=16, V=16, C=16, dtype="f32", B=1, T=64),
    1: Workload("bf16_b2_t2048_h8_k128_c64", H=8, HV=8, K=128, V=128, C=64, dtype="bf16", B=2, T=2048,
                has_h0=True, has_dsf=True),
    2: Workload("bf16_b1_t16384_h16_k128_c64", H=16, HV=16, K=128, V=128, C=64, dtype="bf16", B=1, T=16384,
                has_dsf=True),
    3: Workload("bf16_varlen16_t32768_h16_k128_c64", H=16, HV=16, K=128, V=128, C=64, dtype="bf16",
                varlen=16, total=32768, has_h0=True, has_dsf=True),
    4: Workload("bf16_gva_b4_t4096_h8_hv32_k128_c64", H=8, HV=32, K=128, V=128, C=64, dtype="bf16", B=4, T=4096,
                has_h0=True, has_dsf=True),
}


def varlen_lengths(gen: torch.Generator, n: int, total: int, lo: int, hi: int):
    """n lengths: the first n-1 ~ UniformInt[lo, hi], the last = total - sum, all n-1
    redrawn until the last also lies in [lo, hi]."""
    while True:
        first = torch.randint(lo, hi + 1, (n - 1,), generator=gen).tolist()
        last = total - sum(first)
        if lo <= last <= hi:
            return first + [last]


def make_inputs(w: Workload, seed: int | None = None, wid: int | None = None):
    """Draw one workload's tensors on the CPU. Returns a dict with
    q, k [B, T, H, K]; v, dO [B, T, HV, V]; g [B, T, HV, K] fp32; beta [B, T, HV] fp32;
    h0, dS_final [N, HV, K, V] or None; cu_seqlens (list of N+1 ints, or None when dense);
    scale; and the workload."""
    if seed is None:
        seed = 1000 + (wid if wid is not None else 0)
    gen = torch.Generator("cpu").manual_seed(seed)
    if w.varlen:
        lens = varlen_lengths(gen, w.varlen, w.total, w.len_lo, w.len_hi)
        cu = [0]
        for ln in lens:
            cu.append(cu[-1] + ln)
        B, T, N = 1, w.total, w.varlen
    else:
        cu = None
        B, T, N = w.B, w.T, w.B
    dt = w.torch_dtype

    def normal(*shape, std=1.0, mean=0.0):
        return torch.randn(*shape, generator=gen, dtype=torch.float32) * std + mean

    q = normal(B, T, w.H, w.K)
    k = normal(B, T, w.H, w.K)
    q = q / q.norm(dim=-1, keepdim=True)
    k = k / k.norm(dim=-1, keepdim=True)
    v = normal(B, T, w.HV, w.V)
    g = torch.nn.functional.logsigmoid(normal(B, T, w.HV, w.K, mean=3.0))
    beta = torch.sigmoid(normal(B, T, w.HV))
    h0 = normal(N, w.HV, w.K, w.V, std=0.1) if w.has_h0 else None
    dsf = normal(N, w.HV, w.K, w.V, std=0.1) if w.has_dsf else None
    dO = normal(B, T, w.HV, w.V)
    rnd = (lambda x: None if x is None else x.to(dt))
    return dict(q=rnd(q), k=rnd(k), v=rnd(v), g=g.contiguous(), beta=beta.contiguous(), h0=rnd(h0),
                dS_final=rnd(dsf), dO=rnd(dO), cu_seqlens=cu, scale=1.0 / math.sqrt(w.K), workload=w,
                B=B, T=T, N=N)


def flat_cu(inp):
    """cu_seqlens covering every sequence, dense batches included (for the oracle)."""
    if inp["cu_seqlens"] is not None:
        return list(inp["cu_seqlens"])
    return [b * inp["T"] for b in range(inp["B"] + 1)]


def token_heads(inp):
    """Work units of the metric: tokens x v-heads."""
    return inp["B"] * inp["T"] * inp["workload"].HV
