"""Training entry point: the chunked KDA forward (output o and final state) with its backward
wired into torch autograd.

Forward: `kda_fwd_states` (per-chunk states S_in, WY/UT inverses, o, S_T). Backward:
`kda_chunk_bwd` on the saved states and inverses with dO and the gradient of S_T. With
``save_operands`` (the default) the pair is `kda_fwd_states_save` / `kda_chunk_bwd_saved`: the
forward also keeps the backward's chunk operands (kr, -w^T, Q'^T, e^gam), so the backward
skips their recomputation (FLA chunk_bwd page: the disable_recompute switch). Both run
entirely in the HIP library; this module only marshals tensors (FLA chunk_bwd page:
`chunk_kda_bwd` takes the forward's saved inverses and states and returns dq, dk, dv,
dbeta, dg, dh0; FlashKDA backward page: the chunk kernel's inputs are the forward
workspace and dO).
"""
from __future__ import annotations

import torch

from . import chunk_bwd, fwd_states


class KdaChunkFunction(torch.autograd.Function):
    """o, S_T = KDA(q, k, v, g, beta, h0) with gradients for q, k, v, g, beta and h0.

    g is the per-channel log decay (fp32, natural log), beta the write strength (fp32). The
    gradient of S_T reaches the backward in the input precision (bf16 for bf16 inputs), the
    precision in which the library takes dS_final."""

    @staticmethod
    def forward(ctx, q, k, v, g, beta, h0, cu_seqlens, C, scale, output_final_state, beta_logits, save_operands):
        fw = fwd_states(q, k, v, g, beta, h0=h0, cu_seqlens=cu_seqlens, C=C, scale=scale, output_o=True,
                        output_final_state=output_final_state, beta_logits=beta_logits, save=save_operands)
        ctx.save_for_backward(q, k, v, g, beta, fw["states"], fw["inv"], fw["saved"])
        ctx.cu_seqlens, ctx.C, ctx.scale, ctx.beta_logits = cu_seqlens, C, scale, beta_logits
        ctx.h0_dtype = None if h0 is None else h0.dtype
        return fw["o"], fw["final_state"]

    @staticmethod
    def backward(ctx, do, dfinal):
        q, k, v, g, beta, states, inv, saved = ctx.saved_tensors
        dS = None if dfinal is None else dfinal.to(q.dtype).contiguous()
        r = chunk_bwd(q, k, v, g, beta, states, inv, do.to(q.dtype).contiguous(), dS_final=dS,
                      cu_seqlens=ctx.cu_seqlens, C=ctx.C, scale=ctx.scale, output_dh0=ctx.h0_dtype is not None,
                      beta_logits=ctx.beta_logits, saved=saved)
        dh0 = None if ctx.h0_dtype is None else r["dh0"].to(ctx.h0_dtype)
        return r["dq"], r["dk"], r["dv"], r["dg"], r["dbeta"], dh0, None, None, None, None, None, None


def kda_chunk(q, k, v, g, beta, h0=None, cu_seqlens=None, C=64, scale=None, output_final_state=True,
              beta_logits=False, save_operands=True):
    """Differentiable chunked KDA. Shapes: q, k [B,T,H,K]; v [B,T,HV,V]; g [B,T,HV,K] fp32;
    beta [B,T,HV] fp32 (write strengths, or their logits with ``beta_logits``); h0
    [N,HV,K,V] or None; packed sequences via cu_seqlens (host list, B = 1).
    ``save_operands``: keep the backward's chunk operands from the forward (saved-operand
    mode) rather than recomputing them in the backward. Returns (o [B,T,HV,V], S_T
    [N,HV,K,V] fp32 or None)."""
    return KdaChunkFunction.apply(q, k, v, g, beta, h0, cu_seqlens, C, scale, output_final_state, beta_logits,
                                  save_operands)
