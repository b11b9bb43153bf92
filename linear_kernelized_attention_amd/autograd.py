"""torch.autograd wrapper: FAVOR attention as a differentiable op.

The forward runs favor_attention with the row normalisers (the saved-forward
pair of include/favor.h); the backward hands the saved output and
normalisers to favor_attention_backward, so no part of the forward is
recomputed on the MFMA path.  Omega is a fixed input (no gradient), as in
the method, where the random features are redrawn, not learned.  Argument
marshalling only: every step runs in libfavor.so.
"""
from __future__ import annotations

import torch

from . import _lib


class FavorAttentionFunction(torch.autograd.Function):
    @staticmethod
    def forward(ctx, q, k, v, omega, kind="trig", causal=False, path="auto"):
        q, k, v = (x.contiguous() for x in (q, k, v))
        out, den = _lib.favor_attention(q, k, v, omega, kind=kind, causal=causal, path=path, den=True)
        ctx.save_for_backward(q, k, v, omega, out, den)
        ctx.kind, ctx.causal, ctx.path = kind, causal, path
        return out

    @staticmethod
    def backward(ctx, dout):
        q, k, v, omega, out, den = ctx.saved_tensors
        dq, dk, dv = _lib.favor_attention_backward(q, k, v, omega, dout.contiguous(), kind=ctx.kind,
                                                   causal=ctx.causal, path=ctx.path,
                                                   saved=(out, den))
        return dq, dk, dv, None, None, None, None


def favor_attention_fn(q, k, v, omega, kind: str = "trig", causal: bool = False, path: str = "auto"):
    """Differentiable FAVOR attention of [B, H, L, d] tensors (gradients for
    q, k and v)."""
    return FavorAttentionFunction.apply(q, k, v, omega, kind, causal, path)
