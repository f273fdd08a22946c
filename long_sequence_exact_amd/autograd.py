"""Attention as torch.autograd functions whose forward and backward are the
library's kernels (the backward recomputes P from the saved O and LSE).

    segment_attention(q, k, v, causal_offset=None, scale=None) -> o
    dilated_attention(q, k, v, segment_lengths, dilations, causal=False,
                      scale=None, head_shift=False) -> o (fp32)

Inputs are bf16 on the GPU (the backward takes bf16 q, k, v).  o of
segment_attention has q's dtype; o of dilated_attention is the fp32 merge
accumulator.  Gradients come back in fp32; autograd casts them to the
inputs' dtype.
"""
from __future__ import annotations

import torch

from . import attn_segment_bwd, attn_segment_fwd, dilated_attn_bwd, dilated_attn_fwd

__all__ = ["segment_attention", "dilated_attention"]


def _grad_in(d_o):
    """The upstream gradient as the kernels take it: bf16 and contiguous (so
    its rows are 16-byte aligned)."""
    if d_o.dtype != torch.bfloat16:
        d_o = d_o.to(torch.bfloat16)
    return d_o.contiguous()


class _SegmentAttention(torch.autograd.Function):
    @staticmethod
    def forward(ctx, q, k, v, causal_offset, scale):
        o, lse = attn_segment_fwd(q, k, v, causal_offset=causal_offset, scale=scale)
        ctx.save_for_backward(q, k, v, o, lse)
        ctx.causal_offset, ctx.scale = causal_offset, scale
        return o

    @staticmethod
    def backward(ctx, d_o):
        q, k, v, o, lse = ctx.saved_tensors
        dq, dk, dv = attn_segment_bwd(q, k, v, o, lse, _grad_in(d_o),
                                      causal_offset=ctx.causal_offset, scale=ctx.scale)
        return dq, dk, dv, None, None


class _DilatedAttention(torch.autograd.Function):
    @staticmethod
    def forward(ctx, q, k, v, segment_lengths, dilations, causal, scale, head_shift):
        o, lse = dilated_attn_fwd(q, k, v, segment_lengths, dilations, causal=causal,
                                  scale=scale, head_shift=head_shift)
        ctx.save_for_backward(q, k, v, o, lse)
        ctx.args = (tuple(segment_lengths), tuple(dilations), causal, scale, head_shift)
        return o

    @staticmethod
    def backward(ctx, d_o):
        q, k, v, o, lse = ctx.saved_tensors
        ws, rs, causal, scale, head_shift = ctx.args
        dq, dk, dv = dilated_attn_bwd(q, k, v, o, lse, _grad_in(d_o), ws, rs,
                                      causal=causal, scale=scale, head_shift=head_shift)
        return dq, dk, dv, None, None, None, None, None


def segment_attention(q, k, v, causal_offset=None, scale=None):
    """attn_segment_fwd's O with a backward through attn_segment_bwd.
    causal_offset: None (non-causal) or delta (key j visible to query i iff
    j <= i + delta)."""
    return _SegmentAttention.apply(q, k, v, causal_offset, scale)


def dilated_attention(q, k, v, segment_lengths, dilations, causal=False, scale=None,
                      head_shift=False):
    """dilated_attn_fwd's merged O (fp32) with a backward through
    dilated_attn_bwd."""
    return _DilatedAttention.apply(q, k, v, segment_lengths, dilations, causal, scale,
                                   head_shift)
