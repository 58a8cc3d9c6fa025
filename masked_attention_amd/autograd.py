"""torch.autograd wrapper of the E2D2 training attentions: the fused forward
(e2d2_attn_train_fwd) and its backward (e2d2_attn_train_bwd) as one differentiable op.

Pages cited, by title and section:
  [Notes] "Encoder-Decoder Diffusion Language Models for Efficient Training and
          Inference", Paper-Notes page: 方法详解 §4 训练算法 (one encoder pass over the
          clean blocks and one decoder pass over the noised blocks per training step;
          the decoder's loss flows back through both attentions).

Argument marshalling only: the forward and the backward are the library's kernels;
this module allocates their outputs, the LSE rows the backward reads and its
workspace, and makes strided upstream gradients contiguous.  bf16 only (the
backward's dtype).
"""
from __future__ import annotations

import torch

from . import (BF16, e2d2_attn_train_bwd, e2d2_attn_train_bwd_workspace_bytes,
               e2d2_attn_train_fwd)


class _E2D2Attention(torch.autograd.Function):
    @staticmethod
    def forward(ctx, q_dec, k_ctx, v_ctx, k_dec, v_dec, q_enc, S, scale):
        ins = [t.contiguous() for t in (q_dec, k_ctx, v_ctx, k_dec, v_dec)]
        q_dec, k_ctx, v_ctx, k_dec, v_dec = ins
        with_enc = q_enc is not None
        if with_enc:
            q_enc = q_enc.contiguous()
        B, Hq, L, _ = q_dec.shape
        o_dec = torch.empty_like(q_dec)
        lse_dec = torch.empty((B, Hq, L), dtype=torch.float32, device=q_dec.device)
        o_enc = torch.empty_like(q_dec) if with_enc else None
        lse_enc = torch.empty_like(lse_dec) if with_enc else None
        e2d2_attn_train_fwd(q_dec, k_ctx, v_ctx, k_dec, v_dec, o_dec, S, lse_dec=lse_dec,
                            q_enc=q_enc, o_enc=o_enc, lse_enc=lse_enc, scale=scale)
        saved = [q_dec, k_ctx, v_ctx, k_dec, v_dec, o_dec, lse_dec]
        if with_enc:
            saved += [q_enc, o_enc, lse_enc]
        ctx.save_for_backward(*saved)
        ctx.with_enc = with_enc
        ctx.S = S
        ctx.scale = scale
        if with_enc:
            return o_dec, o_enc
        return o_dec

    @staticmethod
    def backward(ctx, *grads):
        with_enc = ctx.with_enc
        saved = ctx.saved_tensors
        q_dec, k_ctx, v_ctx, k_dec, v_dec, o_dec, lse_dec = saved[:7]
        q_enc, o_enc, lse_enc = saved[7:] if with_enc else (None, None, None)
        do_dec = grads[0]
        do_dec = torch.zeros_like(o_dec) if do_dec is None else do_dec.contiguous()
        do_enc = None
        if with_enc:
            do_enc = grads[1]
            do_enc = torch.zeros_like(o_enc) if do_enc is None else do_enc.contiguous()
        B, Hq, L, _ = q_dec.shape
        dq_dec = torch.empty_like(q_dec)
        dk_ctx, dv_ctx = torch.empty_like(k_ctx), torch.empty_like(v_ctx)
        dk_dec, dv_dec = torch.empty_like(k_dec), torch.empty_like(v_dec)
        dq_enc = torch.empty_like(q_enc) if with_enc else None
        ws = torch.empty(e2d2_attn_train_bwd_workspace_bytes(BF16, B, Hq, L, with_enc),
                         dtype=torch.uint8, device=q_dec.device)
        enc = dict(q_enc=q_enc, o_enc=o_enc, lse_enc=lse_enc, do_enc=do_enc,
                   dq_enc=dq_enc) if with_enc else {}
        e2d2_attn_train_bwd(q_dec, k_ctx, v_ctx, k_dec, v_dec, o_dec, lse_dec, do_dec, ctx.S,
                            dq_dec, dk_ctx, dv_ctx, dk_dec, dv_dec, ws, scale=ctx.scale, **enc)
        return dq_dec, dk_ctx, dv_ctx, dk_dec, dv_dec, dq_enc, None, None


def e2d2_attention(q_dec, k_ctx, v_ctx, k_dec, v_dec, S: int, q_enc=None, scale=None):
    """Differentiable E2D2 training attention (bf16).

    q_dec [B, Hq, L, d] attends [clean | noised] keys: k_ctx/v_ctx [B, Hkv, L, d] of
    earlier blocks and k_dec/v_dec [B, Hkv, L, d] of its own block, in one softmax.
    With q_enc, the encoder's block-causal attention of (q_enc, k_ctx, v_ctx) runs in
    the same launch.  Returns o_dec, or (o_dec, o_enc); gradients flow to every input
    (k_ctx, v_ctx collect those of both attentions)."""
    if q_dec.dtype != torch.bfloat16:
        raise ValueError("e2d2_attention is bf16 (the backward's dtype)")
    return _E2D2Attention.apply(q_dec, k_ctx, v_ctx, k_dec, v_dec, q_enc, int(S), scale)
