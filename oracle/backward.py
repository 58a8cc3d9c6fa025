"""fp64 gradients of the E2D2 training attentions (the backward pass).

TEST INFRASTRUCTURE ONLY (see the package docstring).

Pages cited, by title and section:
  [Notes]   "Encoder-Decoder Diffusion Language Models for Efficient Training and
            Inference", Paper-Notes page (zhaoyang97.github.io): 方法详解 §4 训练算法
            (training runs one encoder pass over the clean blocks and one decoder pass
            over the noised blocks and learns from the decoder's loss, so the
            gradient flows through both attentions; the clean keys/values feed both).

The pages print no backward; what is computed is the derivative of the forward in
oracle.attention, written out by the chain rule.  For one (batch, query head) with
scores s_ij = scale <q_i, k_j> on allowed pairs and upstream gradient do_i:
    p_ij  = exp(s_ij - lse_i)                 (0 where the pair is not allowed)
    dv_j  = sum_i p_ij do_i
    dp_ij = <do_i, v_j>
    ds_ij = p_ij (dp_ij - sum_j' p_ij' dp_ij')
    dq_i  = scale sum_j ds_ij k_j
    dk_j  = scale sum_i ds_ij q_i
Every query head adds its dk, dv into the key/value head it reads (grouped heads),
and the clean context keys/values collect the gradients of both attentions that read
them: the encoder's block-causal attention and the decoder's cross half.
"""
from __future__ import annotations

import numpy as np

from .attention import _f64, _kv_head, _scale64
from .masks import decoder_mask, encoder_mask


def masked_softmax_attention_grad(q, k, v, allowed, scale, do):
    """Gradients of o = softmax(scale q k^T on allowed pairs) v for one head.

    q, do [M, d]; k, v [N, d]; allowed [M, N] bool.  Returns (dq [M, d], dk [N, d],
    dv [N, d]) in fp64."""
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(do)
    allowed = np.asarray(allowed, dtype=bool)
    sc = _scale64(scale)
    s = np.where(allowed, (q @ k.T) * sc, -np.inf)
    m = s.max(axis=1, keepdims=True)
    e = np.exp(s - m)
    p = e / e.sum(axis=1, keepdims=True)
    dv = p.T @ do
    dp = do @ v.T
    ds = p * (dp - (p * dp).sum(axis=1, keepdims=True))
    dq = sc * (ds @ k)
    dk = sc * (ds.T @ q)
    return dq, dk, dv


def train_bwd(q_dec, k_ctx, v_ctx, k_dec, v_dec, S: int, scale, do_dec, q_enc=None,
              do_enc=None, kv_heads=None):
    """Gradients of one training forward of both E2D2 attentions (oracle.attention.
    train_fwd) for upstream gradients do_dec (and do_enc when q_enc is given).

    Shapes: q_dec, do_dec, q_enc, do_enc [B, Hq, L, d]; k_ctx, v_ctx, k_dec, v_dec
    [B, Hkv, L, d].  ``kv_heads``: iterable of (b, hk) to evaluate (default all); a kv
    head's gradients need every query head of its group, which are evaluated with it.
    Returns (dq_dec, dk_ctx, dv_ctx, dk_dec, dv_dec, dq_enc) in fp64, NaN where not
    evaluated; dq_enc is None when q_enc is None."""
    B, Hq, L, d = q_dec.shape
    Hkv = k_ctx.shape[1]
    g = Hq // Hkv
    if Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    with_enc = q_enc is not None
    if with_enc and do_enc is None:
        raise ValueError("do_enc is needed with q_enc")
    dq_dec = np.full(q_dec.shape, np.nan)
    dq_enc = np.full(q_dec.shape, np.nan) if with_enc else None
    dk_ctx = np.full(k_ctx.shape, np.nan)
    dv_ctx = np.full(k_ctx.shape, np.nan)
    dk_dec = np.full(k_ctx.shape, np.nan)
    dv_dec = np.full(k_ctx.shape, np.nan)
    mdec = decoder_mask(L, S)
    menc = encoder_mask(L, S)
    for b, hk in (kv_heads if kv_heads is not None else [(b, h) for b in range(B) for h in range(Hkv)]):
        kc, vc, kd, vd = (_f64(t[b, hk]) for t in (k_ctx, v_ctx, k_dec, v_dec))
        keys = np.concatenate([kc, kd], axis=0)
        vals = np.concatenate([vc, vd], axis=0)
        acc_k = np.zeros((2 * L, d))
        acc_v = np.zeros((2 * L, d))
        for hq in range(hk * g, (hk + 1) * g):
            assert _kv_head(hq, Hq, Hkv) == hk
            dq, dk, dv = masked_softmax_attention_grad(q_dec[b, hq], keys, vals, mdec, scale,
                                                       do_dec[b, hq])
            dq_dec[b, hq] = dq
            acc_k += dk
            acc_v += dv
            if with_enc:
                dq, dk, dv = masked_softmax_attention_grad(q_enc[b, hq], kc, vc, menc, scale,
                                                           do_enc[b, hq])
                dq_enc[b, hq] = dq
                acc_k[:L] += dk
                acc_v[:L] += dv
        dk_ctx[b, hk], dk_dec[b, hk] = acc_k[:L], acc_k[L:]
        dv_ctx[b, hk], dv_dec[b, hk] = acc_v[:L], acc_v[L:]
    return dq_dec, dk_ctx, dv_ctx, dk_dec, dv_dec, dq_enc
