"""fp64 attention sublayer of one decoder layer in a denoising step: the projections
around the denoise attention.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Pages cited, by title and section:
  [Notes]   "Encoder-Decoder Diffusion Language Models for Efficient Training and
            Inference", Paper-Notes page (zhaoyang97.github.io): 方法详解 §2 两种连接方式
            (shared KV cache: a decoder layer reuses an encoder layer's KV cache for the
            clean context), §3 采样算法 (every denoising step of a block calls only the
            small decoder on the block's tokens; the cost per block is one encoder pass
            plus T decoder passes).

What is computed, for hidden states x [B, S, Dm] of the block's S noised tokens:
    qkv = x W_qkv^T                       W_qkv [(Hq + 2 Hkv) d, Dm]: the d rows of
                                          query head 0, 1, ..., then of key head 0,
                                          ..., then of value head 0, ...
    q [B, Hq, S, d], k, v [B, Hkv, S, d]  the per-head slices of qkv
    (o, lse) = denoise attention of q over the cached clean keys/values (rows
               [0, C) of the encoder's cache) and the block's own k, v
    y = o_cat W_o^T                       o_cat [B, S, Hq d] with head h's d values at
                                          columns [h d, h d + d); W_o [Dm, Hq d]
Readings (the pages give no layer code):
  * the sublayer is the attention part only (projections and attention); norms,
    residual and MLP are outside it;
  * the layer's activations q, k, v and o are bf16 tensors: with store_bf16 (the
    default) they are rounded to the nearest bf16 value (ties to even) where the
    layer stores them; every other step is fp64.
"""
from __future__ import annotations

import numpy as np

from .attention import _f64, denoise_step


def round_bf16(x) -> np.ndarray:
    """Nearest bf16 value (8 significant bits, ties to even) of each fp64 element, as
    fp64.  x = m 2^e with 0.5 <= |m| < 1, and m is rounded to a multiple of 2^-8.
    Finite values inside the bf16 normal range only (no overflow handling)."""
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)
    return np.ldexp(np.round(m * 256.0) / 256.0, e)


def decoder_layer_denoise(x, w_qkv, w_o, k_cache, v_cache, cache_len: int, Hq: int, Hkv: int,
                          d: int, scale, store_bf16: bool = True):
    """One denoising step of a decoder layer's attention sublayer (module docstring).

    x [B, S, Dm]; w_qkv [(Hq + 2 Hkv) d, Dm]; w_o [Dm, Hq d]; k_cache, v_cache
    [B, Hkv, cap, d] (rows [0, cache_len) used).  Returns (q, k, v, o, lse, y) in fp64:
    q, o [B, Hq, S, d]; k, v [B, Hkv, S, d]; lse [B, Hq, S]; y [B, S, Dm]."""
    x = _f64(x)
    w_qkv = _f64(w_qkv)
    w_o = _f64(w_o)
    B, S, Dm = x.shape
    if w_qkv.shape != ((Hq + 2 * Hkv) * d, Dm):
        raise ValueError("w_qkv must be [(Hq + 2 Hkv) d, Dm]")
    if w_o.shape != (Dm, Hq * d):
        raise ValueError("w_o must be [Dm, Hq d]")
    rnd = round_bf16 if store_bf16 else (lambda t: t)
    qkv = x @ w_qkv.T  # [B, S, (Hq + 2 Hkv) d]

    def heads(cols, H):
        return rnd(cols.reshape(B, S, H, d).transpose(0, 2, 1, 3))

    q = heads(qkv[:, :, :Hq * d], Hq)
    k = heads(qkv[:, :, Hq * d:(Hq + Hkv) * d], Hkv)
    v = heads(qkv[:, :, (Hq + Hkv) * d:], Hkv)
    o, lse = denoise_step(q, k_cache, v_cache, cache_len, k, v, scale)
    o = rnd(o)
    o_cat = o.transpose(0, 2, 1, 3).reshape(B, S, Hq * d)
    y = o_cat @ w_o.T
    return q, k, v, o, lse, y
