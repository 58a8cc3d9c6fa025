"""fp64 masked softmax attention for the three E2D2 attention calls, and the cache append.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Pages cited, by title and section:
  [Notes]   "Encoder-Decoder Diffusion Language Models for Efficient Training and
            Inference", Paper-Notes page (zhaoyang97.github.io).
  [Summary] ai.info "AI summary" page on the same paper.

What is computed (the plain definition, nothing blocked, fused or reordered):
  for one (batch, query head) and every requested query row i,
      s_ij = scale * <q_i, k_j>       for allowed (i, j), else -inf
      m_i  = max_j s_ij,  p_ij = exp(s_ij - m_i),  l_i = sum_j p_ij
      o_i  = sum_j p_ij v_j / l_i,    lse_i = m_i + ln(l_i)
  with ONE softmax over every allowed key, whichever source it comes from: the fused
  self+cross attention puts encoder keys and the block's own keys in a single call
  ([Notes] 方法详解 §2 两种连接方式), and the decoder then has to share its attention
  between the two ([Notes] 局限性).

Readings taken where the pages are silent:
  * scale arrives as a float32 (1/sqrt(d) in the workloads); the oracle uses that
    float32 value exactly, widened to fp64;
  * LSE is the natural-log log-sum-exp of the scaled scores over allowed keys;
  * grouped query heads: query head hq reads key/value head hq // (Hq // Hkv);
  * inputs are the exact bf16 or fp32 values the device receives, widened to fp64.
Query rows are independent by definition, so rows may be requested in any subset;
large requests are evaluated a slab of rows at a time only to bound memory.
"""
from __future__ import annotations

import numpy as np

from .masks import bd3lm_mask, decoder_mask, denoise_mask, encoder_mask

_ROW_SLAB = 512


def _f64(x) -> np.ndarray:
    """Widen a numpy array or CPU torch tensor (bf16, fp32, fp64) to a float64 ndarray."""
    if hasattr(x, "detach"):
        x = x.detach().cpu().double().numpy()
    return np.asarray(x, dtype=np.float64)


def _scale64(scale) -> float:
    return float(np.float32(scale))


def masked_softmax_attention(q, k, v, allowed, scale):
    """q [M, d], k [N, d], v [N, d], allowed [M, N] bool -> (o [M, d], lse [M]) in fp64.

    Every row must allow at least one key (no row of any E2D2 mask is empty: each
    query sees at least its own block)."""
    q = _f64(q)
    k = _f64(k)
    v = _f64(v)
    allowed = np.asarray(allowed, dtype=bool)
    if allowed.shape != (q.shape[0], k.shape[0]):
        raise ValueError("mask shape does not match q and k")
    if q.shape[0] and not allowed.any(axis=1).all():
        raise ValueError("a query row has no allowed key")
    s = (q @ k.T) * _scale64(scale)
    s = np.where(allowed, s, -np.inf)
    m = s.max(axis=1)
    p = np.exp(s - m[:, None])
    l = p.sum(axis=1)
    o = (p @ v) / l[:, None]
    lse = m + np.log(l)
    return o, lse


def _rows_arg(rows, n):
    return np.arange(n) if rows is None else np.asarray(rows, dtype=np.int64)


def _kv_head(hq: int, Hq: int, Hkv: int) -> int:
    if Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    return hq // (Hq // Hkv)


def _run_rows(q_bh, keys, vals, mask_rows_fn, rows, scale):
    """Evaluate the requested rows of one (batch, head), a slab of rows at a time."""
    o = np.empty((len(rows), vals.shape[1]))
    lse = np.empty(len(rows))
    for s0 in range(0, len(rows), _ROW_SLAB):
        r = rows[s0:s0 + _ROW_SLAB]
        o[s0:s0 + len(r)], lse[s0:s0 + len(r)] = masked_softmax_attention(
            q_bh[r], keys, vals, mask_rows_fn(r), scale)
    return o, lse


def encoder_blockcausal(q, k, v, S: int, scale, rows=None, heads=None):
    """Encoder block-causal attention ([Notes] §4 训练算法: a clean token attends to its
    own block and every earlier block).

    q [B, Hq, L, d]; k, v [B, Hkv, L, d].  ``rows``: query rows to evaluate (default
    all); ``heads``: iterable of (b, hq) to evaluate (default all).  Returns
    o [B, Hq, R, d] and lse [B, Hq, R] in fp64 (NaN where a head was not requested)."""
    B, Hq, L, d = q.shape
    Hkv = k.shape[1]
    rows = _rows_arg(rows, L)
    o = np.full((B, Hq, len(rows), v.shape[3]), np.nan)
    lse = np.full((B, Hq, len(rows)), np.nan)
    full = encoder_mask(L, S)
    for b, hq in (heads if heads is not None else [(b, h) for b in range(B) for h in range(Hq)]):
        hk = _kv_head(hq, Hq, Hkv)
        o[b, hq], lse[b, hq] = _run_rows(_f64(q[b, hq]), _f64(k[b, hk]), _f64(v[b, hk]),
                                         lambda r: full[r], rows, scale)
    return o, lse


def decoder_fused(q_dec, k_ctx, v_ctx, k_dec, v_dec, S: int, scale, rows=None, heads=None):
    """Decoder fused self+cross attention over 2L keys [clean context | noised block
    keys] ([Notes] §4 训练算法 and §2 两种连接方式).  Shapes as in encoder_blockcausal;
    returns o [B, Hq, R, d], lse [B, Hq, R] in fp64."""
    B, Hq, L, d = q_dec.shape
    Hkv = k_ctx.shape[1]
    rows = _rows_arg(rows, L)
    o = np.full((B, Hq, len(rows), v_ctx.shape[3]), np.nan)
    lse = np.full((B, Hq, len(rows)), np.nan)
    full = decoder_mask(L, S)
    for b, hq in (heads if heads is not None else [(b, h) for b in range(B) for h in range(Hq)]):
        hk = _kv_head(hq, Hq, Hkv)
        keys = np.concatenate([_f64(k_ctx[b, hk]), _f64(k_dec[b, hk])], axis=0)
        vals = np.concatenate([_f64(v_ctx[b, hk]), _f64(v_dec[b, hk])], axis=0)
        o[b, hq], lse[b, hq] = _run_rows(_f64(q_dec[b, hq]), keys, vals,
                                         lambda r: full[r], rows, scale)
    return o, lse


def train_fwd(q_dec, k_ctx, v_ctx, k_dec, v_dec, S: int, scale, q_enc=None, rows=None,
              heads=None):
    """One training forward of both E2D2 attentions ([Notes] §4 训练算法: all blocks in
    one encoder pass and one decoder pass).  Returns (o_dec, lse_dec, o_enc, lse_enc);
    the encoder pair is None when ``q_enc`` is None.  The encoder half attends the
    clean context keys/values (k_ctx, v_ctx), which are the encoder's own K/V."""
    o_dec, lse_dec = decoder_fused(q_dec, k_ctx, v_ctx, k_dec, v_dec, S, scale, rows, heads)
    if q_enc is None:
        return o_dec, lse_dec, None, None
    o_enc, lse_enc = encoder_blockcausal(q_enc, k_ctx, v_ctx, S, scale, rows, heads)
    return o_dec, lse_dec, o_enc, lse_enc


def bd3lm_layer(q, k, v, S: int, scale, heads=None):
    """Attention of one decoder-only block-diffusion layer over 2L tokens [noised |
    clean] with the explicit 2L x 2L mask (masks.bd3lm_mask): q, k, v [B, H*, 2L, d]
    (query heads Hq, kv heads Hkv).  Returns o [B, Hq, 2L, d], lse [B, Hq, 2L]."""
    B, Hq, L2, d = q.shape
    Hkv = k.shape[1]
    if L2 % 2:
        raise ValueError("the sequence must hold 2L tokens")
    mask = bd3lm_mask(L2 // 2, S)
    o = np.full((B, Hq, L2, v.shape[3]), np.nan)
    lse = np.full((B, Hq, L2), np.nan)
    for b, hq in (heads if heads is not None else [(b, h) for b in range(B) for h in range(Hq)]):
        hk = _kv_head(hq, Hq, Hkv)
        o[b, hq], lse[b, hq] = _run_rows(_f64(q[b, hq]), _f64(k[b, hk]), _f64(v[b, hk]),
                                         lambda r: mask[r], np.arange(L2), scale)
    return o, lse


def denoise_step(q_blk, k_cache, v_cache, cache_len: int, k_blk, v_blk, scale, heads=None):
    """One denoising step ([Notes] §3 采样算法; [Summary] "Methodology in Plain
    English"): the S queries of the current block attend every cached clean key
    (rows [0, cache_len) of the cache) and every key of their own block.

    q_blk [B, Hq, S, d]; k_cache, v_cache [B, Hkv, cap, d]; k_blk, v_blk [B, Hkv, S, d].
    Returns o [B, Hq, S, d], lse [B, Hq, S] in fp64."""
    B, Hq, S, d = q_blk.shape
    Hkv = k_blk.shape[1]
    C = int(cache_len)
    if C < 0 or C > k_cache.shape[2]:
        raise ValueError("cache_len outside the cache")
    o = np.full((B, Hq, S, v_blk.shape[3]), np.nan)
    lse = np.full((B, Hq, S), np.nan)
    mask = denoise_mask(S, C)
    for b, hq in (heads if heads is not None else [(b, h) for b in range(B) for h in range(Hq)]):
        hk = _kv_head(hq, Hq, Hkv)
        keys = np.concatenate([_f64(k_cache[b, hk, :C]), _f64(k_blk[b, hk])], axis=0)
        vals = np.concatenate([_f64(v_cache[b, hk, :C]), _f64(v_blk[b, hk])], axis=0)
        o[b, hq], lse[b, hq] = masked_softmax_attention(_f64(q_blk[b, hq]), keys, vals, mask,
                                                        scale)
    return o, lse


def kv_cache_append(cache: np.ndarray, cache_len: int, new: np.ndarray) -> np.ndarray:
    """Cache after a finished block's clean K (or V) rows are appended at row
    ``cache_len`` ([Notes] §3 采样算法: the finished block goes through the encoder,
    which updates the KV cache).  cache [B, H, cap, d]; new [B, H, S, d].  Returns a
    copy; raises when the block does not fit."""
    cache = np.array(cache, copy=True)
    S = new.shape[2]
    if cache_len < 0 or cache_len + S > cache.shape[2]:
        raise ValueError("append past the cache capacity")
    cache[:, :, cache_len:cache_len + S] = new
    return cache
