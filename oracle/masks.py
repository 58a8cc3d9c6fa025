"""Block index, the three attention masks, and pair / tile counting (fp-free, exact).

TEST INFRASTRUCTURE ONLY (see the package docstring).

Pages cited, by title and section:
  [Notes]   "Encoder-Decoder Diffusion Language Models for Efficient Training and
            Inference", Paper-Notes page (zhaoyang97.github.io), NeurIPS 2025 notes.
  [Summary] ai.info "AI summary" page on the same paper.
  [BD3]     "Block Diffusion: Interpolating Between Autoregressive and Diffusion
            Language Models", xllm-io paper review.

Readings taken where the pages leave a step open:
  * blocks start at position 0 and hold S consecutive tokens, the last one may be
    shorter ([BD3] 三 技术架构, 块级分解);
  * inside a block attention is bidirectional; the encoder row sees its own block and
    every earlier block ([Notes] 方法详解 §4 训练算法);
  * a decoder (noised) row sees the clean keys of strictly earlier blocks plus the
    noised keys of its own block, over a 2L-key axis ordered [clean | noised]
    ([Notes] §4 训练算法);
  * a denoising step's S queries see every cached clean key plus every key of their
    own block ([Notes] §3 采样算法; [Summary] "Methodology in Plain English").
"""
from __future__ import annotations

import numpy as np


def block_of(pos, S: int):
    """Block index of token position(s) ``pos`` for block size ``S``: floor(pos / S)."""
    if S <= 0:
        raise ValueError("block size must be positive")
    return np.asarray(pos) // S


def encoder_mask(L: int, S: int) -> np.ndarray:
    """[L, L] bool: clean query i may attend clean key j iff block(j) <= block(i)."""
    i = np.arange(L)[:, None]
    j = np.arange(L)[None, :]
    return block_of(j, S) <= block_of(i, S)


def decoder_mask(L: int, S: int) -> np.ndarray:
    """[L, 2L] bool over keys [clean 0..L-1 | noised 0..L-1]: noised query i may attend
    clean key j iff block(j) < block(i), and noised key j iff block(j) == block(i)."""
    i = np.arange(L)[:, None]
    j = np.arange(L)[None, :]
    clean = block_of(j, S) < block_of(i, S)
    noised = block_of(j, S) == block_of(i, S)
    return np.concatenate([clean, noised], axis=1)


def bd3lm_mask(L: int, S: int) -> np.ndarray:
    """[2L, 2L] bool of a decoder-only block-diffusion layer over the sequence
    [noised 0..L-1 | clean 0..L-1] ([Notes] 背景与动机: such a model processes the whole
    clean sequence and the whole noised sequence, 2L tokens, in one stack; FLOPs table,
    BD3LM row).  Noised query i (block b) may attend noised key j iff block(j) == b and
    clean key j iff block(j) < b; clean query i may attend clean key j iff block(j) <= b
    and no noised key (the clean stream must not see the noise)."""
    i = np.arange(L)[:, None]
    j = np.arange(L)[None, :]
    bi, bj = block_of(i, S), block_of(j, S)
    noised_rows = np.concatenate([bj == bi, bj < bi], axis=1)
    clean_rows = np.concatenate([np.zeros((L, L), dtype=bool), bj <= bi], axis=1)
    return np.concatenate([noised_rows, clean_rows], axis=0)


def denoise_mask(S: int, C: int) -> np.ndarray:
    """[S, C+S] bool over keys [cache 0..C-1 | own block 0..S-1]: all allowed."""
    return np.ones((S, C + S), dtype=bool)


def count_pairs(mask: np.ndarray) -> int:
    """Number of allowed (query, key) pairs."""
    return int(np.count_nonzero(mask))


def count_tiles(mask: np.ndarray, bm: int, bn: int, sources) -> tuple[int, int]:
    """Visited and full tiles of ``mask`` for query tiles of ``bm`` rows (from row 0)
    and key tiles of ``bn`` columns laid out separately inside each key source
    ``(start, end)``.  A tile is visited when it holds at least one allowed pair and
    full when every (existing) pair in it is allowed."""
    M = mask.shape[0]
    visited = 0
    full = 0
    for r0 in range(0, M, bm):
        rows = mask[r0:min(M, r0 + bm)]
        for (c_start, c_end) in sources:
            for c0 in range(c_start, c_end, bn):
                t = rows[:, c0:min(c_end, c0 + bn)]
                if t.any():
                    visited += 1
                    if t.all():
                        full += 1
    return visited, full
