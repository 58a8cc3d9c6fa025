"""Pins of the CPU oracle to facts fixed outside it (CPU only).

Each test ties an oracle function to something other than its own formula: masks
drawn by hand from the pages' prose, pair counts from the pages' FLOPs table, the
block-size-1 and block-size-L reductions the pages state, torch's scaled-dot-product
attention (a library routine) on those reductions, closed forms at Q = 0, brute force
with pure-Python loops on tiny shapes, and the exact-caching and blockwise
factorisation properties.

Pages cited, by title and section:
  [Notes]   "Encoder-Decoder Diffusion Language Models for Efficient Training and
            Inference", Paper-Notes page.
  [Summary] ai.info "AI summary" page on the same paper.
  [BD3]     "Block Diffusion: Interpolating Between Autoregressive and Diffusion
            Language Models", xllm-io review.
"""
import math
import os

import numpy as np
import pytest
import torch

import oracle
from synth import TensorKind, host_tensor, tensor_id

pytestmark = pytest.mark.filterwarnings("ignore::UserWarning")


# ----------------------------------------------------------------------------- fixtures
def _read_cases(path):
    cases = {}
    name = None
    for line in open(path, encoding="utf-8"):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        if line.startswith("case "):
            _, name, kind, ls, ss = line.split()
            cases[name] = dict(kind=kind, L=int(ls[2:]), S=int(ss[2:]), rows=[])
            continue
        cases[name]["rows"].append([c == "1" for c in line.replace("|", "")])
    return cases


def _read_table(path):
    out = {}
    for line in open(path, encoding="utf-8"):
        line = line.split("#")[0].strip()
        if line:
            model, expr = line.split(None, 1)
            out[model] = expr
    return out


def _rand(shape, seed, tid, dtype="f32"):
    return host_tensor(seed, tid, shape, dtype).double().numpy()


# ----------------------------------------------------------------------------- masks
def test_block_index_last_block_shorter():
    # [BD3] 三 技术架构, 块级分解: blocks of S tokens from the start, last may be shorter.
    assert list(oracle.block_of(np.arange(5), 2)) == [0, 0, 1, 1, 2]
    assert list(oracle.block_of(np.arange(7), 3)) == [0, 0, 0, 1, 1, 1, 2]
    with pytest.raises(ValueError):
        oracle.block_of(0, 0)


def test_masks_match_hand_drawn(golden_dir):
    cases = _read_cases(os.path.join(golden_dir, "masks_hand_drawn.txt"))
    assert len(cases) == 8
    for name, c in cases.items():
        want = np.array(c["rows"], dtype=bool)
        got = oracle.encoder_mask(c["L"], c["S"]) if c["kind"] == "encoder" \
            else oracle.decoder_mask(c["L"], c["S"])
        assert got.shape == want.shape, name
        assert np.array_equal(got, want), name


def test_pair_counts_match_flops_table(golden_dir):
    table = _read_table(os.path.join(golden_dir, "flops_table.txt"))
    for L in range(1, 49):
        for S in range(1, L + 1):
            enc = oracle.count_pairs(oracle.encoder_mask(L, S))
            dec = oracle.count_pairs(oracle.decoder_mask(L, S))
            # One encoder layer and one decoder layer evaluate the same number of pairs
            # for every S, ragged last block included.
            assert enc == dec, (L, S)
            if L % S == 0:
                assert enc == eval(table["E2D2"], {"L": L, "S": S}), (L, S)
                # BD3LM's single stack covers the clean half and the noised half.
                assert enc + dec == eval(table["BD3LM"], {"L": L, "S": S}), (L, S)
        # Block size L is full-sequence diffusion (MDLM): every pair allowed.
        assert oracle.count_pairs(oracle.encoder_mask(L, L)) == eval(table["MDLM"], {"L": L, "S": L})


def test_pair_counts_at_workload_shapes(golden_dir):
    table = _read_table(os.path.join(golden_dir, "flops_table.txt"))
    n = 0
    for line in open(os.path.join(golden_dir, "pair_counts.txt"), encoding="utf-8"):
        line = line.split("#")[0].strip()
        if not line:
            continue
        L, S, pairs = (int(x) for x in line.split()[:3])
        assert pairs == eval(table["E2D2"], {"L": L, "S": S})
        assert oracle.count_pairs(oracle.encoder_mask(L, S)) == pairs
        assert oracle.count_pairs(oracle.decoder_mask(L, S)) == pairs
        n += 1
    assert n == 5


def test_count_tiles_by_hand_and_aligned_closed_form():
    enc = oracle.encoder_mask(6, 2)
    # Tiles of 4x4 over a 6x6 block-causal mask (worked out by hand): (0,0) partial,
    # (0,1) empty, (1,0) full, (1,1) full.
    assert oracle.count_tiles(enc, 4, 4, [(0, 6)]) == (3, 2)
    # Tiles aligned with the blocks are all-or-nothing: n blocks give n(n+1)/2 tiles.
    for L, S in [(64, 8), (48, 4), (30, 5)]:
        n = L // S
        e = oracle.count_tiles(oracle.encoder_mask(L, S), S, S, [(0, L)])
        d = oracle.count_tiles(oracle.decoder_mask(L, S), S, S, [(0, L), (L, 2 * L)])
        assert e == (n * (n + 1) // 2,) * 2
        assert d == (n * (n + 1) // 2,) * 2
    # Denoise: every key of the cache and of the block is visited, all tiles full
    # except none (the mask is all ones); ragged key tiles still count once.
    assert oracle.count_tiles(oracle.denoise_mask(4, 100), 4, 32, [(0, 100), (100, 104)]) == (5, 5)


# ----------------------------------------------------------------------------- reductions
def _sdpa(q, k, v, scale, causal=False, mask=None):
    """torch's scaled-dot-product attention in fp64 on the CPU (library routine)."""
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a))[None, None]
    m = None if mask is None else torch.from_numpy(mask)[None, None]
    return torch.nn.functional.scaled_dot_product_attention(
        t(q), t(k), t(v), attn_mask=m, is_causal=causal, scale=float(np.float32(scale)))[0, 0].numpy()


def _lse_lib(q, k, mask, scale):
    from scipy.special import logsumexp

    s = (torch.from_numpy(q) @ torch.from_numpy(k).T).numpy() * float(np.float32(scale))
    return logsumexp(np.where(mask, s, -np.inf), axis=1)


@pytest.mark.parametrize("L,d", [(16, 8), (37, 16)])
def test_block_size_one_is_causal_attention(L, d):
    # [BD3] 二 核心思想: block size 1 is pure autoregression.
    q, k, v = (_rand((1, 1, L, d), 7, t)[0, 0] for t in (1, 2, 3))
    scale = 1 / math.sqrt(d)
    o, lse = oracle.encoder_blockcausal(q[None, None], k[None, None], v[None, None], 1, scale)
    np.testing.assert_allclose(o[0, 0], _sdpa(q, k, v, scale, causal=True), rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse[0, 0], _lse_lib(q, k, np.tril(np.ones((L, L), bool)), scale),
                               rtol=0, atol=1e-12)
    # Decoder with its clean context equal to its own keys is causal too: strictly earlier
    # clean keys plus the one own key.
    od, lsed = oracle.decoder_fused(q[None, None], k[None, None], v[None, None], k[None, None],
                                    v[None, None], 1, scale)
    np.testing.assert_allclose(od[0, 0], o[0, 0], rtol=0, atol=1e-12)
    np.testing.assert_allclose(lsed[0, 0], lse[0, 0], rtol=0, atol=1e-12)


@pytest.mark.parametrize("L,d", [(16, 8), (33, 4)])
def test_block_size_L_is_full_attention(L, d):
    # [BD3] 二 核心思想: block size equal to the sequence length is pure diffusion
    # (bidirectional attention over the whole sequence).
    q, k, v, kd, vd = (_rand((1, 1, L, d), 9, t)[0, 0] for t in (1, 2, 3, 5, 6))
    scale = 1 / math.sqrt(d)
    o, lse = oracle.encoder_blockcausal(q[None, None], k[None, None], v[None, None], L, scale)
    np.testing.assert_allclose(o[0, 0], _sdpa(q, k, v, scale), rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse[0, 0], _lse_lib(q, k, np.ones((L, L), bool), scale),
                               rtol=0, atol=1e-12)
    # The decoder's clean part is empty when there is one block: it attends its own
    # noised block only.
    od, lsed = oracle.decoder_fused(q[None, None], k[None, None], v[None, None], kd[None, None],
                                    vd[None, None], L, scale)
    np.testing.assert_allclose(od[0, 0], _sdpa(q, kd, vd, scale), rtol=0, atol=1e-12)
    np.testing.assert_allclose(lsed[0, 0], _lse_lib(q, kd, np.ones((L, L), bool), scale),
                               rtol=0, atol=1e-12)


@pytest.mark.parametrize("S", [1, 2, 3, 5, 8, 24])
def test_decoder_with_equal_sources_is_encoder(S):
    # Earlier clean blocks plus the own block is the same key set as "current and
    # earlier blocks" ([Notes] §4 训练算法), under one softmax ([Notes] §2).
    L, d = 24, 8
    q, k, v = (_rand((1, 2, L, d), 11, t) for t in (1, 2, 3))
    scale = 1 / math.sqrt(d)
    o, lse = oracle.encoder_blockcausal(q, k, v, S, scale)
    od, lsed = oracle.decoder_fused(q, k, v, k, v, S, scale)
    np.testing.assert_allclose(od, o, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lsed, lse, rtol=0, atol=1e-12)


def test_one_softmax_over_both_sources():
    # The fused call takes one softmax over [earlier clean | own noised] keys: its output
    # is the log-sum-exp weighted merge of attention over each source alone, computed
    # here with torch's library attention (masked per source).
    L, S, d = 12, 4, 8
    q, kc, vc, kd, vd = (_rand((1, 1, L, d), 13, t)[0, 0] for t in (4, 2, 3, 5, 6))
    scale = 1 / math.sqrt(d)
    od, lsed = oracle.decoder_fused(q[None, None], kc[None, None], vc[None, None],
                                    kd[None, None], vd[None, None], S, scale)
    blk = np.arange(L) // S
    own = blk[None, :] == blk[:, None]
    earlier = blk[None, :] < blk[:, None]
    o_own = _sdpa(q, kd, vd, scale, mask=own)
    l_own = _lse_lib(q, kd, own, scale)
    rows = np.nonzero(blk > 0)[0]
    o_ctx = _sdpa(q[rows], kc, vc, scale, mask=earlier[rows])
    l_ctx = _lse_lib(q[rows], kc, earlier[rows], scale)
    want = o_own.copy()
    want_l = l_own.copy()
    w1 = np.exp(l_ctx - np.logaddexp(l_ctx, l_own[rows]))
    want[rows] = w1[:, None] * o_ctx + (1 - w1)[:, None] * o_own[rows]
    want_l[rows] = np.logaddexp(l_ctx, l_own[rows])
    np.testing.assert_allclose(od[0, 0], want, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lsed[0, 0], want_l, rtol=0, atol=1e-12)


# ----------------------------------------------------------------------------- closed forms
@pytest.mark.parametrize("L,S", [(20, 4), (19, 4), (16, 1), (16, 16)])
def test_zero_queries_average_allowed_values(L, S):
    # With q = 0 every allowed key gets the same weight: o_i is the mean of the allowed
    # value rows and lse_i = ln(#allowed keys).  Allowed sets are written from block
    # boundaries here: [0, end of own block) for the encoder, [0, start of own block)
    # of the clean values plus the own block of the noised values for the decoder.
    d = 4
    v, vd = (_rand((1, 1, L, d), 17, t) for t in (3, 6))
    z = np.zeros((1, 1, L, d))
    k = _rand((1, 1, L, d), 17, 2)
    o, lse = oracle.encoder_blockcausal(z, k, v, S, 0.125)
    od, lsed = oracle.decoder_fused(z, k, v, k, vd, S, 0.125)
    for i in range(L):
        start = (i // S) * S
        end = min(L, start + S)
        np.testing.assert_allclose(o[0, 0, i], v[0, 0, :end].mean(axis=0), rtol=0, atol=1e-14)
        assert abs(lse[0, 0, i] - math.log(end)) < 1e-14
        pooled = np.concatenate([v[0, 0, :start], vd[0, 0, start:end]])
        np.testing.assert_allclose(od[0, 0, i], pooled.mean(axis=0), rtol=0, atol=1e-14)
        assert abs(lsed[0, 0, i] - math.log(end)) < 1e-14


def _brute(q, keys, vals, allowed_sets, scale):
    """Pure-Python loops on tiny inputs: softmax over the listed key indices."""
    sc = float(np.float32(scale))
    out, lses = [], []
    for i, allowed in enumerate(allowed_sets):
        s = {j: sc * sum(q[i][c] * keys[j][c] for c in range(len(q[i]))) for j in allowed}
        m = max(s.values())
        w = {j: math.exp(s[j] - m) for j in allowed}
        tot = sum(w.values())
        out.append([sum(w[j] * vals[j][c] for j in allowed) / tot for c in range(len(vals[0]))])
        lses.append(m + math.log(tot))
    return np.array(out), np.array(lses)


@pytest.mark.parametrize("L,S", [(5, 2), (6, 3), (7, 7), (4, 1)])
def test_brute_force_tiny(L, S):
    d = 3
    q, kc, vc, kd, vd = (_rand((1, 1, L, d), 23, t)[0, 0].tolist() for t in (1, 2, 3, 5, 6))
    blocks = [list(range(s, min(L, s + S))) for s in range(0, L, S)]
    own = {i: b for b in blocks for i in b}
    enc_sets = [[j for b in blocks if b[0] <= own[i][0] for j in b] for i in range(L)]
    dec_sets = [[j for b in blocks if b[0] < own[i][0] for j in b] + [L + j for j in own[i]]
                for i in range(L)]
    o, lse = oracle.encoder_blockcausal(np.array(q)[None, None], np.array(kc)[None, None],
                                        np.array(vc)[None, None], S, 0.5)
    bo, blse = _brute(q, kc, vc, enc_sets, 0.5)
    np.testing.assert_allclose(o[0, 0], bo, rtol=0, atol=1e-13)
    np.testing.assert_allclose(lse[0, 0], blse, rtol=0, atol=1e-13)
    od, lsed = oracle.decoder_fused(np.array(q)[None, None], np.array(kc)[None, None],
                                    np.array(vc)[None, None], np.array(kd)[None, None],
                                    np.array(vd)[None, None], S, 0.5)
    bo, blse = _brute(q, kc + kd, vc + vd, dec_sets, 0.5)
    np.testing.assert_allclose(od[0, 0], bo, rtol=0, atol=1e-13)
    np.testing.assert_allclose(lsed[0, 0], blse, rtol=0, atol=1e-13)


# ----------------------------------------------------------------------------- invariants
@pytest.mark.parametrize("L,S", [(24, 8), (22, 8), (16, 1)])
def test_denoise_step_equals_training_rows(L, S):
    # Caching is exact ([Summary] "Future Directions": exact encoder-decoder caching;
    # [Notes] §3 采样算法): block b's denoising step over the cached clean prefix plus
    # its own block equals the training decoder's rows of block b.
    B, Hq, Hkv, d = 2, 4, 2, 8
    qd = _rand((B, Hq, L, d), 29, 4)
    kc, vc, kd, vd = (_rand((B, Hkv, L, d), 29, t) for t in (2, 3, 5, 6))
    scale = 1 / math.sqrt(d)
    od, lsed = oracle.decoder_fused(qd, kc, vc, kd, vd, S, scale)
    for start in range(0, L, S):
        end = min(L, start + S)
        cap = np.zeros((B, Hkv, L + S, d))
        cap[:, :, :start] = kc[:, :, :start]
        o, lse = oracle.denoise_step(qd[:, :, start:end], cap, np.concatenate(
            [vc[:, :, :start], np.zeros((B, Hkv, L + S - start, d))], axis=2), start,
            kd[:, :, start:end], vd[:, :, start:end], scale)
        np.testing.assert_allclose(o, od[:, :, start:end], rtol=0, atol=1e-12)
        np.testing.assert_allclose(lse, lsed[:, :, start:end], rtol=0, atol=1e-12)


def test_blocks_do_not_see_the_future():
    # Blockwise autoregressive factorisation ([BD3] 三 技术架构, 块级自回归似然): rows of
    # block b are unchanged, bit for bit, when keys/values of later blocks change.
    L, S, d = 20, 4, 8
    q, qd = (_rand((1, 2, L, d), 31, t) for t in (1, 4))
    kc, vc, kd, vd = (_rand((1, 2, L, d), 31, t) for t in (2, 3, 5, 6))
    o, lse = oracle.encoder_blockcausal(q, kc, vc, S, 0.3)
    od, lsed = oracle.decoder_fused(qd, kc, vc, kd, vd, S, 0.3)
    for b in range(L // S):
        cut = (b + 1) * S
        pert = [x.copy() for x in (kc, vc, kd, vd)]
        for x in pert:
            x[:, :, cut:] += 5.0
        o2, lse2 = oracle.encoder_blockcausal(q, pert[0], pert[1], S, 0.3)
        od2, lsed2 = oracle.decoder_fused(qd, *pert, S, 0.3)
        assert np.array_equal(o2[:, :, :cut], o[:, :, :cut])
        assert np.array_equal(lse2[:, :, :cut], lse[:, :, :cut])
        assert np.array_equal(od2[:, :, :cut], od[:, :, :cut])
        assert np.array_equal(lsed2[:, :, :cut], lsed[:, :, :cut])
        if cut < L:
            assert not np.array_equal(o2[:, :, cut:], o[:, :, cut:])


def test_grouped_heads_match_repeated_heads():
    B, Hq, Hkv, L, S, d = 1, 6, 2, 10, 3, 4
    q = _rand((B, Hq, L, d), 37, 1)
    k, v = (_rand((B, Hkv, L, d), 37, t) for t in (2, 3))
    o, lse = oracle.encoder_blockcausal(q, k, v, S, 0.4)
    rep = lambda x: torch.from_numpy(x).repeat_interleave(Hq // Hkv, dim=1).numpy()
    o2, lse2 = oracle.encoder_blockcausal(q, rep(k), rep(v), S, 0.4)
    assert np.array_equal(o, o2) and np.array_equal(lse, lse2)


def test_row_subsets_and_heads_subsets():
    B, H, L, S, d = 2, 2, 12, 4, 4
    q, k, v = (_rand((B, H, L, d), 41, t) for t in (1, 2, 3))
    o, lse = oracle.encoder_blockcausal(q, k, v, S, 0.5)
    rows = [11, 0, 5]
    o2, lse2 = oracle.encoder_blockcausal(q, k, v, S, 0.5, rows=rows, heads=[(1, 0)])
    assert np.array_equal(o2[1, 0], o[1, 0, rows]) and np.array_equal(lse2[1, 0], lse[1, 0, rows])
    assert np.isnan(o2[0, 0]).all()


def test_scale_is_the_float32_value():
    L, d = 8, 5
    q, k, v = (_rand((1, 1, L, d), 43, t)[0, 0] for t in (1, 2, 3))
    scale = 1 / math.sqrt(d)
    o, _ = oracle.encoder_blockcausal(q[None, None], k[None, None], v[None, None], L, scale)
    np.testing.assert_allclose(o[0, 0], _sdpa(q, k, v, np.float32(scale)), rtol=0, atol=1e-13)


def test_empty_cache_denoise_is_attention_over_own_block():
    S, d = 6, 4
    q, kb, vb = (_rand((1, 1, S, d), 47, t) for t in (7, 8, 9))
    cache = np.zeros((1, 1, 10, d))
    o, lse = oracle.denoise_step(q, cache, cache, 0, kb, vb, 0.5)
    np.testing.assert_allclose(o[0, 0], _sdpa(q[0, 0], kb[0, 0], vb[0, 0], 0.5), rtol=0, atol=1e-13)
    with pytest.raises(ValueError):
        oracle.denoise_step(q, cache, cache, 11, kb, vb, 0.5)


def test_cache_append_is_a_copy():
    cache = _rand((2, 3, 10, 4), 53, 12)
    new = _rand((2, 3, 4, 4), 53, 10)
    out = oracle.kv_cache_append(cache, 5, new)
    assert np.array_equal(out[:, :, 5:9], new)
    assert np.array_equal(out[:, :, :5], cache[:, :, :5])
    assert np.array_equal(out[:, :, 9:], cache[:, :, 9:])
    with pytest.raises(ValueError):
        oracle.kv_cache_append(cache, 7, new)


def test_every_row_has_a_key():
    with pytest.raises(ValueError):
        oracle.masked_softmax_attention(np.zeros((2, 2)), np.zeros((3, 2)), np.zeros((3, 2)),
                                        np.array([[1, 0, 0], [0, 0, 0]], bool), 1.0)


def test_synth_inputs_are_reproducible_and_sliceable():
    a = host_tensor(5, tensor_id(TensorKind.Q_DEC), (2, 3, 40, 16), "bf16")
    b = host_tensor(5, tensor_id(TensorKind.Q_DEC), (1, 2, 10, 16), "bf16", n0=30, b0=1, h0=1)
    assert torch.equal(a[1:2, 1:3, 30:40], b)
    x = host_tensor(5, tensor_id(TensorKind.K_CACHE), (4, 8, 512, 64), "f32").numpy()
    assert abs(x.mean()) < 5e-3 and abs(x.var() - 1) < 5e-3
    assert not torch.equal(host_tensor(5, tensor_id(TensorKind.Q_BLK, step=1), (1, 1, 4, 8), "f32"),
                           host_tensor(5, tensor_id(TensorKind.Q_BLK, step=2), (1, 1, 4, 8), "f32"))


@pytest.mark.parametrize("L,S", [(L, S) for L in range(1, 41, 3) for S in (1, 2, 4, 5, 8) if S <= L])
def test_bd3lm_pair_count_is_twice_each_e2d2_mask(L, S):
    # FLOPs table: a decoder-only block-diffusion layer costs 4ND(L^2 + LS) attention
    # flops, an E2D2 encoder or decoder layer 4ND(L^2 + LS)/2: twice the pairs per layer.
    m = oracle.bd3lm_mask(L, S)
    n_bd = oracle.count_pairs(m)
    assert n_bd == oracle.count_pairs(oracle.encoder_mask(L, S)) + oracle.count_pairs(oracle.decoder_mask(L, S))
    if L % S == 0:
        assert n_bd == L * L + L * S


def test_bd3lm_block_size_one_and_L():
    # S = 1: clean half is causal attention and noised tokens see strictly earlier
    # clean tokens plus themselves; S = L: one block, noised tokens see only noised.
    L = 6
    m1 = oracle.bd3lm_mask(L, 1)
    assert np.array_equal(m1[L:, L:], np.tril(np.ones((L, L), dtype=bool)))
    assert np.array_equal(m1[:L, :L], np.eye(L, dtype=bool))
    assert np.array_equal(m1[:L, L:], np.tril(np.ones((L, L), dtype=bool), -1))
    mL = oracle.bd3lm_mask(L, L)
    assert mL[:L, :L].all() and not mL[:L, L:].any() and mL[L:, L:].all() and not mL[L:, :L].any()


def test_bd3lm_layer_is_the_fused_e2d2_call_on_its_halves():
    # Splitting the 2L tokens into [noised | clean] halves, the single-stack layer equals
    # the decoder attention of the noised half (clean keys as context) and the encoder
    # attention of the clean half.
    B, H, L, S, d = 1, 2, 10, 3, 4
    g = lambda kind: host_tensor(0xBD3, tensor_id(kind), (B, H, 2 * L, d), "f32")
    q, k, v = g(TensorKind.Q_DEC), g(TensorKind.K_CTX), g(TensorKind.V_CTX)
    o, lse = oracle.bd3lm_layer(q, k, v, S, 0.4)
    od, ld, oe, le = oracle.train_fwd(q[:, :, :L], k[:, :, L:], v[:, :, L:], k[:, :, :L],
                                      v[:, :, :L], S, 0.4, q_enc=q[:, :, L:])
    np.testing.assert_allclose(o[:, :, :L], od, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(o[:, :, L:], oe, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(lse[:, :, :L], ld, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(lse[:, :, L:], le, rtol=1e-12, atol=1e-12)
