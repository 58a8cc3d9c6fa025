"""GPU parity of the encoder side of the sampling loop against the fp64 oracle.

"Encoder-Decoder Diffusion Language Models for Efficient Training and Inference",
Paper-Notes page, 方法详解 §3 采样算法: sampling encodes the prompt into the encoder's
KV cache, runs the decoder T times per block against that cache, then feeds the
finished block to the encoder, which extends the cache.  Covered here:
  * the encoder update of a finished block is e2d2_attn_denoise_step with the block's
    clean queries and its own K/V; its rows equal the training encoder's rows of that
    block (a clean token sees its own and every earlier block);
  * prompt encoding for prompts of different lengths
    (e2d2_attn_encoder_blockcausal_varlen), K/V read in the cache layout, lengths read
    on the device (also from a replayed HIP graph while the lengths change);
  * a short sampling loop -- prompt encode, decoder steps, encoder updates, appends,
    all with per-sequence lengths -- whose encoder outputs equal the one-shot training
    encoder over the finished sequence (exact caching) and whose cache ends up holding
    exactly the sequence's K/V.
Tolerances as in test_gpu_train.py (bf16: |got - ref| <= 2e-2 on O and LSE); cache
contents bitwise.
"""
import sys

import numpy as np
import pytest
import torch

import masked_attention_amd as m
import oracle
from helpers import TensorKind as K, check, counter, gpu_fill, host, scale_of

pytestmark = pytest.mark.gpu

SENT_O, SENT_LSE = 3.0, -5.0  # values rows past a sequence's end must keep


def say(msg):
    print(msg, file=sys.__stderr__, flush=True)


def _ws(B, Hq, Hkv, S, d, C):
    n = m.e2d2_attn_denoise_workspace_bytes(m.BF16, B, Hq, Hkv, S, d, C)
    return torch.empty(n, dtype=torch.uint8, device="cuda") if n else None


# ----------------------------------------------------------------------------- encoder update
@pytest.mark.parametrize("B,Hq,Hkv,d,S,nblk,blocks", [
    (1, 2, 1, 32, 8, 5, [0, 2, 4]),         # tiny; block 0 has an empty cache
    (2, 4, 2, 64, 16, 7, [3, 6]),
    (1, 2, 2, 128, 5, 9, [1, 8]),           # a block size that is not a tile multiple
])
def test_encoder_update_equals_training_encoder_rows(B, Hq, Hkv, d, S, nblk, blocks):
    L = nblk * S
    seed = 0xE2D2E000 + d + S
    say(f"[enc-update] B{B} Hq{Hq} Hkv{Hkv} d{d} S{S} L{L} blocks {blocks}")
    q = host((B, Hq, L, d), seed, K.Q_ENC, "bf16")
    k = host((B, Hkv, L, d), seed, K.K_CTX, "bf16")
    v = host((B, Hkv, L, d), seed, K.V_CTX, "bf16")
    _update_case(q, k, v, S, blocks, heads=None)


def test_encoder_update_denoise_workload_heads():
    # the denoise workload's heads: B32 Hq16 Hkv8 d128, block 32, a cache of 2048 clean
    # rows, i.e. the update of block 64; inputs drawn on the device (bit-identical to
    # the host generator) and copied back for the oracle
    B, Hq, Hkv, d, S = 32, 16, 8, 128, 32
    L = 2048 + S
    seed = 0xE2D2E100
    say(f"[enc-update] denoise workload B{B} Hq{Hq} Hkv{Hkv} d{d} cache 2048 block {S}")
    q = gpu_fill((B, Hq, L, d), seed, K.Q_ENC, "bf16").cpu()
    k = gpu_fill((B, Hkv, L, d), seed, K.K_CTX, "bf16").cpu()
    v = gpu_fill((B, Hkv, L, d), seed, K.V_CTX, "bf16").cpu()
    _update_case(q, k, v, S, [64], heads=None)


def _update_case(q, k, v, S, blocks, heads):
    B, Hq, L, d = q.shape
    Hkv = k.shape[1]
    cap = L + 8
    gq = q.cuda()
    kc = torch.zeros((B, Hkv, cap, d), dtype=torch.bfloat16, device="cuda")
    vc = torch.zeros_like(kc)
    kc[:, :, :L] = k.cuda()
    vc[:, :, :L] = v.cuda()
    for blk in blocks:
        r0, r1 = blk * S, min(L, (blk + 1) * S)
        n = r1 - r0
        if n != S:
            continue
        q_blk = gq[:, :, r0:r1].contiguous()
        k_blk = kc[:, :, r0:r1].contiguous()
        v_blk = vc[:, :, r0:r1].contiguous()
        o = torch.full((B, Hq, S, d), float("nan"), dtype=torch.bfloat16, device="cuda")
        lse = torch.full((B, Hq, S), float("nan"), device="cuda")
        # the cache holds the clean rows before the block (rows past r0 are not read)
        m.e2d2_attn_denoise_step(q_blk, kc, vc, r0, k_blk, v_blk, o, lse_blk=lse,
                                 workspace=_ws(B, Hq, Hkv, S, d, r0))
        torch.cuda.synchronize()
        ro, rl = oracle.encoder_blockcausal(q, k, v, S, scale_of(d), rows=np.arange(r0, r1),
                                            heads=heads)
        check(o, ro, "bf16", f"encoder update O, block {blk}")
        check(lse, rl, "bf16", f"encoder update LSE, block {blk}")


# ----------------------------------------------------------------------------- prompt encode
def _tile_count(Hq, L, S, d):
    bm, bn = m.e2d2_attn_tile_shape(m.KIND_ENC, m.BF16, d)
    return m.e2d2_attn_count_tiles(m.KIND_ENC, 1, Hq, L, S, 0, bm, bn)[0] if L > 0 else 0


def _prompt_inputs(B, Hq, Hkv, L, d, kv_rows, seed):
    q = host((B, Hq, L, d), seed, K.Q_ENC, "bf16")
    k = host((B, Hkv, kv_rows, d), seed, K.K_CACHE, "bf16")
    v = host((B, Hkv, kv_rows, d), seed, K.V_CACHE, "bf16")
    return q, k, v


def _check_prompt(o, lse, q, k, v, lens, S, what):
    d = q.shape[3]
    for b, n in enumerate(lens):
        n = max(0, min(int(n), q.shape[2]))
        if n > 0:
            ro, rl = oracle.encoder_blockcausal(q[b:b + 1, :, :n], k[b:b + 1, :, :n],
                                                v[b:b + 1, :, :n], S, scale_of(d))
            check(o[b:b + 1, :, :n], ro, "bf16", f"{what} O, sequence {b} (length {n})")
            check(lse[b:b + 1, :, :n], rl, "bf16", f"{what} LSE, sequence {b} (length {n})")
        rest_o = o[b, :, n:].float().cpu()
        rest_l = lse[b, :, n:].cpu()
        assert bool((rest_o == SENT_O).all()), f"{what}: rows past sequence {b}'s end written"
        assert bool((rest_l == SENT_LSE).all()), f"{what}: LSE past sequence {b}'s end written"


@pytest.mark.parametrize("B,Hq,Hkv,L,S,d,lens,kv_rows", [
    (4, 4, 2, 200, 16, 64, [0, 1, 150, 200], 256),     # empty, one-token and full prompts
    (3, 16, 8, 300, 32, 128, [300, 33, 129], 330),     # the denoise workload's heads
    (2, 2, 2, 70, 1, 32, [70, 64], 70),                # block size 1: causal
    (2, 2, 1, 130, 130, 64, [130, 77], 140),           # one block: bidirectional prompt
    (3, 8, 8, 1024, 16, 64, [1024, 999, 513], 1100),   # the training workload's head shape
])
def test_prompt_encode_varlen_matches_oracle(B, Hq, Hkv, L, S, d, lens, kv_rows):
    seed = 0xE2D2E200 + L + S + d
    say(f"[prompt] B{B} Hq{Hq} Hkv{Hkv} L{L} S{S} d{d} lens {lens} kv_rows {kv_rows}")
    q, k, v = _prompt_inputs(B, Hq, Hkv, L, d, kv_rows, seed)
    g = [t.cuda() for t in (q, k, v)]
    lens_t = torch.tensor(lens, dtype=torch.int32, device="cuda")
    o = torch.full((B, Hq, L, d), SENT_O, dtype=torch.bfloat16, device="cuda")
    lse = torch.full((B, Hq, L), SENT_LSE, device="cuda")
    vis = counter()
    m.e2d2_attn_encoder_blockcausal_varlen(g[0], g[1], g[2], lens_t, o, S, lse=lse, tile_visits=vis)
    torch.cuda.synchronize()
    _check_prompt(o, lse, q, k, v, lens, S, "prompt encode")
    assert int(vis.item()) == sum(_tile_count(Hq, n, S, d) for n in lens)


def test_prompt_encode_full_lengths_equal_encoder_call():
    # every length at L and K/V rows = L: the per-sequence call is the plain encoder
    B, Hq, Hkv, L, S, d = 2, 4, 2, 256, 16, 64
    q, k, v = _prompt_inputs(B, Hq, Hkv, L, d, L, 0xE2D2E300)
    g = [t.cuda() for t in (q, k, v)]
    lens_t = torch.full((B,), L, dtype=torch.int32, device="cuda")
    o1, o2 = torch.empty_like(g[0]), torch.empty_like(g[0])
    l1, l2 = (torch.empty((B, Hq, L), device="cuda") for _ in range(2))
    m.e2d2_attn_encoder_blockcausal_varlen(g[0], g[1], g[2], lens_t, o1, S, lse=l1)
    m.e2d2_attn_encoder_blockcausal(g[0], g[1], g[2], o2, S, lse=l2)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_prompt_encode_graph_replay_follows_device_lengths():
    # one captured launch, replayed while the lengths change on the device
    B, Hq, Hkv, L, S, d = 3, 4, 2, 160, 16, 64
    q, k, v = _prompt_inputs(B, Hq, Hkv, L, d, L + 16, 0xE2D2E400)
    g = [t.cuda() for t in (q, k, v)]
    lens_t = torch.tensor([16, 100, 160], dtype=torch.int32, device="cuda")
    o = torch.full((B, Hq, L, d), SENT_O, dtype=torch.bfloat16, device="cuda")
    lse = torch.full((B, Hq, L), SENT_LSE, device="cuda")

    def call():
        m.e2d2_attn_encoder_blockcausal_varlen(g[0], g[1], g[2], lens_t, o, S, lse=lse)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call()
    torch.cuda.synchronize()
    for lens in ([16, 100, 160], [160, 0, 37], [1, 64, 129]):
        o.fill_(SENT_O)
        lse.fill_(SENT_LSE)
        lens_t.copy_(torch.tensor(lens, dtype=torch.int32))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        _check_prompt(o, lse, q, k, v, lens, S, f"graph replay, lengths {lens}")


# ----------------------------------------------------------------------------- sampling loop
@pytest.mark.parametrize("prompts,aligned", [([16, 8, 24], True), ([13, 8, 21], False)])
def test_sampling_loop_matches_oracle(prompts, aligned):
    """Prompt encode, then per block T decoder steps, the encoder update and the append,
    every sequence at its own length.  The clean sequence of sequence b is drawn up
    front: positions [0, P_b) its prompt, then block j at [P_b + j S, P_b + (j+1) S);
    Q_ENC / K_CTX / V_CTX are the encoder's queries and K/V of those positions."""
    B, Hq, Hkv, d, S, T, nblk = 3, 4, 2, 64, 8, 2, 3
    seed = 0xE2D2E500 + (1 if aligned else 0)
    Ltot = max(prompts) + nblk * S
    cap = Ltot + S
    scale = scale_of(d)
    say(f"[loop] prompts {prompts} S{S} T{T} blocks {nblk} d{d}")
    q_all = host((B, Hq, Ltot, d), seed, K.Q_ENC, "bf16")
    k_all = host((B, Hkv, Ltot, d), seed, K.K_CTX, "bf16")
    v_all = host((B, Hkv, Ltot, d), seed, K.V_CTX, "bf16")
    # clean sequence b: prompt rows [0, P_b) then its nblk blocks, taken from row P_b on
    kc = torch.zeros((B, Hkv, cap, d), dtype=torch.bfloat16, device="cuda")
    vc = torch.zeros_like(kc)
    for b, P in enumerate(prompts):  # the prompt's K/V, written straight into the cache
        kc[b, :, :P] = k_all[b, :, :P].cuda()
        vc[b, :, :P] = v_all[b, :, :P].cuda()
    lens_t = torch.tensor(prompts, dtype=torch.int32, device="cuda")
    maxP = max(prompts)

    # 1. prompt encode
    qp = q_all[:, :, :maxP].contiguous()
    o = torch.full((B, Hq, maxP, d), SENT_O, dtype=torch.bfloat16, device="cuda")
    lse = torch.full((B, Hq, maxP), SENT_LSE, device="cuda")
    m.e2d2_attn_encoder_blockcausal_varlen(qp.cuda(), kc, vc, lens_t, o, S, lse=lse)
    torch.cuda.synchronize()
    _check_prompt(o, lse, qp, k_all, v_all, prompts, S, "loop prompt encode")

    ws = _ws(B, Hq, Hkv, S, d, Ltot)
    for j in range(nblk):
        lens = [P + j * S for P in prompts]
        # 2. T decoder steps against the cache (fresh noised block each step)
        for t in range(T):
            qd = host((B, Hq, S, d), seed, K.Q_BLK, "bf16", step=t, block=j)
            kd = host((B, Hkv, S, d), seed, K.K_BLK, "bf16", step=t, block=j)
            vd = host((B, Hkv, S, d), seed, K.V_BLK, "bf16", step=t, block=j)
            od = torch.empty((B, Hq, S, d), dtype=torch.bfloat16, device="cuda")
            ld = torch.empty((B, Hq, S), device="cuda")
            m.e2d2_attn_denoise_step_varlen(qd.cuda(), kc, vc, lens_t, Ltot, kd.cuda(), vd.cuda(),
                                            od, lse_blk=ld, workspace=ws)
            torch.cuda.synchronize()
            kch, vch = kc.cpu(), vc.cpu()
            for b, C in enumerate(lens):
                ro, rl = oracle.denoise_step(qd[b:b + 1], kch[b:b + 1], vch[b:b + 1], C,
                                             kd[b:b + 1], vd[b:b + 1], scale)
                check(od[b:b + 1], ro, "bf16", f"block {j} step {t} decoder O, seq {b}")
                check(ld[b:b + 1], rl, "bf16", f"block {j} step {t} decoder LSE, seq {b}")
        # 3. encoder update of the finished block, then 4. append its K/V
        qe = torch.stack([q_all[b, :, C:C + S] for b, C in enumerate(lens)])
        ke = torch.stack([k_all[b, :, C:C + S] for b, C in enumerate(lens)])
        ve = torch.stack([v_all[b, :, C:C + S] for b, C in enumerate(lens)])
        oe = torch.empty((B, Hq, S, d), dtype=torch.bfloat16, device="cuda")
        le = torch.empty((B, Hq, S), device="cuda")
        gk, gv = ke.cuda(), ve.cuda()
        m.e2d2_attn_denoise_step_varlen(qe.cuda(), kc, vc, lens_t, Ltot, gk, gv, oe, lse_blk=le,
                                        workspace=ws)
        m.e2d2_kv_cache_append_varlen(kc, vc, lens_t, Ltot, gk, gv)
        lens_t += S
        torch.cuda.synchronize()
        for b, C in enumerate(lens):
            if aligned:
                # exact caching: the incremental update equals the one-shot training
                # encoder over the whole clean sequence, rows of this block
                n = prompts[b] + nblk * S
                ro, rl = oracle.encoder_blockcausal(q_all[b:b + 1, :, :n], k_all[b:b + 1, :, :n],
                                                    v_all[b:b + 1, :, :n], S, scale,
                                                    rows=np.arange(C, C + S))
            else:
                # prompt blocks off the grid: the update is the cache plus its own block
                ro, rl = oracle.denoise_step(qe[b:b + 1], k_all[b:b + 1], v_all[b:b + 1], C,
                                             ke[b:b + 1], ve[b:b + 1], scale)
            check(oe[b:b + 1], ro, "bf16", f"block {j} encoder update O, seq {b}")
            check(le[b:b + 1], rl, "bf16", f"block {j} encoder update LSE, seq {b}")
    assert lens_t.cpu().tolist() == [P + nblk * S for P in prompts]
    kch, vch = kc.cpu(), vc.cpu()
    for b, P in enumerate(prompts):
        n = P + nblk * S
        assert torch.equal(kch[b, :, :n], k_all[b, :, :n]), f"cache K of sequence {b}"
        assert torch.equal(vch[b, :, :n], v_all[b, :, :n]), f"cache V of sequence {b}"
