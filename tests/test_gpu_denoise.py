"""GPU parity of the denoising step and the KV-cache append against the fp64 oracle
(needs an MI355X).  Tolerances as in test_gpu_train.py; the append is a bitwise copy.
"""
import math
import sys

import numpy as np
import pytest
import torch

import masked_attention_amd as m
import oracle
from helpers import TensorKind as K, check, counter, gpu_fill, host, scale_of
from synth import host_tensor, tensor_id

pytestmark = pytest.mark.gpu


def say(msg):
    print(msg, file=sys.__stderr__, flush=True)


def _workspace(dtype, B, Hq, Hkv, S, d, C):
    code = m.BF16 if dtype == "bf16" else m.F32
    n = m.e2d2_attn_denoise_workspace_bytes(code, B, Hq, Hkv, S, d, C)
    return (torch.empty(n, dtype=torch.uint8, device="cuda") if n else None), n


def _denoise_case(B, Hq, Hkv, S, d, C, cap, dtype, seed, heads=None, step=0, inputs=None):
    say(f"[denoise] B{B} Hq{Hq} Hkv{Hkv} S{S} d{d} C{C} cap{cap} {dtype} seed {seed:#x}"
        + (" shaped scores" if inputs is not None else ""))
    if inputs is None:
        q = host((B, Hq, S, d), seed, K.Q_BLK, dtype, step=step)
        kb = host((B, Hkv, S, d), seed, K.K_BLK, dtype, step=step)
        vb = host((B, Hkv, S, d), seed, K.V_BLK, dtype, step=step)
        kc = host((B, Hkv, cap, d), seed, K.K_CACHE, dtype)
        vc = host((B, Hkv, cap, d), seed, K.V_CACHE, dtype)
    else:
        q, kc, vc, kb, vb = (inputs[n] for n in ("q", "kc", "vc", "kb", "vb"))
    g = [t.cuda() for t in (q, kc, vc, kb, vb)]
    o = torch.full_like(g[0], float("nan"))
    lse = torch.full((B, Hq, S), float("nan"), device="cuda")
    ws, nws = _workspace(dtype, B, Hq, Hkv, S, d, C)
    vis = counter()
    m.e2d2_attn_denoise_step(g[0], g[1], g[2], C, g[3], g[4], o, lse_blk=lse, workspace=ws,
                             tile_visits=vis)
    torch.cuda.synchronize()
    ro, rl = oracle.denoise_step(q, kc, vc, C, kb, vb, scale_of(d), heads=heads)
    hs = heads if heads is not None else [(b, h) for b in range(B) for h in range(Hq)]
    for b, h in hs:
        check(o[b, h], ro[b, h], dtype, f"o[{b},{h}]")
        check(lse[b, h], rl[b, h], dtype, f"lse[{b},{h}]")
    code = m.BF16 if dtype == "bf16" else m.F32
    bm, bn = m.e2d2_attn_tile_shape(m.KIND_DENOISE, code, d)
    want = m.e2d2_attn_count_tiles(m.KIND_DENOISE, B, Hq, 0, S, C, bm, bn)[0]
    brute = oracle.count_tiles(oracle.denoise_mask(S, C), bm, bn, [(0, C), (C, C + S)])[0]
    assert want == brute * B * Hq
    assert int(vis.item()) == want
    return o, lse, nws


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("B,Hq,Hkv,S,d,C,cap", [
    (2, 4, 2, 8, 64, 100, 130),      # small batch: key axis split over workgroups
    (1, 2, 1, 32, 128, 4096, 4096),  # grouped heads + split + workspace
    (3, 2, 2, 64, 32, 77, 200),      # two 32-row chunks per head
    (2, 4, 2, 48, 128, 33, 64),      # ragged row chunk and ragged key tiles
    (1, 1, 1, 4, 64, 0, 8),          # empty cache: own block only
    (1, 8, 1, 5, 64, 300, 300),      # eight query heads on one kv head
])
def test_denoise_shapes(B, Hq, Hkv, S, d, C, cap, dtype):
    _denoise_case(B, Hq, Hkv, S, d, C, cap, dtype, 0xE2D2D000 + C + S)


# The online softmax's rescaling, and the split path's merge of partial results, under
# scores that climb along the cache: every query row is 16 u plus small noise, u a unit
# direction per KV head, cache key j is span * sqrt(d) / 16 * (j / C) u plus N(0, 1)
# noise (the running max rises in most tiles and differs between the key slices that the
# split path merges), and the block's own keys are N(0, 1).  Span 200 nats in bf16, 8 in
# fp32 (where the scores' own rounding stays inside the 1e-5 bound).
@pytest.mark.parametrize("dtype,span,B,C", [
    ("bf16", 200.0, 1, 4000), ("bf16", 200.0, 8, 700), ("f32", 8.0, 1, 4000),
])
def test_rescaling_under_growing_cache_scores(dtype, span, B, C):
    Hq, Hkv, S, d = 4, 2, 16, 128
    seed = 0xE2D2DC01
    g = lambda shape, kind, step=0: host(shape, seed, kind, "f32", step=step).double()
    u = g((B, Hkv, 1, d), K.K_CACHE, step=1)
    u = u / u.norm(dim=-1, keepdim=True)
    j = torch.arange(C, dtype=torch.float64).view(1, 1, C, 1) / C
    dt = torch.bfloat16 if dtype == "bf16" else torch.float32
    inputs = dict(
        q=16.0 * u.repeat_interleave(Hq // Hkv, dim=1) + 0.1 * g((B, Hq, S, d), K.Q_BLK),
        kc=span * math.sqrt(d) / 16.0 * j * u + g((B, Hkv, C, d), K.K_CACHE),
        vc=g((B, Hkv, C, d), K.V_CACHE), kb=g((B, Hkv, S, d), K.K_BLK),
        vb=g((B, Hkv, S, d), K.V_BLK))
    inputs = {n: t.to(dt) for n, t in inputs.items()}
    _denoise_case(B, Hq, Hkv, S, d, C, C, dtype, seed, inputs=inputs)


def test_split_path_is_used():
    _, _, nws = _denoise_case(1, 2, 1, 32, 128, 4096, 4096, "bf16", 0xE2D2D100)
    assert nws > 0


def test_denoise_full_size_shared_kv_cache():
    # B32 Hq16 Hkv8 d128, cache 2048, block 32: all heads checked.
    _denoise_case(32, 16, 8, 32, 128, 2048, 2080, "bf16", 0xE2D20003, step=0)


def test_denoise_step_equals_training_rows():
    # Exact caching: the denoising step of block b over (clean prefix keys, own block
    # keys) reproduces the training decoder's rows of block b.
    B, Hq, Hkv, L, S, d = 2, 4, 2, 192, 32, 128
    seed = 0xE2D2D200
    qd = host((B, Hq, L, d), seed, K.Q_DEC, "bf16").cuda()
    kc, vc, kd, vd = (host((B, Hkv, L, d), seed, k, "bf16").cuda()
                      for k in (K.K_CTX, K.V_CTX, K.K_DEC, K.V_DEC))
    od = torch.empty_like(qd)
    ld = torch.empty((B, Hq, L), device="cuda")
    m.e2d2_attn_train_fwd(qd, kc, vc, kd, vd, od, S, lse_dec=ld)
    for blk in range(L // S):
        s0 = blk * S
        o = torch.empty((B, Hq, S, d), dtype=torch.bfloat16, device="cuda")
        lse = torch.empty((B, Hq, S), device="cuda")
        ws, _ = _workspace("bf16", B, Hq, Hkv, S, d, s0)
        m.e2d2_attn_denoise_step(qd[:, :, s0:s0 + S].contiguous(), kc, vc, s0,
                                 kd[:, :, s0:s0 + S].contiguous(), vd[:, :, s0:s0 + S].contiguous(),
                                 o, lse_blk=lse, workspace=ws)
        torch.cuda.synchronize()
        check(o, od[:, :, s0:s0 + S].double().cpu().numpy(), "bf16", f"block {blk} o")
        check(lse, ld[:, :, s0:s0 + S].double().cpu().numpy(), "bf16", f"block {blk} lse")


def test_append_is_bitwise_copy():
    for dtype in ("bf16", "f32"):
        B, Hkv, cap, S, d = 3, 2, 50, 7, 64
        kc = host((B, Hkv, cap, d), 5, K.K_CACHE, dtype).cuda()
        vc = host((B, Hkv, cap, d), 5, K.V_CACHE, dtype).cuda()
        kn = host((B, Hkv, S, d), 5, K.K_NEW, dtype).cuda()
        vn = host((B, Hkv, S, d), 5, K.V_NEW, dtype).cuda()
        k0, v0 = kc.clone(), vc.clone()
        m.e2d2_kv_cache_append(kc, vc, 40, kn, vn)
        torch.cuda.synchronize()
        want_k = oracle.kv_cache_append(k0.cpu().float().numpy(), 40, kn.cpu().float().numpy())
        want_v = oracle.kv_cache_append(v0.cpu().float().numpy(), 40, vn.cpu().float().numpy())
        assert np.array_equal(kc.cpu().float().numpy(), want_k)
        assert np.array_equal(vc.cpu().float().numpy(), want_v)
        with pytest.raises(m.E2D2Error):
            m.e2d2_kv_cache_append(kc, vc, 44, kn, vn)


def test_near_ar_decode_full_size_with_appends():
    # B64 H32 (MHA) d128, cache 32768, block 4: 16 blocks of 4 steps, the finished
    # block's K/V appended after each block.  Caches (2 x 17 GB) are filled on the GPU;
    # eight fixed heads are checked against the oracle at every one of the 64 steps, their
    # cache rows rebuilt on the host from the same generator (the prefix once, then each
    # appended block).
    B, H, d, C0, S, T, NB = 64, 32, 128, 32768, 4, 4, 16
    cap = C0 + S * NB
    seed = 0xE2D20005
    say(f"[near-AR] B{B} H{H} d{d} C0 {C0} S{S} T{T} blocks {NB}")
    kc = gpu_fill((B, H, cap, d), seed, K.K_CACHE, "bf16", rows=C0)
    vc = gpu_fill((B, H, cap, d), seed, K.V_CACHE, "bf16", rows=C0)
    heads = [(0, 0), (17, 5), (63, 31), (5, 30), (31, 16), (42, 1), (50, 9), (9, 23)]
    host_k = {bh: host_tensor(seed, tensor_id(K.K_CACHE), (1, 1, C0, d), "bf16", b0=bh[0], h0=bh[1])
              for bh in heads}
    host_v = {bh: host_tensor(seed, tensor_id(K.V_CACHE), (1, 1, C0, d), "bf16", b0=bh[0], h0=bh[1])
              for bh in heads}
    o = torch.empty((B, H, S, d), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((B, H, S), device="cuda")
    ws, _ = _workspace("bf16", B, H, H, S, d, cap)
    assert ws is None
    C = C0
    for blk in range(NB):
        for t in range(T):
            q = gpu_fill((B, H, S, d), seed, K.Q_BLK, "bf16", step=t, block=blk)
            kb = gpu_fill((B, H, S, d), seed, K.K_BLK, "bf16", step=t, block=blk)
            vb = gpu_fill((B, H, S, d), seed, K.V_BLK, "bf16", step=t, block=blk)
            m.e2d2_attn_denoise_step(q, kc, vc, C, kb, vb, o, lse_blk=lse)
            torch.cuda.synchronize()
            for b, h in heads:
                # oracle inputs for head (b, h): regenerate only that slice
                qh = host_tensor(seed, tensor_id(K.Q_BLK, t, blk), (1, 1, S, d), "bf16", b0=b, h0=h)
                kbh = host_tensor(seed, tensor_id(K.K_BLK, t, blk), (1, 1, S, d), "bf16", b0=b, h0=h)
                vbh = host_tensor(seed, tensor_id(K.V_BLK, t, blk), (1, 1, S, d), "bf16", b0=b, h0=h)
                assert host_k[(b, h)].shape[2] == C
                ro, rl = oracle.denoise_step(qh, host_k[(b, h)], host_v[(b, h)], C, kbh, vbh, scale_of(d))
                check(o[b, h], ro[0, 0], "bf16", f"block {blk} step {t} o[{b},{h}]")
                check(lse[b, h], rl[0, 0], "bf16", f"block {blk} step {t} lse[{b},{h}]")
        kn = gpu_fill((B, H, S, d), seed, K.K_NEW, "bf16", block=blk)
        vn = gpu_fill((B, H, S, d), seed, K.V_NEW, "bf16", block=blk)
        m.e2d2_kv_cache_append(kc, vc, C, kn, vn)
        for b, h in heads:
            host_k[(b, h)] = torch.cat([host_k[(b, h)], host_tensor(seed, tensor_id(K.K_NEW, 0, blk),
                                                                    (1, 1, S, d), "bf16", b0=b, h0=h)], dim=2)
            host_v[(b, h)] = torch.cat([host_v[(b, h)], host_tensor(seed, tensor_id(K.V_NEW, 0, blk),
                                                                    (1, 1, S, d), "bf16", b0=b, h0=h)], dim=2)
        C += S
    torch.cuda.synchronize()
    assert C == cap
