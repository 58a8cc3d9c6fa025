"""GPU parity of the per-sequence-length denoising step and KV-cache append (a batch
decoded together, each sequence at its own cache length) against the fp64 oracle
applied sequence by sequence.  Tolerances as in test_gpu_train.py; appends bitwise.
"""
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


def _inputs(B, Hq, Hkv, S, d, cap, seed, step=0):
    q = host((B, Hq, S, d), seed, K.Q_BLK, "bf16", step=step)
    kb = host((B, Hkv, S, d), seed, K.K_BLK, "bf16", step=step)
    vb = host((B, Hkv, S, d), seed, K.V_BLK, "bf16", step=step)
    kc = host((B, Hkv, cap, d), seed, K.K_CACHE, "bf16")
    vc = host((B, Hkv, cap, d), seed, K.V_CACHE, "bf16")
    return q, kc, vc, kb, vb


def _workspace(B, Hq, Hkv, S, d, C):
    n = m.e2d2_attn_denoise_workspace_bytes(m.BF16, B, Hq, Hkv, S, d, C)
    return torch.empty(n, dtype=torch.uint8, device="cuda") if n else None


@pytest.mark.parametrize("B,Hq,Hkv,S,d,lens,max_len,cap", [
    (6, 4, 2, 8, 64, [0, 1, 31, 32, 200, 300], 300, 308),       # ragged tiles, empty cache
    (4, 16, 8, 32, 128, [2048, 1000, 33, 2047], 2048, 2080),    # the denoise workload's heads
    (1, 2, 1, 8, 128, [1500], 4096, 4104),                      # split key axis + workspace
    (3, 2, 2, 4, 32, [5, 0, 64], 100, 104),
])
def test_varlen_step_matches_oracle_per_sequence(B, Hq, Hkv, S, d, lens, max_len, cap):
    _varlen_case(B, Hq, Hkv, S, d, lens, max_len, cap, 0xE2D20007)


def _varlen_case(B, Hq, Hkv, S, d, lens, max_len, cap, seed):
    say(f"[varlen] B{B} Hq{Hq} Hkv{Hkv} S{S} d{d} lens {lens} max {max_len} seed {seed:#x}")
    q, kc, vc, kb, vb = _inputs(B, Hq, Hkv, S, d, cap, seed)
    g = [t.cuda() for t in (q, kc, vc, kb, vb)]
    lens_t = torch.tensor(lens, dtype=torch.int32, device="cuda")
    o = torch.full_like(g[0], float("nan"))
    lse = torch.full((B, Hq, S), float("nan"), device="cuda")
    vis = counter()
    m.e2d2_attn_denoise_step_varlen(g[0], g[1], g[2], lens_t, max_len, g[3], g[4], o,
                                    lse_blk=lse, workspace=_workspace(B, Hq, Hkv, S, d, max_len),
                                    tile_visits=vis)
    torch.cuda.synchronize()
    visits = 0
    for b, C in enumerate(lens):
        ro, rl = oracle.denoise_step(q[b:b + 1], kc[b:b + 1], vc[b:b + 1], C, kb[b:b + 1],
                                     vb[b:b + 1], scale_of(d))
        for h in range(Hq):
            check(o[b, h], ro[0, h], "bf16", f"o[{b},{h}] C={C}")
            check(lse[b, h], rl[0, h], "bf16", f"lse[{b},{h}] C={C}")
        visits += m.e2d2_attn_count_tiles(m.KIND_DENOISE, 1, Hq, 0, S, C, 32, 32)[0]
    assert int(vis.item()) == visits


def test_varlen_full_size_bench_lengths():
    # The per-sequence-length workload as timed: B32 Hq16/Hkv8 d128, block 32, cache
    # capacity 2048 + 32, lengths drawn from [1024, 2048] with the same seeded generator,
    # inputs filled on the GPU.  Every query head of four sequences (the shortest, the
    # longest and two others) is checked against the oracle; the tile-visit counter
    # against the host schedule summed over all 32 sequences.
    B, Hq, Hkv, d, S, max_len = 32, 16, 8, 128, 32, 2048
    cap = max_len + S
    seed = 0xE2D20009
    lens = np.random.RandomState(seed & 0xFFFFFFFF).randint(1024, max_len + 1, size=B)
    say(f"[varlen full] B{B} Hq{Hq} Hkv{Hkv} d{d} S{S} lens {int(lens.min())}..{int(lens.max())}")
    kc = gpu_fill((B, Hkv, cap, d), seed, K.K_CACHE, "bf16", rows=max_len)
    vc = gpu_fill((B, Hkv, cap, d), seed, K.V_CACHE, "bf16", rows=max_len)
    q = gpu_fill((B, Hq, S, d), seed, K.Q_BLK, "bf16", step=0)
    kb = gpu_fill((B, Hkv, S, d), seed, K.K_BLK, "bf16", step=0)
    vb = gpu_fill((B, Hkv, S, d), seed, K.V_BLK, "bf16", step=0)
    o = torch.full((B, Hq, S, d), float("nan"), dtype=torch.bfloat16, device="cuda")
    lse = torch.full((B, Hq, S), float("nan"), device="cuda")
    vis = counter()
    m.e2d2_attn_denoise_step_varlen(q, kc, vc, torch.tensor(lens, dtype=torch.int32, device="cuda"),
                                    max_len, kb, vb, o, lse_blk=lse,
                                    workspace=_workspace(B, Hq, Hkv, S, d, max_len), tile_visits=vis)
    torch.cuda.synchronize()
    want = sum(m.e2d2_attn_count_tiles(m.KIND_DENOISE, 1, Hq, 0, S, int(C), 32, 32)[0] for C in lens)
    assert int(vis.item()) == want
    picks = sorted({int(lens.argmin()), int(lens.argmax()), 7, 20})
    for b in picks:
        C = int(lens[b])
        qh = host_tensor(seed, tensor_id(K.Q_BLK, 0), (1, Hq, S, d), "bf16", b0=b)
        kch = host_tensor(seed, tensor_id(K.K_CACHE), (1, Hkv, C, d), "bf16", b0=b)
        vch = host_tensor(seed, tensor_id(K.V_CACHE), (1, Hkv, C, d), "bf16", b0=b)
        kbh = host_tensor(seed, tensor_id(K.K_BLK, 0), (1, Hkv, S, d), "bf16", b0=b)
        vbh = host_tensor(seed, tensor_id(K.V_BLK, 0), (1, Hkv, S, d), "bf16", b0=b)
        ro, rl = oracle.denoise_step(qh, kch, vch, C, kbh, vbh, scale_of(d))
        for h in range(Hq):
            check(o[b, h], ro[0, h], "bf16", f"o[{b},{h}] C={C}")
            check(lse[b, h], rl[0, h], "bf16", f"lse[{b},{h}] C={C}")


def test_varlen_with_equal_lengths_is_the_uniform_step_bitwise():
    B, Hq, Hkv, S, d, C, cap = 4, 8, 4, 32, 128, 777, 800
    q, kc, vc, kb, vb = (t.cuda() for t in _inputs(B, Hq, Hkv, S, d, cap, 0xE2D20008))
    o1, o2 = torch.empty_like(q), torch.empty_like(q)
    l1, l2 = (torch.empty((B, Hq, S), device="cuda") for _ in range(2))
    ws = _workspace(B, Hq, Hkv, S, d, C)
    m.e2d2_attn_denoise_step(q, kc, vc, C, kb, vb, o1, lse_blk=l1, workspace=ws)
    lens_t = torch.full((B,), C, dtype=torch.int32, device="cuda")
    m.e2d2_attn_denoise_step_varlen(q, kc, vc, lens_t, C, kb, vb, o2, lse_blk=l2, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_varlen_graph_replays_follow_device_lengths():
    # One captured step replayed while the lengths advance on the device (as a decode
    # loop does between blocks): every replay equals an eager call at those lengths.
    B, Hq, Hkv, S, d, cap = 3, 4, 2, 8, 64, 256
    q, kc, vc, kb, vb = (t.cuda() for t in _inputs(B, Hq, Hkv, S, d, cap, 0xE2D20009))
    max_len = cap - S
    lens_t = torch.tensor([10, 100, 0], dtype=torch.int32, device="cuda")
    o = torch.empty_like(q)
    lse = torch.empty((B, Hq, S), device="cuda")
    ws = _workspace(B, Hq, Hkv, S, d, max_len)

    def step(out, lse_out):
        m.e2d2_attn_denoise_step_varlen(q, kc, vc, lens_t, max_len, kb, vb, out, lse_blk=lse_out,
                                        workspace=ws)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step(o, lse)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step(o, lse)
    ref_o, ref_l = torch.empty_like(o), torch.empty_like(lse)
    for it in range(4):
        lens_t += 16  # eager update between replays
        graph.replay()
        torch.cuda.synchronize()
        step(ref_o, ref_l)
        torch.cuda.synchronize()
        assert torch.equal(o, ref_o) and torch.equal(lse, ref_l), f"replay {it}"
    # and against the oracle at the final lengths
    lens = lens_t.cpu().tolist()
    qh, kch, vch, kbh, vbh = (t.cpu() for t in (q, kc, vc, kb, vb))
    for b, C in enumerate(lens):
        ro, rl = oracle.denoise_step(qh[b:b + 1], kch[b:b + 1], vch[b:b + 1], C, kbh[b:b + 1],
                                     vbh[b:b + 1], scale_of(d))
        check(o[b], ro[0], "bf16", f"o[{b}] C={C}")
        check(lse[b], rl[0], "bf16", f"lse[{b}] C={C}")


def test_append_varlen_writes_each_sequence_at_its_length():
    B, Hkv, S, d, cap, max_len = 4, 2, 8, 64, 64, 56
    kc = torch.randn(B, Hkv, cap, d, device="cuda").to(torch.bfloat16)
    vc = torch.randn(B, Hkv, cap, d, device="cuda").to(torch.bfloat16)
    kn = torch.randn(B, Hkv, S, d, device="cuda").to(torch.bfloat16)
    vn = torch.randn(B, Hkv, S, d, device="cuda").to(torch.bfloat16)
    k0, v0 = kc.clone(), vc.clone()
    lens = [0, 13, 56, 57]  # the last is past max_len: left untouched
    m.e2d2_kv_cache_append_varlen(kc, vc, torch.tensor(lens, dtype=torch.int32, device="cuda"),
                                  max_len, kn, vn)
    torch.cuda.synchronize()
    for b, C in enumerate(lens):
        if C > max_len:
            assert torch.equal(kc[b], k0[b]) and torch.equal(vc[b], v0[b])
            continue
        assert torch.equal(kc[b, :, C:C + S], kn[b]) and torch.equal(vc[b, :, C:C + S], vn[b])
        assert torch.equal(kc[b, :, :C], k0[b, :, :C]) and torch.equal(kc[b, :, C + S:], k0[b, :, C + S:])
        assert torch.equal(vc[b, :, :C], v0[b, :, :C]) and torch.equal(vc[b, :, C + S:], v0[b, :, C + S:])
