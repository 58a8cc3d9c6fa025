"""The allocation-free denoising step (e2d2_attn_denoise_step_noalloc, called through
the C ABI) against e2d2_attn_denoise_step with a caller workspace, on two calls in a
row, the second smaller.  Both run the same kernels, so the outputs must be bitwise
equal; they are also checked against the fp64 oracle to the bf16 bar (2e-2).  The
shapes have few (batch, kv head) items, so the key axis is split and the scratch is
used."""
import sys

import pytest
import torch

import masked_attention_amd as m
import oracle
from helpers import TensorKind as K, check, host, scale_of

pytestmark = pytest.mark.gpu


def say(msg):
    print(msg, file=sys.__stderr__, flush=True)


def _case(B, Hq, Hkv, S, d, C, cap, seed):
    q = host((B, Hq, S, d), seed, K.Q_BLK, "bf16")
    kb = host((B, Hkv, S, d), seed, K.K_BLK, "bf16")
    vb = host((B, Hkv, S, d), seed, K.V_BLK, "bf16")
    kc = host((B, Hkv, cap, d), seed, K.K_CACHE, "bf16")
    vc = host((B, Hkv, cap, d), seed, K.V_CACHE, "bf16")
    return q, kc, vc, kb, vb


def test_noalloc_matches_workspace_call_twice_second_smaller():
    cases = [(1, 2, 1, 8, 128, 4000, 4096, 0xE2D2A100),   # 1 item: many splits
             (2, 4, 2, 4, 64, 1000, 1024, 0xE2D2A200)]    # smaller: fewer splits
    for B, Hq, Hkv, S, d, C, cap, seed in cases:
        need = m.e2d2_attn_denoise_workspace_bytes(m.BF16, B, Hq, Hkv, S, d, C)
        say(f"[noalloc] B{B} Hq{Hq} Hkv{Hkv} S{S} d{d} C{C}: workspace {need} bytes")
        assert need > 0, "the case must split the key axis"
        q, kc, vc, kb, vb = _case(B, Hq, Hkv, S, d, C, cap, seed)
        g = [t.cuda() for t in (q, kc, vc, kb, vb)]
        o_ref = torch.full_like(g[0], float("nan"))
        l_ref = torch.full((B, Hq, S), float("nan"), device="cuda")
        ws = torch.empty(need, dtype=torch.uint8, device="cuda")
        m.e2d2_attn_denoise_step(g[0], g[1], g[2], C, g[3], g[4], o_ref, lse_blk=l_ref,
                                 workspace=ws)
        o = torch.full_like(g[0], float("nan"))
        lse = torch.full((B, Hq, S), float("nan"), device="cuda")
        m.e2d2_attn_denoise_step_noalloc(g[0], g[1], g[2], C, g[3], g[4], o, lse_blk=lse)
        torch.cuda.synchronize()
        assert torch.equal(o, o_ref), "O differs from the workspace call"
        assert torch.equal(lse, l_ref), "LSE differs from the workspace call"
        ro, rl = oracle.denoise_step(q, kc, vc, C, kb, vb, scale_of(d))
        check(o, ro, "bf16", "noalloc O")
        check(lse, rl, "bf16", "noalloc LSE")
