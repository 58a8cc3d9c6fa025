"""The differentiable op (masked_attention_amd.e2d2_attention): torch autograd through
the library's forward and backward kernels, against the fp64 oracle's gradients
(oracle.train_bwd).  Tolerance as in test_gpu_bwd.py: |got - ref| <= 2e-2 *
max(1, max |ref|) per gradient tensor."""
import sys

import numpy as np
import pytest
import torch

import masked_attention_amd as m
import oracle
from helpers import TensorKind as K, check, host, scale_of

pytestmark = pytest.mark.gpu


def _close(got, ref, what):
    g = got.detach().double().cpu().numpy()
    r = np.asarray(ref, dtype=np.float64)
    tol = 2e-2 * max(1.0, float(np.abs(r).max()))
    err = np.abs(g - r).max()
    assert np.isfinite(g).all() and err <= tol, f"{what}: max err {err:.3e} > {tol:.3g}"


@pytest.mark.parametrize("with_enc", [True, False])
def test_autograd_gradients_match_oracle(with_enc):
    B, Hq, Hkv, L, S, d = 1, 4, 2, 100, 7, 64
    seed = 0xE2D2B400
    print(f"[autograd] B{B} Hq{Hq}/{Hkv} L{L} S{S} d{d} enc={with_enc}", file=sys.__stderr__, flush=True)
    q = (B, Hq, L, d)
    kv = (B, Hkv, L, d)
    hq_dec, hq_enc = host(q, seed, K.Q_DEC, "bf16"), host(q, seed, K.Q_ENC, "bf16")
    hk = [host(kv, seed, kind, "bf16") for kind in (K.K_CTX, K.V_CTX, K.K_DEC, K.V_DEC)]
    hdo_dec, hdo_enc = host(q, seed, K.DO_DEC, "bf16"), host(q, seed, K.DO_ENC, "bf16")
    leaves = [t.cuda().requires_grad_() for t in [hq_dec] + hk + ([hq_enc] if with_enc else [])]
    q_dec, k_ctx, v_ctx, k_dec, v_dec = leaves[:5]
    q_enc = leaves[5] if with_enc else None
    out = m.e2d2_attention(q_dec, k_ctx, v_ctx, k_dec, v_dec, S, q_enc=q_enc)
    o_dec, o_enc = out if with_enc else (out, None)
    # a loss whose gradient with respect to o_dec (o_enc) is do_dec (do_enc)
    loss = (o_dec.float() * hdo_dec.cuda().float()).sum()
    if with_enc:
        loss = loss + (o_enc.float() * hdo_enc.cuda().float()).sum()
    loss.backward()
    ref_o = oracle.train_fwd(hq_dec, *hk, S, scale_of(d), q_enc=hq_enc if with_enc else None)
    check(o_dec, ref_o[0], "bf16", "o_dec")
    ref = oracle.train_bwd(hq_dec, *hk, S, scale_of(d), hdo_dec, q_enc=hq_enc if with_enc else None,
                           do_enc=hdo_enc if with_enc else None)
    names = ["dq_dec", "dk_ctx", "dv_ctx", "dk_dec", "dv_dec", "dq_enc"]
    for name, leaf, r in zip(names, leaves, ref):
        _close(leaf.grad, r, name)


def test_autograd_takes_strided_upstream_gradients():
    # an upstream gradient that is a transposed view reaches the kernels contiguous
    B, Hq, L, S, d = 1, 2, 64, 8, 32
    q = host((B, Hq, L, d), 0xE2D2B500, K.Q_DEC, "bf16").cuda().requires_grad_()
    k = [host((B, Hq, L, d), 0xE2D2B500, kind, "bf16").cuda().requires_grad_()
         for kind in (K.K_CTX, K.V_CTX, K.K_DEC, K.V_DEC)]
    o = m.e2d2_attention(q, *k, S)
    torch.manual_seed(0)
    g = torch.randn(B, Hq, d, L, device="cuda").to(torch.bfloat16).transpose(2, 3)
    o.backward(g)
    q2 = q.detach().clone().requires_grad_()
    k2 = [t.detach().clone().requires_grad_() for t in k]
    m.e2d2_attention(q2, *k2, S).backward(g.contiguous())
    assert torch.equal(q.grad, q2.grad)
    for a, b in zip(k, k2):
        assert torch.equal(a.grad, b.grad)
