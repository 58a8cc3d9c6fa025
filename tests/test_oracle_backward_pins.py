"""Pins of the oracle's backward (oracle/backward.py) to things other than its own
formulas (CPU only):
  * torch autograd of the forward written with torch ops in fp64 (explicit masks, one
    softmax over both key sources), for both kinds, grouped heads, ragged last blocks;
  * central finite differences of <do, o> through oracle.train_fwd on a tiny case;
  * exact invariants of a softmax gradient: every row's score gradients sum to zero, so
    the key gradients of a kv head sum to zero over all its keys; the value gradients
    of a kv head sum to the upstream gradients of the query heads that read it.
"""
import numpy as np
import pytest
import torch

import oracle
from synth import TensorKind as K, host_tensor, tensor_id


def _rand(shape, seed, kind, dtype="f32"):
    return host_tensor(seed, tensor_id(kind), shape, dtype)


def _torch_forward(q_dec, k_ctx, v_ctx, k_dec, v_dec, S, scale, q_enc):
    """The E2D2 training forward in torch fp64 (explicit masks), for autograd."""
    B, Hq, L, d = q_dec.shape
    Hkv = k_ctx.shape[1]
    g = Hq // Hkv
    mdec = torch.from_numpy(oracle.decoder_mask(L, S))
    menc = torch.from_numpy(oracle.encoder_mask(L, S))
    rep = lambda t: t.repeat_interleave(g, dim=1)
    keys = torch.cat([rep(k_ctx), rep(k_dec)], dim=2)
    vals = torch.cat([rep(v_ctx), rep(v_dec)], dim=2)
    s = (q_dec @ keys.transpose(-1, -2)) * scale
    o_dec = torch.softmax(s.masked_fill(~mdec, float("-inf")), dim=-1) @ vals
    s = (q_enc @ rep(k_ctx).transpose(-1, -2)) * scale
    o_enc = torch.softmax(s.masked_fill(~menc, float("-inf")), dim=-1) @ rep(v_ctx)
    return o_dec, o_enc


@pytest.mark.parametrize("B,Hq,Hkv,L,S,d", [(1, 2, 1, 16, 4, 8), (2, 4, 2, 13, 5, 8),
                                             (1, 2, 2, 12, 1, 4), (1, 1, 1, 10, 10, 6)])
def test_backward_matches_torch_autograd(B, Hq, Hkv, L, S, d):
    seed = 0xB0B0 + L + S
    shapes = [(B, Hq, L, d), (B, Hkv, L, d), (B, Hkv, L, d), (B, Hkv, L, d), (B, Hkv, L, d),
              (B, Hq, L, d)]
    kinds = [K.Q_DEC, K.K_CTX, K.V_CTX, K.K_DEC, K.V_DEC, K.Q_ENC]
    ins = [_rand(sh, seed, kd).double().requires_grad_(True) for sh, kd in zip(shapes, kinds)]
    do_dec = _rand((B, Hq, L, d), seed, K.PROBE).double()
    do_enc = _rand((B, Hq, L, d), seed + 1, K.PROBE).double()
    scale = float(np.float32(1.0 / np.sqrt(d)))
    o_dec, o_enc = _torch_forward(*ins[:5], S, scale, ins[5])
    ((o_dec * do_dec).sum() + (o_enc * do_enc).sum()).backward()
    got = oracle.train_bwd(*[t.detach() for t in ins[:5]], S, scale, do_dec,
                           q_enc=ins[5].detach(), do_enc=do_enc)
    want = [ins[0].grad, ins[1].grad, ins[2].grad, ins[3].grad, ins[4].grad, ins[5].grad]
    for name, a, b in zip(["dq_dec", "dk_ctx", "dv_ctx", "dk_dec", "dv_dec", "dq_enc"], got, want):
        np.testing.assert_allclose(a, b.numpy(), rtol=1e-10, atol=1e-12, err_msg=name)


def test_backward_decoder_only_matches_autograd_without_encoder():
    B, Hq, Hkv, L, S, d = 1, 2, 1, 12, 3, 4
    seed = 0xB1B1
    kinds = [K.Q_DEC, K.K_CTX, K.V_CTX, K.K_DEC, K.V_DEC]
    shapes = [(B, Hq, L, d)] + [(B, Hkv, L, d)] * 4
    ins = [_rand(sh, seed, kd).double().requires_grad_(True) for sh, kd in zip(shapes, kinds)]
    do = _rand((B, Hq, L, d), seed, K.PROBE).double()
    q_dummy = torch.zeros(B, Hq, L, d, dtype=torch.float64)
    o_dec, _ = _torch_forward(*ins, S, 0.5, q_dummy)
    (o_dec * do).sum().backward()
    got = oracle.train_bwd(*[t.detach() for t in ins], S, 0.5, do)
    assert got[5] is None
    for a, t in zip(got[:5], ins):
        np.testing.assert_allclose(a, t.grad.numpy(), rtol=1e-10, atol=1e-12)


def test_backward_matches_finite_differences():
    B, Hq, Hkv, L, S, d = 1, 2, 1, 6, 2, 3
    seed = 0xB2B2
    kinds = [K.Q_DEC, K.K_CTX, K.V_CTX, K.K_DEC, K.V_DEC, K.Q_ENC]
    shapes = [(B, Hq, L, d)] + [(B, Hkv, L, d)] * 4 + [(B, Hq, L, d)]
    ins = [_rand(sh, seed, kd).double().numpy() for sh, kd in zip(shapes, kinds)]
    do_dec = _rand((B, Hq, L, d), seed, K.PROBE).double().numpy()
    do_enc = _rand((B, Hq, L, d), seed + 7, K.PROBE).double().numpy()
    scale = 0.7

    def loss(arrs):
        o_dec, _, o_enc, _ = oracle.train_fwd(*arrs[:5], S, scale, q_enc=arrs[5])
        return float((o_dec * do_dec).sum() + (o_enc * do_enc).sum())

    grads = oracle.train_bwd(*ins[:5], S, scale, do_dec, q_enc=ins[5], do_enc=do_enc)
    order = [0, 1, 2, 3, 4, 5]  # dq_dec, dk_ctx, dv_ctx, dk_dec, dv_dec, dq_enc
    rng = np.random.default_rng(5)
    h = 1e-6
    for which in order:
        for _ in range(6):
            idx = tuple(int(rng.integers(0, n)) for n in ins[which].shape)
            plus = [a.copy() for a in ins]
            minus = [a.copy() for a in ins]
            plus[which][idx] += h
            minus[which][idx] -= h
            fd = (loss(plus) - loss(minus)) / (2 * h)
            assert abs(fd - grads[which][idx]) < 1e-7 * max(1.0, abs(fd)), (which, idx, fd, grads[which][idx])


@pytest.mark.parametrize("L,S", [(32, 8), (33, 5), (16, 16), (9, 1)])
def test_backward_invariants(L, S):
    B, Hq, Hkv, d = 2, 4, 2, 8
    seed = 0xB3B3 + L
    kinds = [K.Q_DEC, K.K_CTX, K.V_CTX, K.K_DEC, K.V_DEC, K.Q_ENC]
    shapes = [(B, Hq, L, d)] + [(B, Hkv, L, d)] * 4 + [(B, Hq, L, d)]
    ins = [_rand(sh, seed, kd).double().numpy() for sh, kd in zip(shapes, kinds)]
    do_dec = _rand((B, Hq, L, d), seed, K.PROBE).double().numpy()
    do_enc = _rand((B, Hq, L, d), seed + 3, K.PROBE).double().numpy()
    dq_dec, dk_ctx, dv_ctx, dk_dec, dv_dec, dq_enc = oracle.train_bwd(
        *ins[:5], S, 0.3, do_dec, q_enc=ins[5], do_enc=do_enc)
    g = Hq // Hkv
    for b in range(B):
        for hk in range(Hkv):
            # sum_j dk_j = scale sum_i q_i sum_j ds_ij = 0 (each row's ds sums to zero)
            tot_k = dk_ctx[b, hk].sum(axis=0) + dk_dec[b, hk].sum(axis=0)
            np.testing.assert_allclose(tot_k, 0.0, atol=1e-11)
            # sum_j dv_j = sum_i do_i (each row's p sums to one), over the group's heads
            want_v = sum(do_dec[b, h].sum(axis=0) + do_enc[b, h].sum(axis=0)
                         for h in range(hk * g, (hk + 1) * g))
            np.testing.assert_allclose(dv_ctx[b, hk].sum(axis=0) + dv_dec[b, hk].sum(axis=0),
                                       want_v, rtol=1e-11, atol=1e-11)
    # a zero upstream gradient gives zero gradients
    z = oracle.train_bwd(*ins[:5], S, 0.3, np.zeros_like(do_dec), q_enc=ins[5],
                         do_enc=np.zeros_like(do_enc))
    for a in z:
        assert np.all(a == 0.0)


def test_backward_kv_head_subsets():
    B, Hq, Hkv, L, S, d = 2, 4, 2, 16, 4, 8
    seed = 0xB4B4
    kinds = [K.Q_DEC, K.K_CTX, K.V_CTX, K.K_DEC, K.V_DEC]
    shapes = [(B, Hq, L, d)] + [(B, Hkv, L, d)] * 4
    ins = [_rand(sh, seed, kd).double().numpy() for sh, kd in zip(shapes, kinds)]
    do = _rand((B, Hq, L, d), seed, K.PROBE).double().numpy()
    full = oracle.train_bwd(*ins, S, 0.25, do)
    part = oracle.train_bwd(*ins, S, 0.25, do, kv_heads=[(1, 0)])
    for a, b_ in zip(full[:5], part[:5]):
        sl = (1, slice(0, 2)) if a.shape[1] == Hq else (1, 0)
        np.testing.assert_array_equal(a[sl], b_[sl])
