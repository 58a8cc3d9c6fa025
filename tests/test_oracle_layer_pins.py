"""Pins of the decoder-layer oracle (oracle/layer.py) to things other than its own
formulas (CPU only):
  * round_bf16 against hand-worked ties and torch's float32 -> bfloat16 conversion;
  * the whole sublayer against scalar loops written index by index (projections,
    per-head slices, grouped heads, softmax over cache plus own block, concatenation
    and output projection) on tiny shapes;
  * the closed form of uniform attention (W_q = 0): o is the plain mean of the value
    rows the block sees, so y = mean(v) W_o^T;
  * bf16 storage: q, k, v, o come out bf16-representable and within half a bf16 ulp
    of the unrounded layer's values (q, k, v).
"""
import math

import numpy as np
import pytest
import torch

import oracle
from synth import TensorKind as K, host_draw, host_tensor, tensor_id


def _rand(shape, seed, kind, scale=1.0):
    return host_draw(seed, tensor_id(kind), shape, "f32").double().numpy() * scale


def _inputs(B, S, Dm, Hq, Hkv, d, cap, seed):
    x = _rand((B, S, Dm), seed, K.X_BLK)
    w_qkv = _rand(((Hq + 2 * Hkv) * d, Dm), seed, K.W_QKV, Dm ** -0.5)
    w_o = _rand((Dm, Hq * d), seed, K.W_O, (Hq * d) ** -0.5)
    kc = _rand((B, Hkv, cap, d), seed, K.K_CACHE)
    vc = _rand((B, Hkv, cap, d), seed, K.V_CACHE)
    return x, w_qkv, w_o, kc, vc


def test_round_bf16_ties_and_torch():
    # bf16 keeps 8 significant bits: the spacing above 1 is 2^-7.
    cases = {1.0 + 2.0 ** -8: 1.0,                      # tie, rounds to the even 1.0
             1.0 + 3 * 2.0 ** -8: 1.0 + 2.0 ** -6,      # tie, rounds to the even neighbour
             1.0 + 2.0 ** -8 + 2.0 ** -30: 1.0 + 2.0 ** -7,
             -(3.0 + 2.0 ** -7): -3.0,                  # spacing 2^-6 at 3: tie to even
             0.0: 0.0, 2.0 ** -100: 2.0 ** -100}
    for x, want in cases.items():
        assert oracle.round_bf16(np.array([x]))[0] == want, x
    # float32 inputs: torch's conversion is single rounding too
    v = host_tensor(5, 99, (1, 1, 64, 64), "f32").reshape(-1)
    want = v.to(torch.bfloat16).double().numpy()
    np.testing.assert_array_equal(oracle.round_bf16(v.double().numpy()), want)


def _brute(x, w_qkv, w_o, kc, vc, C, Hq, Hkv, d, scale):
    """The sublayer with scalar loops (no bf16 storage)."""
    B, S, Dm = x.shape
    g = Hq // Hkv
    sc = float(np.float32(scale))

    def proj(b, s, row):
        return sum(x[b, s, i] * w_qkv[row, i] for i in range(Dm))

    q = [[[[proj(b, s, h * d + c) for c in range(d)] for s in range(S)] for h in range(Hq)]
         for b in range(B)]
    k = [[[[proj(b, s, Hq * d + h * d + c) for c in range(d)] for s in range(S)]
          for h in range(Hkv)] for b in range(B)]
    v = [[[[proj(b, s, (Hq + Hkv) * d + h * d + c) for c in range(d)] for s in range(S)]
          for h in range(Hkv)] for b in range(B)]
    o = np.zeros((B, Hq, S, d))
    lse = np.zeros((B, Hq, S))
    for b in range(B):
        for h in range(Hq):
            hk = h // g
            keys = [list(kc[b, hk, j]) for j in range(C)] + [k[b][hk][t] for t in range(S)]
            vals = [list(vc[b, hk, j]) for j in range(C)] + [v[b][hk][t] for t in range(S)]
            for s in range(S):
                scores = [sc * sum(q[b][h][s][c] * key[c] for c in range(d)) for key in keys]
                m = max(scores)
                p = [math.exp(z - m) for z in scores]
                l = sum(p)
                for c in range(d):
                    o[b, h, s, c] = sum(pj * val[c] for pj, val in zip(p, vals)) / l
                lse[b, h, s] = m + math.log(l)
    y = np.zeros((B, S, Dm))
    for b in range(B):
        for s in range(S):
            for n in range(Dm):
                y[b, s, n] = sum(o[b, h, s, c] * w_o[n, h * d + c] for h in range(Hq)
                                 for c in range(d))
    return np.array(q), np.array(k), np.array(v), o, lse, y


@pytest.mark.parametrize("B,S,Dm,Hq,Hkv,d,C", [(2, 3, 5, 4, 2, 2, 4),   # grouped heads
                                                (1, 2, 3, 2, 2, 3, 0),   # empty cache
                                                (1, 4, 4, 3, 1, 2, 5)])  # three heads per kv head
def test_layer_matches_scalar_loops(B, S, Dm, Hq, Hkv, d, C):
    x, w_qkv, w_o, kc, vc = _inputs(B, S, Dm, Hq, Hkv, d, C + 2, 0xE2D2C000 + Dm)
    scale = d ** -0.5
    got = oracle.decoder_layer_denoise(x, w_qkv, w_o, kc, vc, C, Hq, Hkv, d, scale,
                                       store_bf16=False)
    ref = _brute(x, w_qkv, w_o, kc, vc, C, Hq, Hkv, d, scale)
    for name, a, r in zip(["q", "k", "v", "o", "lse", "y"], got, ref):
        np.testing.assert_allclose(a, r, rtol=1e-12, atol=1e-12, err_msg=name)


def test_uniform_attention_closed_form():
    # W_q = 0: every score is 0, so o is the plain mean of the C cached and S own value
    # rows of the query's kv head.
    B, S, Dm, Hq, Hkv, d, C = 2, 5, 24, 4, 2, 8, 7
    x, w_qkv, w_o, kc, vc = _inputs(B, S, Dm, Hq, Hkv, d, C + 3, 0xE2D2C100)
    w_qkv[:Hq * d] = 0.0
    _, _, v, o, lse, y = oracle.decoder_layer_denoise(x, w_qkv, w_o, kc, vc, C, Hq, Hkv, d,
                                                      0.125, store_bf16=False)
    g = Hq // Hkv
    v_rows = x @ w_qkv[(Hq + Hkv) * d:].T  # [B, S, Hkv d]
    for b in range(B):
        for h in range(Hq):
            hk = h // g
            allv = np.concatenate([vc[b, hk, :C], v_rows[b, :, hk * d:(hk + 1) * d]], axis=0)
            mean = allv.mean(axis=0)
            np.testing.assert_allclose(o[b, h], np.broadcast_to(mean, (S, d)), rtol=1e-12,
                                       atol=1e-13)
            np.testing.assert_allclose(lse[b, h], math.log(C + S), rtol=1e-13)
    o_cat = np.concatenate([o[:, h] for h in range(Hq)], axis=-1)  # [B, S, Hq d]
    np.testing.assert_allclose(y, np.einsum("bsk,nk->bsn", o_cat, w_o), rtol=1e-11, atol=1e-13)


def test_bf16_storage():
    B, S, Dm, Hq, Hkv, d, C = 1, 6, 40, 4, 2, 16, 9
    args = _inputs(B, S, Dm, Hq, Hkv, d, C, 0xE2D2C200)
    exact = oracle.decoder_layer_denoise(*args, C, Hq, Hkv, d, 0.25, store_bf16=False)
    stored = oracle.decoder_layer_denoise(*args, C, Hq, Hkv, d, 0.25)
    for name, a, e in zip(["q", "k", "v"], stored[:3], exact[:3]):
        np.testing.assert_array_equal(oracle.round_bf16(a), a, err_msg=name)
        # half an ulp: for |e| in [2^(x-1), 2^x) the bf16 spacing is 2^(x-8)
        _, ex = np.frexp(e)
        assert (np.abs(a - e) <= np.ldexp(1.0, ex - 9)).all(), name
    np.testing.assert_array_equal(oracle.round_bf16(stored[3]), stored[3])
