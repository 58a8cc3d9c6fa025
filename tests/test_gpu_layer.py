"""GPU parity of the decoder-layer denoise step (e2d2_decoder_layer_denoise_step)
against the fp64 oracle (oracle.decoder_layer_denoise, which stores q, k, v and o in
bf16 as the layer does).

Tolerances, element-wise:
  * q, k, v: one bf16 spacing of the reference's binade (2^(e-8) for |ref| in
    [2^(e-1), 2^e)), floor 2^-20.  Both sides round the same projection to bf16; the
    GPU's fp32 sum sits within a tiny fraction of a spacing of the exact one, so they
    differ by at most one step where the exact value is near a rounding midpoint.
  * o, lse: the attention's bf16 bar, |d| <= 2e-2.
  * y: |d| <= 2e-2 * max(|y_ref|, rms of y_ref's row over the model width), element by
    element.  y is a sum over the heads' o (bf16, ~2^-8 relative from bf16 P and O)
    times bf16 weights, accumulated in fp32, plus y's own bf16 rounding (2^-9): its
    error follows the size of its terms, with the row's RMS as the floor for elements
    the sum cancels to near zero.
"""
import math
import sys

import numpy as np
import pytest
import torch

import masked_attention_amd as m
import oracle
from helpers import TensorKind as K, check, check_scaled, gpu_fill, host, scale_of
from synth import device_draw, host_draw, tensor_id

pytestmark = pytest.mark.gpu


def say(msg):
    print(msg, file=sys.__stderr__, flush=True)


def _wscale(k):
    """Power of two near 1/sqrt(k): scales N(0, 1) weights without changing their bf16 bits."""
    return 2.0 ** -round(math.log2(math.sqrt(k)))


def _host_inputs(B, S, Dm, Hq, Hkv, d, seed):
    x = host_draw(seed, tensor_id(K.X_BLK), (B, S, Dm), "bf16")
    w_qkv = host_draw(seed, tensor_id(K.W_QKV), ((Hq + 2 * Hkv) * d, Dm), "bf16") * _wscale(Dm)
    w_o = host_draw(seed, tensor_id(K.W_O), (Dm, Hq * d), "bf16") * _wscale(Hq * d)
    return x, w_qkv, w_o


def _run(x, w_qkv, w_o, kc, vc, C, Hq, Hkv, d):
    B, S, Dm = x.shape
    q = torch.full((B, Hq, S, d), float("nan"), dtype=torch.bfloat16, device="cuda")
    o = torch.full_like(q, float("nan"))
    k = torch.full((B, Hkv, S, d), float("nan"), dtype=torch.bfloat16, device="cuda")
    v = torch.full_like(k, float("nan"))
    y = torch.full_like(x, float("nan"))
    lse = torch.full((B, Hq, S), float("nan"), device="cuda")
    n = m.e2d2_attn_denoise_workspace_bytes(m.BF16, B, Hq, Hkv, S, d, C)
    ws = torch.empty(n, dtype=torch.uint8, device="cuda") if n else None
    m.e2d2_decoder_layer_denoise_step(x, w_qkv, w_o, kc, vc, C, q, k, v, o, y, lse_blk=lse,
                                      workspace=ws)
    torch.cuda.synchronize()
    return q, k, v, o, lse, y


def check_bf16_step(got, ref, what):
    g = got.detach().double().cpu().numpy()
    r = np.asarray(ref, dtype=np.float64)
    assert g.shape == r.shape, (what, g.shape, r.shape)
    _, ex = np.frexp(r)
    tol = np.maximum(np.ldexp(1.0, ex - 8), 2.0 ** -20)
    bad = ~(np.abs(g - r) <= tol)
    if bad.any():
        idx = np.unravel_index(np.argmax(bad), bad.shape)
        raise AssertionError(f"{what}: {int(bad.sum())} elements beyond one bf16 step; first at "
                             f"{idx} (got {g[idx]}, ref {r[idx]})")


def check_rel(got, ref, what, rel=2e-2):
    check_scaled(got, ref, what, rel)


@pytest.mark.parametrize("B,S,Dm,Hq,Hkv,d,C", [
    (2, 7, 96, 4, 2, 32, 50),      # ragged: 14 tokens, k axis of 96 (a partial stage)
    (3, 32, 256, 4, 2, 64, 300),   # several k stages, grouped heads
    (2, 16, 512, 4, 4, 128, 0),    # empty cache: the own block only
    (1, 1, 64, 2, 1, 64, 33),      # one token
    (4, 32, 1024, 8, 4, 128, 700), # 16 k stages, a 128-row token tile, two heads per kv head
])
def test_layer_matches_oracle(B, S, Dm, Hq, Hkv, d, C):
    seed = 0xE2D2C300 + Dm + C
    say(f"[layer] B{B} S{S} Dm{Dm} Hq{Hq} Hkv{Hkv} d{d} C{C}")
    x, w_qkv, w_o = _host_inputs(B, S, Dm, Hq, Hkv, d, seed)
    cap = C + 8
    kc = host((B, Hkv, cap, d), seed, K.K_CACHE, "bf16")
    vc = host((B, Hkv, cap, d), seed, K.V_CACHE, "bf16")
    got = _run(x.cuda(), w_qkv.cuda(), w_o.cuda(), kc.cuda(), vc.cuda(), C, Hq, Hkv, d)
    ref = oracle.decoder_layer_denoise(x, w_qkv, w_o, kc, vc, C, Hq, Hkv, d, scale_of(d))
    for name, g, r in zip("qkv", got[:3], ref[:3]):
        check_bf16_step(g, r, name)
    check(got[3], ref[3], "bf16", "o")
    check(got[4], ref[4], "bf16", "lse")
    check_rel(got[5], ref[5], "y")


def test_layer_uniform_attention_pins_output_projection():
    # Zero query weights: every score is 0 and o is the mean of the value rows the block
    # sees, computed with exact p = 1; y then checks the output projection closely.
    B, S, Dm, Hq, Hkv, d, C = 2, 32, 512, 4, 2, 128, 96
    seed = 0xE2D2C400
    x, w_qkv, w_o = _host_inputs(B, S, Dm, Hq, Hkv, d, seed)
    w_qkv[:Hq * d] = 0
    kc = host((B, Hkv, C, d), seed, K.K_CACHE, "bf16")
    vc = host((B, Hkv, C, d), seed, K.V_CACHE, "bf16")
    got = _run(x.cuda(), w_qkv.cuda(), w_o.cuda(), kc.cuda(), vc.cuda(), C, Hq, Hkv, d)
    ref = oracle.decoder_layer_denoise(x, w_qkv, w_o, kc, vc, C, Hq, Hkv, d, scale_of(d))
    check(got[3], ref[3], "bf16", "o")
    check_rel(got[5], ref[5], "y", rel=2.0 ** -6)


def test_layer_denoise_workload_sampled():
    # B32 Hq16/Hkv8 d128 S32, cache length 2048, model width 2048 (Hq d): q, k, v in
    # full; o, lse and y of three sequences.
    B, S, Hq, Hkv, d, C = 32, 32, 16, 8, 128, 2048
    Dm = Hq * d
    seed = 0xE2D2C500
    say(f"[layer] full B{B} S{S} Dm{Dm} Hq{Hq}/{Hkv} d{d} C{C}")
    x, w_qkv, w_o = _host_inputs(B, S, Dm, Hq, Hkv, d, seed)
    cap = C + S
    kc = gpu_fill((B, Hkv, cap, d), seed, K.K_CACHE, "bf16")
    vc = gpu_fill((B, Hkv, cap, d), seed, K.V_CACHE, "bf16")
    got = _run(x.cuda(), w_qkv.cuda(), w_o.cuda(), kc, vc, C, Hq, Hkv, d)
    # q, k, v of every token: the projection alone (fp64, rounded to bf16 as stored)
    qkv = x.double().numpy() @ w_qkv.double().numpy().T
    for name, lo, H in (("q", 0, Hq), ("k", Hq * d, Hkv), ("v", (Hq + Hkv) * d, Hkv)):
        ref = oracle.round_bf16(qkv[:, :, lo:lo + H * d].reshape(B, S, H, d).transpose(0, 2, 1, 3))
        check_bf16_step(got["qkv".index(name)], ref, name)
    for b in (0, 17, 31):
        kcb = host((1, Hkv, C, d), seed, K.K_CACHE, "bf16", b0=b)
        vcb = host((1, Hkv, C, d), seed, K.V_CACHE, "bf16", b0=b)
        ref = oracle.decoder_layer_denoise(x[b:b + 1], w_qkv, w_o, kcb, vcb, C, Hq, Hkv, d,
                                           scale_of(d))
        check(got[3][b:b + 1], ref[3], "bf16", f"o[{b}]")
        check(got[4][b:b + 1], ref[4], "bf16", f"lse[{b}]")
        check_rel(got[5][b:b + 1], ref[5], f"y[{b}]")


def test_layer_is_deterministic_and_matches_device_inputs():
    # device-drawn inputs equal the host draw, and two calls agree bitwise
    B, S, Dm, Hq, Hkv, d, C = 2, 32, 256, 4, 2, 64, 200
    seed = 0xE2D2C600
    x = torch.empty((B, S, Dm), dtype=torch.bfloat16, device="cuda")
    device_draw(x, seed, tensor_id(K.X_BLK))
    xh, _, _ = _host_inputs(B, S, Dm, Hq, Hkv, d, seed)
    assert torch.equal(x.cpu(), xh)
    _, w_qkv, w_o = (t.cuda() for t in _host_inputs(B, S, Dm, Hq, Hkv, d, seed))
    kc = gpu_fill((B, Hkv, C, d), seed, K.K_CACHE, "bf16")
    vc = gpu_fill((B, Hkv, C, d), seed, K.V_CACHE, "bf16")
    a = _run(x, w_qkv, w_o, kc, vc, C, Hq, Hkv, d)
    b = _run(x, w_qkv, w_o, kc, vc, C, Hq, Hkv, d)
    for name, u, w in zip(["q", "k", "v", "o", "lse", "y"], a, b):
        assert torch.equal(u, w), name


def test_layer_graph_replays_follow_new_hidden_states():
    # One captured layer step replayed while the hidden states change on the device (a
    # denoising loop feeds each step's tokens back in): every replay equals an eager call.
    B, S, Dm, Hq, Hkv, d, C = 2, 16, 256, 4, 2, 64, 150
    seed = 0xE2D2C700
    xh, w_qkv, w_o = _host_inputs(B, S, Dm, Hq, Hkv, d, seed)
    x, w_qkv, w_o = xh.cuda(), w_qkv.cuda(), w_o.cuda()
    kc = gpu_fill((B, Hkv, C, d), seed, K.K_CACHE, "bf16")
    vc = gpu_fill((B, Hkv, C, d), seed, K.V_CACHE, "bf16")
    q = torch.empty((B, Hq, S, d), dtype=torch.bfloat16, device="cuda")
    o = torch.empty_like(q)
    k = torch.empty((B, Hkv, S, d), dtype=torch.bfloat16, device="cuda")
    v = torch.empty_like(k)
    y = torch.empty_like(x)
    n = m.e2d2_attn_denoise_workspace_bytes(m.BF16, B, Hq, Hkv, S, d, C)
    ws = torch.empty(n, dtype=torch.uint8, device="cuda") if n else None

    def step(out):
        m.e2d2_decoder_layer_denoise_step(x, w_qkv, w_o, kc, vc, C, q, k, v, o, out, workspace=ws)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step(y)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step(y)
    ref = torch.empty_like(y)
    for it in range(3):
        x.mul_(-0.5).add_(0.25)  # eager update between replays
        graph.replay()
        torch.cuda.synchronize()
        got = y.clone()
        step(ref)
        torch.cuda.synchronize()
        assert torch.equal(got, ref), f"replay {it}"
    xf = x.cpu()
    want = oracle.decoder_layer_denoise(xf, w_qkv.cpu(), w_o.cpu(), kc.cpu(), vc.cpu(), C, Hq, Hkv,
                                        d, scale_of(d))
    check_rel(y, want[5], "y after replays")
