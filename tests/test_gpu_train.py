"""GPU parity of the training calls against the fp64 oracle (needs an MI355X).

Every case draws seeded inputs, runs the C-ABI call through the binding, and compares
O and LSE element by element with the oracle on the same inputs: bf16 within 2e-2
absolute, fp32 within 1e-5 * max(1, |ref|).  Tile-visit counters must equal the host
schedule's count and the oracle's brute-force count exactly, and the mask the kernels
apply is read back exactly through one-hot probes.
"""
import math
import sys

import numpy as np
import pytest
import torch

import masked_attention_amd as m
import oracle
from helpers import TORCH_DT, TensorKind as K, check, counter, host, scale_of

pytestmark = pytest.mark.gpu


def say(msg):
    print(msg, file=sys.__stderr__, flush=True)


def _train_case(B, Hq, Hkv, L, S, d, dtype, seed, with_enc=True, heads=None, rows=None,
                inputs=None):
    say(f"[train] B{B} Hq{Hq} Hkv{Hkv} L{L} S{S} d{d} {dtype} seed {seed:#x} enc={with_enc}"
        + (" shaped scores" if inputs is not None else ""))
    if inputs is None:
        qd = host((B, Hq, L, d), seed, K.Q_DEC, dtype)
        qe = host((B, Hq, L, d), seed, K.Q_ENC, dtype)
        kc, vc, kd, vd = (host((B, Hkv, L, d), seed, k, dtype)
                          for k in (K.K_CTX, K.V_CTX, K.K_DEC, K.V_DEC))
    else:
        qd, qe, kc, vc, kd, vd = (inputs[n] for n in ("qd", "qe", "kc", "vc", "kd", "vd"))
    g = {n: t.cuda() for n, t in dict(qd=qd, qe=qe, kc=kc, vc=vc, kd=kd, vd=vd).items()}
    od = torch.full_like(g["qd"], float("nan"))
    oe = torch.full_like(g["qe"], float("nan"))
    ld = torch.full((B, Hq, L), float("nan"), device="cuda")
    le = torch.full((B, Hq, L), float("nan"), device="cuda")
    vis = counter()
    m.e2d2_attn_train_fwd(g["qd"], g["kc"], g["vc"], g["kd"], g["vd"], od, S, lse_dec=ld,
                          q_enc=g["qe"] if with_enc else None, o_enc=oe if with_enc else None,
                          lse_enc=le if with_enc else None, tile_visits=vis)
    torch.cuda.synchronize()
    scale = scale_of(d)
    ro_d, rl_d, ro_e, rl_e = oracle.train_fwd(qd, kc, vc, kd, vd, S, scale,
                                              q_enc=qe if with_enc else None, rows=rows, heads=heads)
    sel = (lambda t: t) if rows is None else (lambda t: t[:, :, rows])
    hs = heads if heads is not None else [(b, h) for b in range(B) for h in range(Hq)]
    for b, h in hs:
        check(sel(od)[b, h], ro_d[b, h], dtype, f"o_dec[{b},{h}]")
        check(sel(ld)[b, h], rl_d[b, h], dtype, f"lse_dec[{b},{h}]")
        if with_enc:
            check(sel(oe)[b, h], ro_e[b, h], dtype, f"o_enc[{b},{h}]")
            check(sel(le)[b, h], rl_e[b, h], dtype, f"lse_enc[{b},{h}]")
    # visits: host schedule == oracle brute force on the explicit masks
    code = m.BF16 if dtype == "bf16" else m.F32
    bm, bn = m.e2d2_attn_tile_shape(m.KIND_DEC, code, d)
    want = m.e2d2_attn_count_tiles(m.KIND_DEC, B, Hq, L, S, 0, bm, bn)[0]
    if with_enc:
        want += m.e2d2_attn_count_tiles(m.KIND_ENC, B, Hq, L, S, 0, bm, bn)[0]
    if L <= 1024:
        brute = oracle.count_tiles(oracle.decoder_mask(L, S), bm, bn, [(0, L), (L, 2 * L)])[0]
        if with_enc:
            brute += oracle.count_tiles(oracle.encoder_mask(L, S), bm, bn, [(0, L)])[0]
        assert want == brute * B * Hq
    assert int(vis.item()) == want
    return dict(od=od, oe=oe, ld=ld, le=le, g=g)


# Tiny check: B1 H2 d32 L64 fp32, blocks of 8, and the degenerate 1 and 64.
@pytest.mark.parametrize("S", [8, 1, 64])
def test_tiny_fp32(S):
    _train_case(1, 2, 2, 64, S, 32, "f32", 0xE2D20001)


@pytest.mark.parametrize("S", [8, 1, 64])
def test_tiny_bf16(S):
    _train_case(1, 2, 2, 64, S, 32, "bf16", 0xE2D20001)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("B,Hq,Hkv,L,S,d", [
    (2, 4, 2, 100, 7, 64),     # ragged last block, ragged last tile, grouped heads
    (1, 3, 3, 257, 16, 128),   # several query tiles + a 1-row tail
    (1, 2, 1, 200, 48, 32),    # blocks straddle 64-key tiles
    (1, 1, 1, 37, 37, 64),     # one block = full attention
    (2, 2, 2, 130, 1, 64),     # block size 1 = causal
    (1, 2, 2, 1, 1, 128),      # a single token
])
def test_ragged_shapes(B, Hq, Hkv, L, S, d, dtype):
    _train_case(B, Hq, Hkv, L, S, d, dtype, 0xE2D2A000 + L)


def test_decoder_only_launch():
    _train_case(2, 4, 2, 160, 16, 64, "bf16", 0xE2D2B001, with_enc=False)


def test_encoder_call_matches_combined_launch_bitwise():
    B, Hq, Hkv, L, S, d = 2, 4, 2, 300, 16, 64
    r = _train_case(B, Hq, Hkv, L, S, d, "bf16", 0xE2D2B002)
    o = torch.empty_like(r["oe"])
    lse = torch.empty_like(r["le"])
    vis = counter()
    m.e2d2_attn_encoder_blockcausal(r["g"]["qe"], r["g"]["kc"], r["g"]["vc"], o, S, lse=lse,
                                    tile_visits=vis)
    torch.cuda.synchronize()
    assert torch.equal(o, r["oe"]) and torch.equal(lse, r["le"])
    bm, bn = m.e2d2_attn_tile_shape(m.KIND_ENC, m.BF16, d)
    assert int(vis.item()) == m.e2d2_attn_count_tiles(m.KIND_ENC, B, Hq, L, S, 0, bm, bn)[0]


def test_training_attention_full_size():
    # B8 H16 d64 L1024 S16 bf16, checked on every row of a spread of heads.
    heads = [(0, 0), (3, 7), (7, 15), (5, 2)]
    _train_case(8, 16, 16, 1024, 16, 64, "bf16", 0xE2D20002, heads=heads)


def test_layer_calls_equal_combined_launch_full_size():
    # The per-layer calls the layer-split benchmark times, at the training workload's size:
    # the encoder-only call and the decoder-only launch are bitwise the combined launch's
    # encoder and decoder outputs on every head (the combined launch is checked against
    # the oracle here on one head and on a spread of heads in the full-size test above).
    B, Hq, Hkv, L, S, d = 8, 16, 16, 1024, 16, 64
    r = _train_case(B, Hq, Hkv, L, S, d, "bf16", 0xE2D20002, heads=[(5, 11)])
    g = r["g"]
    oe, od = torch.empty_like(r["oe"]), torch.empty_like(r["od"])
    le, ld = torch.empty_like(r["le"]), torch.empty_like(r["ld"])
    m.e2d2_attn_encoder_blockcausal(g["qe"], g["kc"], g["vc"], oe, S, lse=le)
    m.e2d2_attn_train_fwd(g["qd"], g["kc"], g["vc"], g["kd"], g["vd"], od, S, lse_dec=ld)
    torch.cuda.synchronize()
    assert torch.equal(oe, r["oe"]) and torch.equal(le, r["le"])
    assert torch.equal(od, r["od"]) and torch.equal(ld, r["ld"])


def test_long_sequence_full_size_sampled_rows():
    # B2 Hq16 Hkv8 d128 L8192 S64 bf16: sampled rows of sampled heads.
    rows = np.unique(np.concatenate([np.arange(0, 70), np.arange(8100, 8192),
                                     np.random.default_rng(4).integers(0, 8192, 160)]))
    _train_case(2, 16, 8, 8192, 64, 128, "bf16", 0xE2D20004, heads=[(0, 0), (1, 9), (1, 15)],
                rows=rows)


def test_deterministic_and_future_independent():
    B, Hq, Hkv, L, S, d = 1, 2, 2, 256, 16, 64
    r1 = _train_case(B, Hq, Hkv, L, S, d, "bf16", 0xE2D2B003)
    g = r1["g"]
    od = torch.empty_like(r1["od"]); ld = torch.empty_like(r1["ld"])
    oe = torch.empty_like(r1["oe"]); le = torch.empty_like(r1["le"])
    m.e2d2_attn_train_fwd(g["qd"], g["kc"], g["vc"], g["kd"], g["vd"], od, S, lse_dec=ld,
                          q_enc=g["qe"], o_enc=oe, lse_enc=le)
    torch.cuda.synchronize()
    for a, b in ((od, r1["od"]), (ld, r1["ld"]), (oe, r1["oe"]), (le, r1["le"])):
        assert torch.equal(a, b)
    # Perturb K/V of blocks >= 5: rows of blocks 0..4 must not change at all.
    cut = 5 * S
    p = {k: v.clone() for k, v in g.items()}
    for k in ("kc", "vc", "kd", "vd"):
        p[k][:, :, cut:] += 3.0
    m.e2d2_attn_train_fwd(p["qd"], p["kc"], p["vc"], p["kd"], p["vd"], od, S, lse_dec=ld,
                          q_enc=p["qe"], o_enc=oe, lse_enc=le)
    torch.cuda.synchronize()
    for a, b in ((od, r1["od"]), (ld, r1["ld"]), (oe, r1["oe"]), (le, r1["le"])):
        assert torch.equal(a[:, :, :cut], b[:, :, :cut])
        assert not torch.equal(a[:, :, cut:], b[:, :, cut:])


def _probe_masks(L, S, d, dtype):
    """Read the applied masks back exactly: with q = 0 every allowed key gets weight
    1/count, so exp(LSE) is the allowed count and, with one-hot values on a chunk of d
    keys, O[i][c] != 0 exactly when key (chunk*d + c) is allowed for row i."""
    B, H = 1, 1
    dt = TORCH_DT[dtype]
    z = torch.zeros((B, H, L, d), dtype=dt, device="cuda")
    kk = host((B, H, L, d), 0xE2D2C000, K.K_CTX, dtype).cuda()
    enc = np.zeros((L, L), bool)
    dec = np.zeros((L, 2 * L), bool)
    o = torch.empty_like(z); o2 = torch.empty_like(z)
    lse = torch.empty((B, H, L), device="cuda"); lse2 = torch.empty_like(lse)
    for src in range(2):
        for p0 in range(0, L, d):
            onehot = torch.zeros((B, H, L, d), dtype=dt, device="cuda")
            n = min(d, L - p0)
            onehot[0, 0, p0:p0 + n, :n] = torch.eye(n, dtype=dt, device="cuda")
            zero = torch.zeros_like(onehot)
            vc, vd = (onehot, zero) if src == 0 else (zero, onehot)
            m.e2d2_attn_train_fwd(z, kk, vc, kk, vd, o, S, lse_dec=lse, q_enc=z, o_enc=o2,
                                  lse_enc=lse2)
            torch.cuda.synchronize()
            dec[:, src * L + p0:src * L + p0 + n] = (o[0, 0, :, :n] != 0).cpu().numpy()
            if src == 0:
                enc[:, p0:p0 + n] = (o2[0, 0, :, :n] != 0).cpu().numpy()
    cnt_enc = np.rint(np.exp(lse2[0, 0].double().cpu().numpy())).astype(int)
    cnt_dec = np.rint(np.exp(lse[0, 0].double().cpu().numpy())).astype(int)
    return enc, dec, cnt_enc, cnt_dec


@pytest.mark.parametrize("L,S,d,dtype", [(64, 8, 32, "bf16"), (64, 8, 32, "f32"),
                                         (100, 7, 64, "bf16"), (150, 64, 128, "bf16")])
def test_mask_structure_is_exact(L, S, d, dtype):
    say(f"[mask probe] L{L} S{S} d{d} {dtype}")
    enc, dec, ce, cd = _probe_masks(L, S, d, dtype)
    assert np.array_equal(enc, oracle.encoder_mask(L, S))
    assert np.array_equal(dec, oracle.decoder_mask(L, S))
    assert np.array_equal(ce, oracle.encoder_mask(L, S).sum(1))
    assert np.array_equal(cd, oracle.decoder_mask(L, S).sum(1))


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_bd3lm_single_stack_layer_via_fused_call(dtype):
    # A decoder-only block-diffusion layer over 2L tokens [noised | clean] (the FLOPs
    # table's BD3LM row) is one fused call on its halves: noised queries as the decoder
    # (clean keys as context, own-block noised keys), clean queries as the encoder.
    # Checked against the oracle's explicit 2L x 2L mask.
    B, Hq, Hkv, L, S, d = 2, 4, 2, 96, 16, 64
    seed = 0xE2D2BD30
    say(f"[bd3lm] B{B} Hq{Hq}/{Hkv} 2L={2 * L} S{S} d{d} {dtype}")
    q = host((B, Hq, 2 * L, d), seed, K.Q_DEC, dtype)
    k = host((B, Hkv, 2 * L, d), seed, K.K_CTX, dtype)
    v = host((B, Hkv, 2 * L, d), seed, K.V_CTX, dtype)
    half = lambda t, i: t[:, :, i * L:(i + 1) * L].contiguous().cuda()
    od = torch.empty((B, Hq, L, d), dtype=TORCH_DT[dtype], device="cuda")
    oe = torch.empty_like(od)
    ld = torch.empty((B, Hq, L), device="cuda")
    le = torch.empty_like(ld)
    m.e2d2_attn_train_fwd(half(q, 0), half(k, 1), half(v, 1), half(k, 0), half(v, 0), od, S,
                          lse_dec=ld, q_enc=half(q, 1), o_enc=oe, lse_enc=le)
    torch.cuda.synchronize()
    ro, rl = oracle.bd3lm_layer(q, k, v, S, scale_of(d))
    for b in range(B):
        for h in range(Hq):
            check(od[b, h], ro[b, h, :L], dtype, f"noised o[{b},{h}]")
            check(oe[b, h], ro[b, h, L:], dtype, f"clean o[{b},{h}]")
            check(ld[b, h], rl[b, h, :L], dtype, f"noised lse[{b},{h}]")
            check(le[b, h], rl[b, h, L:], dtype, f"clean lse[{b},{h}]")


def _shaped_scores(B, Hq, Hkv, L, d, dtype, seed, span=0.0, amp=1.0):
    """Seeded inputs with large or growing scores.  Every query row is 16 u plus small
    noise, u a unit direction per KV head; clean key j is span * sqrt(d) / 16 * (j / L) u
    plus N(0, 1) noise, noised key j the same with (1 - j / L): scaled scores climb by
    about span nats along the clean keys (the running max rises in most tiles) and fall
    along the noised ones.  With span = 0, queries and keys are amp * N(0, 1) instead
    (score spread amp^2 nats).  Values are N(0, 1)."""
    g = lambda shape, kind, step=0: host(shape, seed, kind, "f32", step=step).double()
    dt = TORCH_DT[dtype]
    if span == 0.0:
        qd, qe = amp * g((B, Hq, L, d), K.Q_DEC), amp * g((B, Hq, L, d), K.Q_ENC)
        kc, kd = amp * g((B, Hkv, L, d), K.K_CTX), amp * g((B, Hkv, L, d), K.K_DEC)
    else:
        u = g((B, Hkv, 1, d), K.K_CTX, step=1)
        u = u / u.norm(dim=-1, keepdim=True)
        uq = u.repeat_interleave(Hq // Hkv, dim=1)
        bk = span * math.sqrt(d) / 16.0
        j = torch.arange(L, dtype=torch.float64).view(1, 1, L, 1) / L
        qd = 16.0 * uq + 0.1 * g((B, Hq, L, d), K.Q_DEC)
        qe = 16.0 * uq + 0.1 * g((B, Hq, L, d), K.Q_ENC)
        kc = bk * j * u + g((B, Hkv, L, d), K.K_CTX)
        kd = bk * (1.0 - j) * u + g((B, Hkv, L, d), K.K_DEC)
    vc, vd = g((B, Hkv, L, d), K.V_CTX), g((B, Hkv, L, d), K.V_DEC)
    return {n: t.to(dt) for n, t in dict(qd=qd, qe=qe, kc=kc, vc=vc, kd=kd, vd=vd).items()}


# The online softmax's rescaling under scores far from N(0, 1): a running max that rises
# in most tiles (span 200 nats in bf16; 8 in fp32, which rescales every tile and where
# the scores' own fp32 rounding stays inside the 1e-5 bound) and large random scores
# (spread 16 nats in bf16, 2.25 in fp32).
@pytest.mark.parametrize("dtype,d,span,amp", [
    ("bf16", 64, 200.0, 1.0), ("bf16", 128, 200.0, 1.0), ("bf16", 64, 0.0, 4.0),
    ("f32", 64, 8.0, 1.0), ("f32", 32, 0.0, 1.5),
])
def test_rescaling_under_large_and_growing_scores(dtype, d, span, amp):
    B, Hq, Hkv, L, S = 1, 4, 2, 512, 16
    inputs = _shaped_scores(B, Hq, Hkv, L, d, dtype, 0xE2D20C01, span=span, amp=amp)
    _train_case(B, Hq, Hkv, L, S, d, dtype, 0xE2D20C01, inputs=inputs)
