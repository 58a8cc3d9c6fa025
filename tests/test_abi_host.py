"""C-ABI library checks that need no GPU: it loads, exports every symbol the header
declares, answers the host-only queries, and rejects bad arguments with the documented
status before anything touches the GPU.  The host tile schedule's counts are checked
bit-exactly against the oracle's brute force over the explicit masks."""
import ctypes
import os
import re

import pytest

import masked_attention_amd as m
import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "e2d2_attn.h")

OK, ERR_NULL, ERR_SHAPE, ERR_UNSUPPORTED, ERR_CAPACITY, ERR_WORKSPACE = 0, 1, 2, 3, 4, 5


def _declared_functions():
    text = open(HEADER, encoding="utf-8").read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(e2d2_[a-z0-9_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    names = _declared_functions()
    assert len(names) >= 10
    h = ctypes.CDLL(m.library_path)
    for n in names:
        assert hasattr(h, n), n
    assert set(names) == set(m._SIGS), "binding and header disagree"


def test_abi_version_and_status_strings():
    assert m.abi_version() == 1
    for s in range(7):
        assert m.lib().e2d2_status_string(s)
    assert m.lib().e2d2_status_string(99) == b"unknown status"
    assert m.lib().e2d2_last_hip_error() == 0


def test_tile_shapes():
    assert m.e2d2_attn_tile_shape(m.KIND_ENC, m.BF16, 64) == (128, 64)
    assert m.e2d2_attn_tile_shape(m.KIND_DEC, m.BF16, 128) == (128, 64)
    assert m.e2d2_attn_tile_shape(m.KIND_DENOISE, m.BF16, 128) == (32, 32)
    assert m.e2d2_attn_tile_shape(m.KIND_ENC, m.F32, 32) == (64, 64)
    with pytest.raises(m.E2D2Error):
        m.e2d2_attn_tile_shape(m.KIND_ENC, m.BF16, 48)
    with pytest.raises(m.E2D2Error):
        m.e2d2_attn_tile_shape(7, m.BF16, 64)


CASES = [(64, 8), (64, 1), (64, 64), (100, 7), (33, 5), (257, 16), (130, 128), (1024, 16),
         (1, 1), (5, 9)]


@pytest.mark.parametrize("L,S", CASES)
@pytest.mark.parametrize("bm,bn", [(128, 64), (64, 64), (32, 32), (16, 48)])
def test_host_tile_counts_equal_oracle_brute_force(L, S, bm, bn):
    enc = oracle.count_tiles(oracle.encoder_mask(L, S), bm, bn, [(0, L)])
    dec = oracle.count_tiles(oracle.decoder_mask(L, S), bm, bn, [(0, L), (L, 2 * L)])
    assert m.e2d2_attn_count_tiles(m.KIND_ENC, 1, 1, L, S, 0, bm, bn) == enc
    assert m.e2d2_attn_count_tiles(m.KIND_DEC, 1, 1, L, S, 0, bm, bn) == dec
    B, H = 3, 5
    v, f = m.e2d2_attn_count_tiles(m.KIND_DEC, B, H, L, S, 0, bm, bn)
    assert (v, f) == (dec[0] * B * H, dec[1] * B * H)


@pytest.mark.parametrize("S,C", [(32, 2048), (4, 32768), (8, 0), (33, 95), (1, 1)])
def test_host_denoise_tile_counts_equal_oracle(S, C):
    for bm, bn in [(32, 32), (64, 64)]:
        want = oracle.count_tiles(oracle.denoise_mask(S, C), bm, bn, [(0, C), (C, C + S)])
        assert m.e2d2_attn_count_tiles(m.KIND_DENOISE, 1, 1, 0, S, C, bm, bn) == want


def test_workload_tile_counts():
    # Training attention at B8 H16 L1024 S16 with 128x64 tiles: per (b, h) the encoder
    # visits 72 tiles (56 full) and the decoder 88 (56 full).
    v, f = m.e2d2_attn_count_tiles(m.KIND_ENC, 1, 1, 1024, 16, 0, 128, 64)
    assert (v, f) == (72, 56)
    v, f = m.e2d2_attn_count_tiles(m.KIND_DEC, 1, 1, 1024, 16, 0, 128, 64)
    assert (v, f) == (88, 56)


def _enc(**kw):
    a = dict(dtype=m.BF16, B=1, Hq=2, Hkv=1, L=64, d=64, S=8, scale=0.125, q=16, k=16, v=16,
             o=16, lse=None, dbg=None, stream=None)
    a.update(kw)
    return m.lib().e2d2_attn_encoder_blockcausal(*a.values())


def test_encoder_validation_returns_before_launch():
    # Fake, aligned, non-NULL "device pointers": validation fails before any use.
    assert _enc(q=None) == ERR_NULL
    assert _enc(d=48) == ERR_UNSUPPORTED
    assert _enc(dtype=5) == ERR_UNSUPPORTED
    assert _enc(B=0) == ERR_SHAPE
    assert _enc(S=0) == ERR_SHAPE
    assert _enc(Hq=3, Hkv=2) == ERR_SHAPE
    assert _enc(scale=0.0) == ERR_SHAPE
    assert _enc(scale=float("nan")) == ERR_SHAPE
    assert _enc(q=18) == ERR_SHAPE  # misaligned
    assert _enc(L=(1 << 24) + 1) == ERR_SHAPE


def _train(**kw):
    a = dict(dtype=m.BF16, B=1, Hq=2, Hkv=2, L=64, d=64, S=8, scale=0.125, q_dec=16, k_ctx=16,
             v_ctx=16, k_dec=16, v_dec=16, o_dec=16, lse_dec=None, q_enc=None, o_enc=None,
             lse_enc=None, dbg=None, stream=None)
    a.update(kw)
    return m.lib().e2d2_attn_train_fwd(*a.values())


def test_train_validation_returns_before_launch():
    assert _train(k_dec=None) == ERR_NULL
    assert _train(q_enc=16) == ERR_NULL          # encoder query without its output
    assert _train(o_enc=16) == ERR_NULL          # encoder output without its query
    assert _train(d=96) == ERR_UNSUPPORTED
    assert _train(Hkv=0) == ERR_SHAPE
    assert _train(dbg=12) == ERR_SHAPE           # misaligned counter


def _denoise(**kw):
    a = dict(dtype=m.BF16, B=1, Hq=2, Hkv=1, S=4, d=128, scale=0.1, q=16, kc=16, vc=16, C=8,
             cap=16, kb=16, vb=16, o=16, lse=None, ws=None, ws_bytes=0, dbg=None, stream=None)
    a.update(kw)
    return m.lib().e2d2_attn_denoise_step(*a.values())


def test_denoise_validation_returns_before_launch():
    assert _denoise(q=None) == ERR_NULL
    assert _denoise(kc=None) == ERR_NULL
    assert _denoise(C=17) == ERR_SHAPE           # cache_len > cache_cap
    assert _denoise(C=-1) == ERR_SHAPE
    assert _denoise(d=16) == ERR_UNSUPPORTED
    # a small batch splits the key axis and needs a workspace
    need = m.e2d2_attn_denoise_workspace_bytes(m.BF16, 1, 2, 1, 4, 128, 4096)
    assert need > 0
    assert _denoise(C=4096, cap=4096) == ERR_WORKSPACE
    assert _denoise(C=4096, cap=4096, ws=16, ws_bytes=need - 1) == ERR_WORKSPACE


def test_denoise_workspace_sizes():
    # Enough (batch, kv head) items to fill the GPU: no split, no workspace.
    assert m.e2d2_attn_denoise_workspace_bytes(m.BF16, 32, 16, 8, 32, 128, 2048) == 0
    assert m.e2d2_attn_denoise_workspace_bytes(m.BF16, 64, 32, 32, 4, 128, 32768) == 0
    assert m.e2d2_attn_denoise_workspace_bytes(m.F32, 1, 2, 1, 4, 128, 4096) == 0
    assert m.e2d2_attn_denoise_workspace_bytes(m.BF16, 1, 2, 3, 4, 128, 4096) == 0  # invalid


def _noalloc(**kw):
    a = dict(dtype=m.BF16, B=1, Hq=2, Hkv=1, S=4, d=128, scale=0.1, q=16, kc=16, vc=16, C=8,
             cap=16, kb=16, vb=16, o=16, lse=None, dbg=None, stream=None)
    a.update(kw)
    return m.lib().e2d2_attn_denoise_step_noalloc(*a.values())


def test_denoise_noalloc_validation_returns_before_launch():
    assert _noalloc(q=None) == ERR_NULL
    assert _noalloc(kc=None) == ERR_NULL
    assert _noalloc(C=17) == ERR_SHAPE           # cache_len > cache_cap
    assert _noalloc(Hq=3, Hkv=2) == ERR_SHAPE
    assert _noalloc(q=24) == ERR_SHAPE           # misaligned
    assert _noalloc(d=16) == ERR_UNSUPPORTED
    assert _noalloc(dtype=7) == ERR_UNSUPPORTED


def _enc_varlen(**kw):
    a = dict(dtype=m.BF16, B=2, Hq=2, Hkv=1, L=64, d=64, S=8, scale=0.125, q=16, k=16, v=16,
             kv_rows=80, lens=16, o=16, lse=None, dbg=None, stream=None)
    a.update(kw)
    return m.lib().e2d2_attn_encoder_blockcausal_varlen(*a.values())


def test_encoder_varlen_validation_returns_before_launch():
    assert _enc_varlen(lens=None) == ERR_NULL
    assert _enc_varlen(k=None) == ERR_NULL
    assert _enc_varlen(lens=18) == ERR_SHAPE      # misaligned int32 array
    assert _enc_varlen(kv_rows=63) == ERR_SHAPE   # K/V rows fewer than the query rows
    assert _enc_varlen(kv_rows=(1 << 24) + 1) == ERR_SHAPE
    assert _enc_varlen(dtype=m.F32) == ERR_UNSUPPORTED
    assert _enc_varlen(d=96) == ERR_UNSUPPORTED
    assert _enc_varlen(S=0) == ERR_SHAPE
    assert _enc_varlen(Hq=3, Hkv=2) == ERR_SHAPE
    assert _enc_varlen(o=40) == ERR_SHAPE         # misaligned


def test_append_validation():
    lib = m.lib()
    assert lib.e2d2_kv_cache_append(m.BF16, 1, 1, 4, 64, 16, 16, 10, 12, 16, 16, None) == ERR_CAPACITY
    assert lib.e2d2_kv_cache_append(m.BF16, 1, 1, 4, 64, None, 16, 0, 12, 16, 16, None) == ERR_NULL
    assert lib.e2d2_kv_cache_append(m.BF16, 1, 1, 4, 64, 16, 16, -1, 12, 16, 16, None) == ERR_SHAPE
    assert lib.e2d2_kv_cache_append(m.BF16, 1, 1, 4, 40, 16, 16, 0, 12, 16, 16, None) == ERR_UNSUPPORTED


def _varlen(**kw):
    a = dict(dtype=m.BF16, B=1, Hq=2, Hkv=1, S=4, d=128, scale=0.1, q=16, kc=16, vc=16, lens=16,
             C=8, cap=16, kb=16, vb=16, o=16, lse=None, ws=None, ws_bytes=0, dbg=None, stream=None)
    a.update(kw)
    return m.lib().e2d2_attn_denoise_step_varlen(*a.values())


def test_denoise_varlen_validation_returns_before_launch():
    assert _varlen(lens=None) == ERR_NULL
    assert _varlen(lens=18) == ERR_SHAPE          # misaligned int32 array
    assert _varlen(dtype=m.F32) == ERR_UNSUPPORTED
    assert _varlen(C=17) == ERR_SHAPE             # max length beyond the capacity
    assert _varlen(kc=None) == ERR_NULL
    need = m.e2d2_attn_denoise_workspace_bytes(m.BF16, 1, 2, 1, 4, 128, 4096)
    assert _varlen(C=4096, cap=4096, ws=16, ws_bytes=need - 1) == ERR_WORKSPACE


def test_append_varlen_validation():
    lib = m.lib()
    f = lib.e2d2_kv_cache_append_varlen
    assert f(m.BF16, 1, 1, 4, 64, 16, 16, 16, 13, 16, 16, 16, None) == ERR_CAPACITY
    assert f(m.BF16, 1, 1, 4, 64, 16, 16, None, 12, 16, 16, 16, None) == ERR_NULL
    assert f(m.BF16, 1, 1, 4, 64, 16, 16, 18, 12, 16, 16, 16, None) == ERR_SHAPE
    assert f(m.BF16, 1, 1, 4, 48, 16, 16, 16, 12, 16, 16, 16, None) == ERR_UNSUPPORTED


def _bwd(**kw):
    a = dict(dtype=m.BF16, B=1, Hq=2, Hkv=1, L=64, d=64, S=8, scale=0.125, q_dec=16, k_ctx=16,
             v_ctx=16, k_dec=16, v_dec=16, o_dec=16, lse_dec=16, do_dec=16, q_enc=None,
             o_enc=None, lse_enc=None, do_enc=None, dq_dec=16, dk_ctx=16, dv_ctx=16, dk_dec=16,
             dv_dec=16, dq_enc=None, ws=16, ws_bytes=1 << 20, stream=None)
    a.update(kw)
    return m.lib().e2d2_attn_train_bwd(*a.values())


def test_train_bwd_validation_returns_before_launch():
    assert _bwd(lse_dec=None) == ERR_NULL
    assert _bwd(dk_ctx=None) == ERR_NULL
    assert _bwd(q_enc=16) == ERR_NULL                 # encoder query without its other tensors
    assert _bwd(dq_enc=16) == ERR_NULL                # encoder output without its query
    assert _bwd(dtype=m.F32) == ERR_UNSUPPORTED
    assert _bwd(d=96) == ERR_UNSUPPORTED
    assert _bwd(Hq=3, Hkv=2) == ERR_SHAPE
    assert _bwd(do_dec=24) == ERR_SHAPE               # misaligned
    assert _bwd(ws=None) == ERR_WORKSPACE
    need = m.e2d2_attn_train_bwd_workspace_bytes(m.BF16, 1, 2, 64, True)
    assert need >= 4 * 2 * 64 * 4
    assert m.e2d2_attn_train_bwd_workspace_bytes(m.BF16, 1, 2, 64, False) * 2 == need
    assert _bwd(q_enc=16, o_enc=16, lse_enc=16, do_enc=16, dq_enc=16, ws_bytes=need - 1) == ERR_WORKSPACE
    assert m.e2d2_attn_train_bwd_workspace_bytes(m.F32, 1, 2, 64, True) == 0


def _layer(**kw):
    a = dict(dtype=m.BF16, B=2, Hq=4, Hkv=2, S=8, d=64, Dm=256, scale=0.125, x=16, w_qkv=16,
             w_o=16, k_cache=16, v_cache=16, cache_len=100, cache_cap=128, q_blk=16, k_blk=16,
             v_blk=16, o_blk=16, lse_blk=None, y=16, ws=16, ws_bytes=1 << 24, stream=None)
    a.update(kw)
    return m.lib().e2d2_decoder_layer_denoise_step(*a.values())


def test_layer_validation_returns_before_launch():
    assert _layer(x=None) == ERR_NULL
    assert _layer(w_o=None) == ERR_NULL
    assert _layer(y=None) == ERR_NULL
    assert _layer(q_blk=None) == ERR_NULL             # the attention's own checks run first too
    assert _layer(k_cache=None) == ERR_NULL
    assert _layer(dtype=m.F32) == ERR_UNSUPPORTED
    assert _layer(d=48) == ERR_UNSUPPORTED
    assert _layer(Dm=100) == ERR_SHAPE                # rows of x must be whole 16-byte chunks
    assert _layer(Hq=3) == ERR_SHAPE
    assert _layer(x=24) == ERR_SHAPE                  # misaligned
    assert _layer(cache_len=200) == ERR_SHAPE         # past the capacity
    assert _layer(B=1 << 14, S=1 << 10, Dm=1 << 10) == ERR_SHAPE  # x reaches 2 GiB
    need = m.e2d2_attn_denoise_workspace_bytes(m.BF16, 1, 2, 1, 8, 128, 1 << 16)
    assert need > 0
    assert _layer(B=1, Hq=2, Hkv=1, d=128, cache_len=1 << 16, cache_cap=1 << 16, ws=None) == ERR_WORKSPACE
