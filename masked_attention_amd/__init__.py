"""Python binding of libe2d2_attn.so, the MI355X (gfx950) E2D2 attention library.

Argument marshalling only: every function here checks the torch tensors it is given
(device, dtype, contiguity, shapes), passes their device pointers, sizes and the
current HIP stream to the C-ABI function of the same name, and raises on a non-OK
status.  All computation happens in the HIP kernels of the library; there is no other
code path.  The C ABI (include/e2d2_attn.h) documents each call.

``torch`` is imported before the library is loaded so that the library binds to the
HIP runtime torch already has in the process (one runtime, shared streams).
"""
from __future__ import annotations

import ctypes
import math
import os

import torch

__all__ = [
    "E2D2Error", "lib", "library_path", "abi_version",
    "e2d2_attn_encoder_blockcausal", "e2d2_attn_encoder_blockcausal_varlen",
    "e2d2_attn_train_fwd", "e2d2_attn_denoise_step", "e2d2_attn_denoise_step_noalloc",
    "e2d2_attn_denoise_workspace_bytes", "e2d2_kv_cache_append", "e2d2_attn_tile_shape",
    "e2d2_attn_count_tiles", "e2d2_attn_denoise_step_varlen", "e2d2_kv_cache_append_varlen",
    "e2d2_attn_train_bwd", "e2d2_attn_train_bwd_workspace_bytes",
    "e2d2_decoder_layer_denoise_step", "KIND_ENC", "KIND_DEC", "KIND_DENOISE", "F32", "BF16",
]

F32, BF16 = 0, 1
KIND_ENC, KIND_DEC, KIND_DENOISE = 0, 1, 2

_HERE = os.path.dirname(os.path.abspath(__file__))
library_path = os.path.join(_HERE, "libe2d2_attn.so")

_vp = ctypes.c_void_p
_i = ctypes.c_int
_ll = ctypes.c_longlong
_f = ctypes.c_float
_sz = ctypes.c_size_t
_ull_p = ctypes.POINTER(ctypes.c_ulonglong)
_int_p = ctypes.POINTER(ctypes.c_int)

_SIGS = {
    "e2d2_abi_version": (_i, []),
    "e2d2_status_string": (ctypes.c_char_p, [_i]),
    "e2d2_last_hip_error": (_i, []),
    "e2d2_attn_encoder_blockcausal": (_i, [_i, _i, _i, _i, _i, _i, _i, _f, _vp, _vp, _vp, _vp, _vp,
                                           _vp, _vp]),
    "e2d2_attn_encoder_blockcausal_varlen": (_i, [_i, _i, _i, _i, _i, _i, _i, _f, _vp, _vp, _vp,
                                                  _ll, _vp, _vp, _vp, _vp, _vp]),
    "e2d2_attn_train_fwd": (_i, [_i, _i, _i, _i, _i, _i, _i, _f, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                 _vp, _vp, _vp, _vp, _vp]),
    "e2d2_attn_denoise_workspace_bytes": (_sz, [_i, _i, _i, _i, _i, _i, _ll]),
    "e2d2_attn_denoise_step": (_i, [_i, _i, _i, _i, _i, _i, _f, _vp, _vp, _vp, _ll, _ll, _vp, _vp,
                                    _vp, _vp, _vp, _sz, _vp, _vp]),
    "e2d2_attn_denoise_step_noalloc": (_i, [_i, _i, _i, _i, _i, _i, _f, _vp, _vp, _vp, _ll, _ll,
                                            _vp, _vp, _vp, _vp, _vp, _vp]),
    "e2d2_kv_cache_append": (_i, [_i, _i, _i, _i, _i, _vp, _vp, _ll, _ll, _vp, _vp, _vp]),
    "e2d2_attn_denoise_step_varlen": (_i, [_i, _i, _i, _i, _i, _i, _f, _vp, _vp, _vp, _vp, _ll, _ll,
                                           _vp, _vp, _vp, _vp, _vp, _sz, _vp, _vp]),
    "e2d2_kv_cache_append_varlen": (_i, [_i, _i, _i, _i, _i, _vp, _vp, _vp, _ll, _ll, _vp, _vp,
                                         _vp]),
    "e2d2_attn_train_bwd_workspace_bytes": (_sz, [_i, _i, _i, _i, _i]),
    "e2d2_attn_train_bwd": (_i, [_i, _i, _i, _i, _i, _i, _i, _f] + [_vp] * 19 + [_sz, _vp]),
    "e2d2_decoder_layer_denoise_step": (_i, [_i, _i, _i, _i, _i, _i, _i, _f, _vp, _vp, _vp, _vp,
                                             _vp, _ll, _ll, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                             _sz, _vp]),
    "e2d2_attn_tile_shape": (_i, [_i, _i, _i, _int_p, _int_p]),
    "e2d2_attn_count_tiles": (_i, [_i, _i, _i, _i, _i, _ll, _i, _i, _ull_p, _ull_p]),
}

_LIB = None


class E2D2Error(RuntimeError):
    """A non-OK status from the library."""

    def __init__(self, fn: str, status: int):
        self.status = status
        msg = lib().e2d2_status_string(status).decode()
        if status == 6:
            msg += f" (hipError {lib().e2d2_last_hip_error()})"
        super().__init__(f"{fn}: status {status}: {msg}")


def lib():
    """The loaded C library (ctypes.CDLL) with typed signatures."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(library_path):
            raise RuntimeError(f"{library_path} is not built: run python -m "
                               "masked_attention_amd.build (hipcc for gfx950) first")
        h = ctypes.CDLL(library_path)
        for name, (res, args) in _SIGS.items():
            f = getattr(h, name)
            f.restype = res
            f.argtypes = args
        _LIB = h
    return _LIB


def abi_version() -> int:
    return lib().e2d2_abi_version()


# ----------------------------------------------------------------------------- helpers
def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return BF16
    if t.dtype == torch.float32:
        return F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _dev(t: torch.Tensor, name: str, ndim: int = 4) -> int:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on the GPU")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims")
    return t.data_ptr()


def _opt(t, name, ndim):
    return None if t is None else _dev(t, name, ndim)


def _stream(t: torch.Tensor) -> int:
    return torch.cuda.current_stream(t.device).cuda_stream


def _check(fn: str, status: int) -> None:
    if status != 0:
        raise E2D2Error(fn, status)


def _same(dt, *ts):
    for t in ts:
        if t is not None and t.dtype != dt:
            raise TypeError("all q/k/v/o tensors must share one dtype")


def _default_scale(d: int, scale):
    return 1.0 / math.sqrt(d) if scale is None else float(scale)


# ----------------------------------------------------------------------------- calls
def e2d2_attn_encoder_blockcausal(q, k, v, o, S: int, lse=None, scale=None, tile_visits=None):
    """Encoder block-causal attention; q/o [B, Hq, L, d], k/v [B, Hkv, L, d]."""
    B, Hq, L, d = q.shape
    Hkv = k.shape[1]
    _same(q.dtype, k, v, o)
    if tuple(k.shape) != (B, Hkv, L, d) or tuple(v.shape) != tuple(k.shape) or o.shape != q.shape:
        raise ValueError("shape mismatch")
    if lse is not None and (lse.dtype != torch.float32 or tuple(lse.shape) != (B, Hq, L)):
        raise ValueError("lse must be float32 [B, Hq, L]")
    st = lib().e2d2_attn_encoder_blockcausal(
        _dtype_code(q), B, Hq, Hkv, L, d, int(S), _default_scale(d, scale), _dev(q, "q"),
        _dev(k, "k"), _dev(v, "v"), _dev(o, "o"), _opt(lse, "lse", 3),
        _opt(tile_visits, "tile_visits", 1), _stream(q))
    _check("e2d2_attn_encoder_blockcausal", st)


def e2d2_attn_encoder_blockcausal_varlen(q, k, v, lens, o, S: int, lse=None, scale=None,
                                         tile_visits=None):
    """Prompt encoding with per-sequence lengths: q/o [B, Hq, L, d]; k/v [B, Hkv, kv_rows,
    d] (kv_rows >= L, e.g. the KV-cache buffers); ``lens`` an int32 CUDA tensor [B] read
    on the device.  Sequence b's rows [0, lens[b]) attend its keys [0, lens[b]) under
    the block-causal mask; the rest of o and lse is left untouched (bf16 only)."""
    B, Hq, L, d = q.shape
    Hkv, kv_rows = k.shape[1], k.shape[2]
    _same(q.dtype, k, v, o)
    if tuple(k.shape) != (B, Hkv, kv_rows, d) or v.shape != k.shape or o.shape != q.shape:
        raise ValueError("shape mismatch")
    if lse is not None and (lse.dtype != torch.float32 or tuple(lse.shape) != (B, Hq, L)):
        raise ValueError("lse must be float32 [B, Hq, L]")
    st = lib().e2d2_attn_encoder_blockcausal_varlen(
        _dtype_code(q), B, Hq, Hkv, L, d, int(S), _default_scale(d, scale), _dev(q, "q"),
        _dev(k, "k"), _dev(v, "v"), kv_rows, _lens(lens, B), _dev(o, "o"), _opt(lse, "lse", 3),
        _opt(tile_visits, "tile_visits", 1), _stream(q))
    _check("e2d2_attn_encoder_blockcausal_varlen", st)


def e2d2_attn_train_fwd(q_dec, k_ctx, v_ctx, k_dec, v_dec, o_dec, S: int, lse_dec=None,
                        q_enc=None, o_enc=None, lse_enc=None, scale=None, tile_visits=None):
    """Fused decoder attention over [clean | noised] keys, plus the encoder
    block-causal attention of (q_enc, k_ctx, v_ctx) in the same launch when q_enc is
    given."""
    B, Hq, L, d = q_dec.shape
    Hkv = k_ctx.shape[1]
    _same(q_dec.dtype, k_ctx, v_ctx, k_dec, v_dec, o_dec, q_enc, o_enc)
    for t in (k_ctx, v_ctx, k_dec, v_dec):
        if tuple(t.shape) != (B, Hkv, L, d):
            raise ValueError("k/v must be [B, Hkv, L, d]")
    for t in (o_dec, q_enc, o_enc):
        if t is not None and t.shape != q_dec.shape:
            raise ValueError("q/o must be [B, Hq, L, d]")
    for t in (lse_dec, lse_enc):
        if t is not None and (t.dtype != torch.float32 or tuple(t.shape) != (B, Hq, L)):
            raise ValueError("lse must be float32 [B, Hq, L]")
    st = lib().e2d2_attn_train_fwd(
        _dtype_code(q_dec), B, Hq, Hkv, L, d, int(S), _default_scale(d, scale),
        _dev(q_dec, "q_dec"), _dev(k_ctx, "k_ctx"), _dev(v_ctx, "v_ctx"), _dev(k_dec, "k_dec"),
        _dev(v_dec, "v_dec"), _dev(o_dec, "o_dec"), _opt(lse_dec, "lse_dec", 3),
        _opt(q_enc, "q_enc", 4), _opt(o_enc, "o_enc", 4), _opt(lse_enc, "lse_enc", 3),
        _opt(tile_visits, "tile_visits", 1), _stream(q_dec))
    _check("e2d2_attn_train_fwd", st)


def e2d2_attn_train_bwd_workspace_bytes(dtype: int, B: int, Hq: int, L: int, with_enc: bool) -> int:
    return int(lib().e2d2_attn_train_bwd_workspace_bytes(dtype, B, Hq, L, 1 if with_enc else 0))


def e2d2_attn_train_bwd(q_dec, k_ctx, v_ctx, k_dec, v_dec, o_dec, lse_dec, do_dec, S: int,
                        dq_dec, dk_ctx, dv_ctx, dk_dec, dv_dec, workspace, q_enc=None,
                        o_enc=None, lse_enc=None, do_enc=None, dq_enc=None, scale=None):
    """Backward of e2d2_attn_train_fwd: writes dq_dec, dk_ctx, dv_ctx, dk_dec, dv_dec
    (and dq_enc when q_enc is given) from the forward's o/lse and the upstream
    gradients do_dec (do_enc).  ``workspace``: uint8 CUDA tensor of at least
    e2d2_attn_train_bwd_workspace_bytes(...) bytes."""
    B, Hq, L, d = q_dec.shape
    Hkv = k_ctx.shape[1]
    kv = (B, Hkv, L, d)
    _same(q_dec.dtype, k_ctx, v_ctx, k_dec, v_dec, o_dec, do_dec, dq_dec, dk_ctx, dv_ctx, dk_dec, dv_dec)
    for t in (o_dec, do_dec, dq_dec):
        if t.shape != q_dec.shape:
            raise ValueError("query-side tensors must be [B, Hq, L, d]")
    for t in (k_ctx, v_ctx, k_dec, v_dec, dk_ctx, dv_ctx, dk_dec, dv_dec):
        if tuple(t.shape) != kv:
            raise ValueError("key-side tensors must be [B, Hkv, L, d]")
    enc = [q_enc, o_enc, lse_enc, do_enc, dq_enc]
    if q_enc is not None:
        if any(t is None for t in enc):
            raise ValueError("q_enc needs o_enc, lse_enc, do_enc and dq_enc")
        _same(q_dec.dtype, q_enc, o_enc, do_enc, dq_enc)
        for t in (q_enc, o_enc, do_enc, dq_enc):
            if t.shape != q_dec.shape:
                raise ValueError("encoder tensors must be [B, Hq, L, d]")
    for t in (lse_dec, lse_enc):
        if t is not None and (t.dtype != torch.float32 or tuple(t.shape) != (B, Hq, L)):
            raise ValueError("lse must be float32 [B, Hq, L]")
    ws_ptr = _dev(workspace, "workspace", workspace.dim())
    ws_bytes = workspace.numel() * workspace.element_size()
    opt = lambda t, n, nd=4: _opt(t, n, nd)
    st = lib().e2d2_attn_train_bwd(
        _dtype_code(q_dec), B, Hq, Hkv, L, d, S, _default_scale(d, scale),
        _dev(q_dec, "q_dec"), _dev(k_ctx, "k_ctx"), _dev(v_ctx, "v_ctx"), _dev(k_dec, "k_dec"),
        _dev(v_dec, "v_dec"), _dev(o_dec, "o_dec"), _dev(lse_dec, "lse_dec", 3),
        _dev(do_dec, "do_dec"), opt(q_enc, "q_enc"), opt(o_enc, "o_enc"),
        opt(lse_enc, "lse_enc", 3), opt(do_enc, "do_enc"), _dev(dq_dec, "dq_dec"),
        _dev(dk_ctx, "dk_ctx"), _dev(dv_ctx, "dv_ctx"), _dev(dk_dec, "dk_dec"),
        _dev(dv_dec, "dv_dec"), opt(dq_enc, "dq_enc"), ws_ptr, ws_bytes, _stream(q_dec))
    _check("e2d2_attn_train_bwd", st)


def e2d2_attn_denoise_workspace_bytes(dtype: int, B: int, Hq: int, Hkv: int, S: int, d: int,
                                      cache_len: int) -> int:
    return int(lib().e2d2_attn_denoise_workspace_bytes(dtype, B, Hq, Hkv, S, d, int(cache_len)))


def e2d2_attn_denoise_step(q_blk, k_cache, v_cache, cache_len: int, k_blk, v_blk, o_blk,
                           lse_blk=None, workspace=None, scale=None, tile_visits=None):
    """One denoising step: q_blk/o_blk [B, Hq, S, d], caches [B, Hkv, cap, d] with rows
    [0, cache_len) valid, k_blk/v_blk [B, Hkv, S, d].  ``workspace`` is a uint8 CUDA
    tensor of at least e2d2_attn_denoise_workspace_bytes(...) bytes (may be None when
    that is 0)."""
    B, Hq, S, d = q_blk.shape
    Hkv, cap = k_cache.shape[1], k_cache.shape[2]
    _same(q_blk.dtype, k_cache, v_cache, k_blk, v_blk, o_blk)
    if tuple(k_cache.shape) != (B, Hkv, cap, d) or v_cache.shape != k_cache.shape:
        raise ValueError("caches must be [B, Hkv, cap, d]")
    if tuple(k_blk.shape) != (B, Hkv, S, d) or v_blk.shape != k_blk.shape or o_blk.shape != q_blk.shape:
        raise ValueError("shape mismatch")
    if lse_blk is not None and (lse_blk.dtype != torch.float32 or tuple(lse_blk.shape) != (B, Hq, S)):
        raise ValueError("lse must be float32 [B, Hq, S]")
    ws_ptr, ws_bytes = None, 0
    if workspace is not None:
        ws_ptr, ws_bytes = _dev(workspace, "workspace", workspace.dim()), workspace.numel() * workspace.element_size()
    st = lib().e2d2_attn_denoise_step(
        _dtype_code(q_blk), B, Hq, Hkv, S, d, _default_scale(d, scale), _dev(q_blk, "q_blk"),
        _dev(k_cache, "k_cache"), _dev(v_cache, "v_cache"), int(cache_len), cap,
        _dev(k_blk, "k_blk"), _dev(v_blk, "v_blk"), _dev(o_blk, "o_blk"),
        _opt(lse_blk, "lse_blk", 3), ws_ptr, ws_bytes, _opt(tile_visits, "tile_visits", 1),
        _stream(q_blk))
    _check("e2d2_attn_denoise_step", st)


def e2d2_attn_denoise_step_noalloc(q_blk, k_cache, v_cache, cache_len: int, k_blk, v_blk, o_blk,
                                   lse_blk=None, scale=None, tile_visits=None):
    """e2d2_attn_denoise_step without a workspace argument: when the step splits its key
    axis, the partials go to the library's own fixed device scratch (nothing is
    allocated).  Calls that may overlap on one GPU race on that scratch."""
    B, Hq, S, d = q_blk.shape
    Hkv, cap = k_cache.shape[1], k_cache.shape[2]
    _same(q_blk.dtype, k_cache, v_cache, k_blk, v_blk, o_blk)
    if tuple(k_cache.shape) != (B, Hkv, cap, d) or v_cache.shape != k_cache.shape:
        raise ValueError("caches must be [B, Hkv, cap, d]")
    if tuple(k_blk.shape) != (B, Hkv, S, d) or v_blk.shape != k_blk.shape or o_blk.shape != q_blk.shape:
        raise ValueError("shape mismatch")
    if lse_blk is not None and (lse_blk.dtype != torch.float32 or tuple(lse_blk.shape) != (B, Hq, S)):
        raise ValueError("lse must be float32 [B, Hq, S]")
    st = lib().e2d2_attn_denoise_step_noalloc(
        _dtype_code(q_blk), B, Hq, Hkv, S, d, _default_scale(d, scale), _dev(q_blk, "q_blk"),
        _dev(k_cache, "k_cache"), _dev(v_cache, "v_cache"), int(cache_len), cap,
        _dev(k_blk, "k_blk"), _dev(v_blk, "v_blk"), _dev(o_blk, "o_blk"),
        _opt(lse_blk, "lse_blk", 3), _opt(tile_visits, "tile_visits", 1), _stream(q_blk))
    _check("e2d2_attn_denoise_step_noalloc", st)


def _lens(cache_lens, B):
    if (cache_lens.dtype != torch.int32 or tuple(cache_lens.shape) != (B,)
            or not cache_lens.is_contiguous()):
        raise ValueError("cache_lens must be a contiguous int32 tensor [B]")
    return _dev(cache_lens, "cache_lens", 1)


def e2d2_attn_denoise_step_varlen(q_blk, k_cache, v_cache, cache_lens, max_cache_len: int, k_blk,
                                  v_blk, o_blk, lse_blk=None, workspace=None, scale=None,
                                  tile_visits=None):
    """One denoising step where sequence b attends cache rows [0, cache_lens[b]);
    ``cache_lens`` is an int32 CUDA tensor [B] read on the device (each length clamped
    to [0, max_cache_len]), other arguments as e2d2_attn_denoise_step."""
    B, Hq, S, d = q_blk.shape
    Hkv, cap = k_cache.shape[1], k_cache.shape[2]
    _same(q_blk.dtype, k_cache, v_cache, k_blk, v_blk, o_blk)
    if tuple(k_cache.shape) != (B, Hkv, cap, d) or v_cache.shape != k_cache.shape:
        raise ValueError("caches must be [B, Hkv, cap, d]")
    if tuple(k_blk.shape) != (B, Hkv, S, d) or v_blk.shape != k_blk.shape or o_blk.shape != q_blk.shape:
        raise ValueError("shape mismatch")
    if lse_blk is not None and (lse_blk.dtype != torch.float32 or tuple(lse_blk.shape) != (B, Hq, S)):
        raise ValueError("lse must be float32 [B, Hq, S]")
    ws_ptr, ws_bytes = None, 0
    if workspace is not None:
        ws_ptr, ws_bytes = _dev(workspace, "workspace", workspace.dim()), workspace.numel() * workspace.element_size()
    st = lib().e2d2_attn_denoise_step_varlen(
        _dtype_code(q_blk), B, Hq, Hkv, S, d, _default_scale(d, scale), _dev(q_blk, "q_blk"),
        _dev(k_cache, "k_cache"), _dev(v_cache, "v_cache"), _lens(cache_lens, B),
        int(max_cache_len), cap, _dev(k_blk, "k_blk"), _dev(v_blk, "v_blk"),
        _dev(o_blk, "o_blk"), _opt(lse_blk, "lse_blk", 3), ws_ptr, ws_bytes,
        _opt(tile_visits, "tile_visits", 1), _stream(q_blk))
    _check("e2d2_attn_denoise_step_varlen", st)


def e2d2_kv_cache_append_varlen(k_cache, v_cache, cache_lens, max_cache_len: int, k_new, v_new):
    """Copy k_new/v_new [B, Hkv, S, d] of sequence b into its cache rows
    [cache_lens[b], cache_lens[b] + S) (cache_lens: int32 CUDA tensor [B])."""
    B, Hkv, cap, d = k_cache.shape
    S = k_new.shape[2]
    _same(k_cache.dtype, v_cache, k_new, v_new)
    if v_cache.shape != k_cache.shape or tuple(k_new.shape) != (B, Hkv, S, d) or v_new.shape != k_new.shape:
        raise ValueError("shape mismatch")
    st = lib().e2d2_kv_cache_append_varlen(
        _dtype_code(k_cache), B, Hkv, S, d, _dev(k_cache, "k_cache"), _dev(v_cache, "v_cache"),
        _lens(cache_lens, B), int(max_cache_len), cap, _dev(k_new, "k_new"), _dev(v_new, "v_new"),
        _stream(k_cache))
    _check("e2d2_kv_cache_append_varlen", st)


def e2d2_kv_cache_append(k_cache, v_cache, cache_len: int, k_new, v_new):
    """Copy k_new/v_new [B, Hkv, S, d] into cache rows [cache_len, cache_len + S)."""
    B, Hkv, cap, d = k_cache.shape
    S = k_new.shape[2]
    _same(k_cache.dtype, v_cache, k_new, v_new)
    if v_cache.shape != k_cache.shape or tuple(k_new.shape) != (B, Hkv, S, d) or v_new.shape != k_new.shape:
        raise ValueError("shape mismatch")
    st = lib().e2d2_kv_cache_append(
        _dtype_code(k_cache), B, Hkv, S, d, _dev(k_cache, "k_cache"), _dev(v_cache, "v_cache"),
        int(cache_len), cap, _dev(k_new, "k_new"), _dev(v_new, "v_new"), _stream(k_cache))
    _check("e2d2_kv_cache_append", st)


def e2d2_decoder_layer_denoise_step(x, w_qkv, w_o, k_cache, v_cache, cache_len: int, q_blk, k_blk,
                                    v_blk, o_blk, y, lse_blk=None, workspace=None, scale=None):
    """Attention sublayer of a decoder layer for one denoising step (bf16): q/k/v =
    per-head slices of x W_qkv^T, the denoise attention over the cache plus the own
    block, y = concat_h(o) W_o^T.  x, y [B, S, Dm]; w_qkv [(Hq + 2 Hkv) d, Dm];
    w_o [Dm, Hq d]; caches [B, Hkv, cap, d]; q_blk, o_blk [B, Hq, S, d] and k_blk,
    v_blk [B, Hkv, S, d] are written; workspace as e2d2_attn_denoise_step."""
    B, S, Dm = x.shape
    _, Hq, _, d = q_blk.shape
    Hkv, cap = k_cache.shape[1], k_cache.shape[2]
    _same(x.dtype, w_qkv, w_o, k_cache, v_cache, q_blk, k_blk, v_blk, o_blk, y)
    if tuple(w_qkv.shape) != ((Hq + 2 * Hkv) * d, Dm) or tuple(w_o.shape) != (Dm, Hq * d):
        raise ValueError("weights must be w_qkv [(Hq + 2 Hkv) d, Dm] and w_o [Dm, Hq d]")
    if tuple(q_blk.shape) != (B, Hq, S, d) or o_blk.shape != q_blk.shape:
        raise ValueError("q_blk and o_blk must be [B, Hq, S, d]")
    if tuple(k_blk.shape) != (B, Hkv, S, d) or v_blk.shape != k_blk.shape:
        raise ValueError("k_blk and v_blk must be [B, Hkv, S, d]")
    if tuple(k_cache.shape) != (B, Hkv, cap, d) or v_cache.shape != k_cache.shape:
        raise ValueError("caches must be [B, Hkv, cap, d]")
    if y.shape != x.shape:
        raise ValueError("y must be [B, S, Dm]")
    if lse_blk is not None and (lse_blk.dtype != torch.float32 or tuple(lse_blk.shape) != (B, Hq, S)):
        raise ValueError("lse must be float32 [B, Hq, S]")
    ws_ptr, ws_bytes = None, 0
    if workspace is not None:
        ws_ptr, ws_bytes = _dev(workspace, "workspace", workspace.dim()), workspace.numel() * workspace.element_size()
    st = lib().e2d2_decoder_layer_denoise_step(
        _dtype_code(x), B, Hq, Hkv, S, d, Dm, _default_scale(d, scale), _dev(x, "x", 3),
        _dev(w_qkv, "w_qkv", 2), _dev(w_o, "w_o", 2), _dev(k_cache, "k_cache"),
        _dev(v_cache, "v_cache"), int(cache_len), cap, _dev(q_blk, "q_blk"), _dev(k_blk, "k_blk"),
        _dev(v_blk, "v_blk"), _dev(o_blk, "o_blk"), _opt(lse_blk, "lse_blk", 3), _dev(y, "y", 3),
        ws_ptr, ws_bytes, _stream(x))
    _check("e2d2_decoder_layer_denoise_step", st)


def e2d2_attn_tile_shape(kind: int, dtype: int, d: int):
    bm, bn = ctypes.c_int(), ctypes.c_int()
    _check("e2d2_attn_tile_shape", lib().e2d2_attn_tile_shape(kind, dtype, d, ctypes.byref(bm),
                                                              ctypes.byref(bn)))
    return bm.value, bn.value


def e2d2_attn_count_tiles(kind: int, B: int, Hq: int, L: int, S: int, cache_len: int, bm: int,
                          bn: int):
    v, f = ctypes.c_ulonglong(), ctypes.c_ulonglong()
    _check("e2d2_attn_count_tiles", lib().e2d2_attn_count_tiles(
        kind, B, Hq, L, S, int(cache_len), bm, bn, ctypes.byref(v), ctypes.byref(f)))
    return v.value, f.value


from .autograd import e2d2_attention  # noqa: E402  (needs the wrappers above)

__all__.append("e2d2_attention")
