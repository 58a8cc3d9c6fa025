"""Counter-based N(0, 1) generator (host side) and the launcher of its device twin.

Definition (the device kernel in ``synth_fill.hip`` implements the same steps):

* ``splitmix64`` is the generator of Steele, Lea and Flood, "Fast Splittable
  Pseudorandom Number Generators" (OOPSLA 2014): state += 0x9E3779B97F4A7C15, then
  the output is mix64(state) with
  ``z ^= z >> 30; z *= 0xBF58476D1CE4E5B9; z ^= z >> 27; z *= 0x94D049BB133111EB;
  z ^= z >> 31`` (all arithmetic mod 2**64).
* A tensor stream key is ``mix64(seed * GOLDEN + tensor_id)``.
* Element (b, h, n, c) has the counter ``e = ((b * 2**12 + h) * 2**24 + n) * 2**10 + c``;
  its three 64-bit words are ``w_t = mix64(key + (3*e + t + 1) * GOLDEN)``, t = 0, 1, 2.
* The twelve 16-bit fields k_1..k_12 of w_0, w_1, w_2 give
  ``x = (sum(k) - 393210) / 65536``, which is sum(u_i) - 6 with u_i = (k_i + 0.5)/65536,
  the classical sum-of-twelve-uniforms approximation of N(0, 1) (mean 0, variance
  1 - 2**-32, support [-6, 6]).  The numerator is an integer below 2**19 and the
  divisor a power of two, so x is exact in float32 on every platform.
* bf16 tensors take x rounded to nearest-even.

Limits: b < 2**18, h < 2**12, n < 2**24, c < 2**10.
"""
from __future__ import annotations

import ctypes
import enum
import os

import numpy as np

GOLDEN = 0x9E3779B97F4A7C15
_M1 = 0xBF58476D1CE4E5B9
_M2 = 0x94D049BB133111EB
_MASK = (1 << 64) - 1


class TensorKind(enum.IntEnum):
    """Stable ids of the tensors a workload draws."""

    Q_ENC = 1
    K_CTX = 2
    V_CTX = 3
    Q_DEC = 4
    K_DEC = 5
    V_DEC = 6
    Q_BLK = 7
    K_BLK = 8
    V_BLK = 9
    K_NEW = 10
    V_NEW = 11
    K_CACHE = 12
    V_CACHE = 13
    PROBE = 14
    DO_DEC = 15   # upstream gradient of the decoder attention output (backward pass)
    DO_ENC = 16   # upstream gradient of the encoder attention output
    X_BLK = 17    # hidden states of a block's noised tokens entering a decoder layer
    W_QKV = 18    # a decoder layer's stacked query/key/value projection weights
    W_O = 19      # a decoder layer's output projection weights


def tensor_id(kind: int, step: int = 0, block: int = 0) -> int:
    """Tensor id of ``kind`` at denoising ``step`` of ``block`` (both default 0)."""
    return int(kind) + 256 * (int(step) + 65536 * int(block))


def _mix64_int(z: int) -> int:
    z &= _MASK
    z = ((z ^ (z >> 30)) * _M1) & _MASK
    z = ((z ^ (z >> 27)) * _M2) & _MASK
    return z ^ (z >> 31)


def stream_key(seed: int, tid: int) -> int:
    return _mix64_int((int(seed) * GOLDEN + int(tid)) & _MASK)


def _mix64(z: np.ndarray) -> np.ndarray:
    z = (z ^ (z >> np.uint64(30))) * np.uint64(_M1)
    z = (z ^ (z >> np.uint64(27))) * np.uint64(_M2)
    return z ^ (z >> np.uint64(31))


def _sum16(w: np.ndarray) -> np.ndarray:
    f = np.uint64(0xFFFF)
    return ((w & f) + ((w >> np.uint64(16)) & f) + ((w >> np.uint64(32)) & f)
            + (w >> np.uint64(48))).astype(np.int64)


def normal_f32(seed: int, tid: int, shape, n0: int = 0, b0: int = 0, h0: int = 0) -> np.ndarray:
    """float32 array of ``shape`` = (B, H, N, D) holding elements
    (b0+b, h0+h, n0+n, c) of tensor ``tid`` under ``seed``."""
    B, H, N, D = (int(s) for s in shape)
    if not (b0 + B <= 1 << 18 and h0 + H <= 1 << 12 and n0 + N <= 1 << 24 and D <= 1 << 10):
        raise ValueError("tensor too large for the counter layout")
    key = np.uint64(stream_key(seed, tid))
    out = np.empty((B, H, N, D), dtype=np.float32)
    c = np.arange(D, dtype=np.uint64)
    gold = np.uint64(GOLDEN)
    rows_per_chunk = max(1, (1 << 21) // max(D, 1))
    with np.errstate(over="ignore"):
        for b in range(B):
            for h in range(H):
                bh = np.uint64(((b0 + b) << 12) + (h0 + h))
                for r in range(0, N, rows_per_chunk):
                    rr = min(N, r + rows_per_chunk)
                    n = np.arange(n0 + r, n0 + rr, dtype=np.uint64)
                    e = ((bh << np.uint64(24)) + n)[:, None] << np.uint64(10)
                    e = e + c[None, :]
                    base = key + (np.uint64(3) * e + np.uint64(1)) * gold
                    s = _sum16(_mix64(base)) + _sum16(_mix64(base + gold)) \
                        + _sum16(_mix64(base + gold + gold))
                    out[b, h, r:rr] = (s - 393210).astype(np.float32) / np.float32(65536.0)
    return out


def draw_view(shape) -> tuple:
    """The [B, H, N, D] view under which a tensor of another shape (a weight matrix, a
    [B, S, Dm] activation) draws its values: the leading dims flatten into B, H = 1,
    and the last dim splits into N x D with D its largest power-of-two divisor up to
    2**10.  Host and device draws of such a tensor both go through this view."""
    *lead, last = (int(s) for s in shape)
    rows = int(np.prod(lead)) if lead else 1
    c = 1
    while c < 1024 and last % (2 * c) == 0:
        c *= 2
    return (rows, 1, last // c, c)


def round_to_bf16_f32(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest-even), returned as float32."""
    bits = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    rounded = (bits + (np.uint32(0x7FFF) + ((bits >> np.uint32(16)) & np.uint32(1)))) \
        & np.uint32(0xFFFF0000)
    return rounded.view(np.float32)


def host_tensor(seed: int, tid: int, shape, dtype: str, n0: int = 0, b0: int = 0, h0: int = 0):
    """CPU torch tensor (bf16 or fp32) of the given slice."""
    import torch

    x = normal_f32(seed, tid, shape, n0=n0, b0=b0, h0=h0)
    if dtype == "bf16":
        return torch.from_numpy(round_to_bf16_f32(x)).to(torch.bfloat16)
    if dtype == "f32":
        return torch.from_numpy(x)
    raise ValueError(dtype)


# ----------------------------------------------------------------------------- device twin
_LIB = None
_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libe2d2_synth.so")


def _lib():
    global _LIB
    if _LIB is None:
        import torch  # noqa: F401  (binds the library to the HIP runtime torch has loaded)

        if not os.path.exists(_LIB_PATH):
            raise RuntimeError(f"{_LIB_PATH} is not built; run python -m masked_attention_amd.build")
        lib = ctypes.CDLL(_LIB_PATH)
        lib.synth_fill_normal.restype = ctypes.c_int
        lib.synth_fill_normal.argtypes = [
            ctypes.c_int, ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_longlong,
            ctypes.c_int, ctypes.c_longlong, ctypes.c_longlong, ctypes.c_longlong,
            ctypes.c_ulonglong, ctypes.c_void_p,
        ]
        _LIB = lib
    return _LIB


def device_available() -> bool:
    return os.path.exists(_LIB_PATH)


def device_fill(t, seed: int, tid: int, rows: int | None = None, n0: int = 0, row0: int = 0) -> None:
    """Fill rows [row0, row0+rows) of the contiguous CUDA tensor ``t`` = [B, H, N, D]
    with logical rows [n0, n0+rows) of tensor ``tid``, on the current stream."""
    import torch

    if t.device.type != "cuda" or not t.is_contiguous() or t.dim() != 4:
        raise ValueError("device_fill wants a contiguous 4-D CUDA tensor")
    if t.dtype == torch.bfloat16:
        dt = 1
    elif t.dtype == torch.float32:
        dt = 0
    else:
        raise ValueError(t.dtype)
    B, H, N, D = t.shape
    rows = N - row0 if rows is None else rows
    if row0 < 0 or rows < 0 or row0 + rows > N:
        raise ValueError("row range outside the tensor")
    if rows == 0 or B * H == 0:
        return
    stream = torch.cuda.current_stream(t.device).cuda_stream
    rc = _lib().synth_fill_normal(dt, ctypes.c_void_p(t.data_ptr()), B, H, N, D, row0, rows,
                                  n0, stream_key(seed, tid), ctypes.c_void_p(stream))
    if rc != 0:
        raise RuntimeError(f"synth_fill_normal failed with HIP error {rc}")


def host_draw(seed: int, tid: int, shape, dtype: str):
    """CPU tensor of any shape, drawn under draw_view(shape)."""
    return host_tensor(seed, tid, draw_view(shape), dtype).reshape(tuple(int(x) for x in shape))


def device_draw(t, seed: int, tid: int) -> None:
    """Fill the contiguous CUDA tensor ``t`` (any shape) as host_draw would."""
    if not t.is_contiguous():
        raise ValueError("device_draw wants a contiguous tensor")
    device_fill(t.view(draw_view(t.shape)), seed, tid)
