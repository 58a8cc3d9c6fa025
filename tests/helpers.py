"""Shared helpers of the GPU tests: seeded inputs, tolerances, visit counters."""
from __future__ import annotations

import math

import numpy as np
import torch

from synth import TensorKind, device_fill, host_tensor, tensor_id

# Tolerances (element-wise on O and LSE):
#   bf16 inputs/outputs: |got - ref| <= 2e-2;
#   fp32: relative, |got - ref| <= 1e-5 * max(|ref|, rms), where rms is the root mean
#   square of ref along its last axis (an O row, or a head's LSE row).  Elements at or
#   above the row's typical size are held to 1e-5 of their own value; an element near
#   zero (a cancelling O entry, a single-key LSE near 0) to 1e-5 of its row's size,
#   since its absolute rounding error is set by the magnitudes that were summed.
BF16_ATOL = 2e-2
F32_RTOL = 1e-5

TORCH_DT = {"bf16": torch.bfloat16, "f32": torch.float32}


def host(shape, seed, kind, dtype, step=0, block=0, n0=0, b0=0):
    """CPU tensor from the seeded generator (rows from n0, batches from b0)."""
    return host_tensor(seed, tensor_id(kind, step, block), shape, dtype, n0=n0, b0=b0)


def on_gpu(shape, seed, kind, dtype, step=0, block=0):
    """(cpu, gpu) pair of the same seeded tensor."""
    h = host(shape, seed, kind, dtype, step, block)
    return h, h.cuda()


def gpu_fill(shape, seed, kind, dtype, step=0, block=0, rows=None):
    """GPU tensor filled on the device by the generator's device twin (rows [0, rows)
    of dim 2; the rest left uninitialised when rows is given)."""
    t = torch.empty(shape, dtype=TORCH_DT[dtype], device="cuda")
    device_fill(t, seed, tensor_id(kind, step, block), rows=rows)
    return t


def counter():
    return torch.zeros(1, dtype=torch.int64, device="cuda")


def check(got, ref, dtype, what=""):
    """Element-wise tolerance check; returns the max abs error."""
    g = got.detach().double().cpu().numpy() if isinstance(got, torch.Tensor) else np.asarray(got)
    r = np.asarray(ref, dtype=np.float64)
    assert g.shape == r.shape, (what, g.shape, r.shape)
    assert np.isfinite(g).all(), f"{what}: non-finite output"
    err = np.abs(g - r)
    if dtype == "bf16":
        bad = err > BF16_ATOL
        rel = err
    else:
        rms = np.sqrt(np.mean(r * r, axis=-1, keepdims=True)) if r.ndim else np.abs(r)
        rel = err / np.maximum(np.maximum(np.abs(r), rms), 1e-300)
        bad = rel > F32_RTOL
    if bad.any():
        idx = np.unravel_index(np.argmax(rel), rel.shape)
        raise AssertionError(f"{what}: {int(bad.sum())} elements out of tolerance; max "
                             f"{'err' if dtype == 'bf16' else 'relative err'} {rel.max():.3e} "
                             f"at {idx} (got {g[idx]}, ref {r[idx]})")
    return float(rel.max())


def check_scaled(got, ref, what="", rel=2e-2):
    """Element-wise check for quantities whose rounding error scales with their row:
    |got - ref| <= rel * max(|ref|, rms of ref's row (last axis), 1e-3 * rms of ref).
    The row floor covers elements that a sum cancels to near zero, whose error still
    follows the size of the terms; the last floor covers rows that are zero in exact
    arithmetic (a query with one allowed key has dS = 0) and come out as rounding
    residue.  Returns the max scaled error."""
    g = got.detach().double().cpu().numpy() if isinstance(got, torch.Tensor) else np.asarray(got)
    r = np.asarray(ref, dtype=np.float64)
    assert g.shape == r.shape, (what, g.shape, r.shape)
    assert np.isfinite(g).all(), f"{what}: non-finite output"
    err = np.abs(g - r)
    rms = np.sqrt(np.mean(r * r, axis=-1, keepdims=True))
    floor = max(1e-3 * float(np.sqrt(np.mean(r * r))), 1e-30)
    scaled = err / np.maximum(np.maximum(np.abs(r), rms), floor)
    bad = scaled > rel
    if bad.any():
        idx = np.unravel_index(np.argmax(scaled), scaled.shape)
        raise AssertionError(f"{what}: {int(bad.sum())} elements beyond {rel} x max(|ref|, row rms); "
                             f"max {scaled.max():.3e} at {idx} (got {g[idx]}, ref {r[idx]})")
    return float(scaled.max())


def scale_of(d):
    return 1.0 / math.sqrt(d)


__all__ = ["TensorKind", "host", "on_gpu", "gpu_fill", "counter", "check", "check_scaled", "scale_of",
           "BF16_ATOL", "F32_RTOL", "TORCH_DT"]
