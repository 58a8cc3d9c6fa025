"""Shared helpers of the GPU tests: seeded inputs, tolerances, visit counters."""
from __future__ import annotations

import math

import numpy as np
import torch

from synth import TensorKind, device_fill, host_tensor, tensor_id

# Tolerances (element-wise on O and LSE):
#   bf16 inputs/outputs: |got - ref| <= 2e-2;
#   fp32: |got - ref| <= 1e-5 * max(1, |ref|).
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
    else:
        bad = err > F32_RTOL * np.maximum(1.0, np.abs(r))
    if bad.any():
        idx = np.unravel_index(np.argmax(err), err.shape)
        raise AssertionError(f"{what}: {int(bad.sum())} elements out of tolerance; max err "
                             f"{err.max():.3e} at {idx} (got {g[idx]}, ref {r[idx]})")
    return float(err.max())


def scale_of(d):
    return 1.0 / math.sqrt(d)


__all__ = ["TensorKind", "host", "on_gpu", "gpu_fill", "counter", "check", "scale_of",
           "BF16_ATOL", "F32_RTOL", "TORCH_DT"]
