"""Seeded synthetic inputs shared by the tests, the bench and the smoke check.

This package draws the i.i.d. N(0, 1) tensors that stand in for the queries, keys
and values of the workloads.  It holds no attention arithmetic: neither the CPU
oracle nor the HIP library is imported here, and both consume what it produces.

Every value is a pure function of (seed, tensor id, b, h, row, col), so any slice
of a tensor can be regenerated on the host without materialising the rest, and the
device fill kernel in ``synth_fill.hip`` reproduces the host values bit for bit.
"""
from .gen import (  # noqa: F401
    TensorKind,
    tensor_id,
    normal_f32,
    round_to_bf16_f32,
    host_tensor,
    device_fill,
    device_available,
    draw_view,
    host_draw,
    device_draw,
)
