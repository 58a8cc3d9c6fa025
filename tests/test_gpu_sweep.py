"""Seeded random shape sweep of the GPU calls against the fp64 oracle (needs an MI355X).

The hand-picked cases in the other files cover each edge on purpose; this sweep draws
shapes at random (fixed seed, so the list is the same on every run) to reach the
combinations nobody picked: odd and ragged block sizes, lengths that are not tile
multiples, one to eight query heads per KV head, empty and ragged caches, both dtypes,
with and without the encoder, per-sequence cache lengths from empty to full.  Each case
runs through the C-ABI binding and is checked element by element with the tolerances of
the other GPU tests.
"""
import os

import numpy as np
import pytest

import oracle
from helpers import scale_of
from test_gpu_bwd import NAMES, check_grad, inputs as bwd_inputs, run_gpu as bwd_run
from test_gpu_denoise import _denoise_case
from test_gpu_train import _train_case
from test_gpu_varlen import _varlen_case

pytestmark = pytest.mark.gpu

_rng = np.random.RandomState(0xE2D25EED)


def _block(L):
    """A block size for length L: small odd/even sizes, tile-sized ones, or L itself."""
    choices = [1, 2, 3, 5, 7, 8, 12, 16, 31, 32, 33, 64, L]
    return int(min(L, choices[_rng.randint(len(choices))]))


def _train_cases(n):
    out = []
    for _ in range(n):
        Hkv = int(_rng.choice([1, 2]))
        Hq = Hkv * int(_rng.choice([1, 2, 4]))
        L = int(_rng.randint(1, 321))
        out.append((int(_rng.choice([1, 2])), Hq, Hkv, L, _block(L), int(_rng.choice([32, 64, 128])),
                    str(_rng.choice(["bf16", "f32"])), bool(_rng.rand() < 0.7)))
    return out


def _denoise_cases(n):
    out = []
    for _ in range(n):
        Hkv = int(_rng.choice([1, 2]))
        Hq = Hkv * int(_rng.choice([1, 2, 4, 8]))
        S = int(_rng.randint(1, 81))
        C = 0 if _rng.rand() < 0.15 else int(_rng.randint(1, 2001))
        cap = C + S + int(_rng.randint(0, 40))
        out.append((int(_rng.choice([1, 2, 3])), Hq, Hkv, S, int(_rng.choice([32, 64, 128])), C, cap,
                    str(_rng.choice(["bf16", "f32"]))))
    return out


def _bwd_cases(n):
    out = []
    for _ in range(n):
        Hkv = int(_rng.choice([1, 2]))
        Hq = Hkv * int(_rng.choice([1, 2]))
        L = int(_rng.randint(2, 261))
        out.append((int(_rng.choice([1, 2])), Hq, Hkv, L, _block(L), int(_rng.choice([32, 64, 128])),
                    bool(_rng.rand() < 0.6)))
    return out


def _varlen_cases(n):
    out = []
    for _ in range(n):
        Hkv = int(_rng.choice([1, 2]))
        Hq = Hkv * int(_rng.choice([1, 2, 4, 8]))
        B = int(_rng.randint(1, 7))
        S = int(_rng.randint(1, 49))
        max_len = int(_rng.randint(1, 1500))
        lens = []
        for _ in range(B):
            u = _rng.rand()
            lens.append(0 if u < 0.15 else max_len if u < 0.3 else int(_rng.randint(1, max_len + 1)))
        cap = max_len + S + int(_rng.randint(0, 20))
        out.append((B, Hq, Hkv, S, int(_rng.choice([32, 64, 128])), lens, max_len, cap))
    return out


# E2D2_SWEEP_SCALE=k draws k times as many cases (the first ones stay the same only for
# k = 1: the draws interleave); the default keeps the suite to a few seconds.
_K = max(1, int(os.environ.get("E2D2_SWEEP_SCALE", "1")))
TRAIN = _train_cases(16 * _K)
DENOISE = _denoise_cases(16 * _K)
BWD = _bwd_cases(10 * _K)
VARLEN = _varlen_cases(10 * _K)


@pytest.mark.parametrize("i", range(len(TRAIN)))
def test_sweep_training_forward(i):
    B, Hq, Hkv, L, S, d, dtype, with_enc = TRAIN[i]
    _train_case(B, Hq, Hkv, L, S, d, dtype, 0xE2D25000 + i, with_enc=with_enc)


@pytest.mark.parametrize("i", range(len(DENOISE)))
def test_sweep_denoise_step(i):
    B, Hq, Hkv, S, d, C, cap, dtype = DENOISE[i]
    _denoise_case(B, Hq, Hkv, S, d, C, cap, dtype, 0xE2D25100 + i)


@pytest.mark.parametrize("i", range(len(BWD)))
def test_sweep_training_backward(i):
    B, Hq, Hkv, L, S, d, with_enc = BWD[i]
    ins = bwd_inputs(B, Hq, Hkv, L, d, 0xE2D25200 + i)
    got = bwd_run(ins, S, with_enc)
    ref = oracle.train_bwd(*ins[:5], S, scale_of(d), ins[6], q_enc=ins[5] if with_enc else None,
                           do_enc=ins[7] if with_enc else None)
    for name, g, r in zip(NAMES, got, ref):
        check_grad(g, r, f"{name} (case {BWD[i]})")


@pytest.mark.parametrize("i", range(len(VARLEN)))
def test_sweep_denoise_step_per_sequence_lengths(i):
    B, Hq, Hkv, S, d, lens, max_len, cap = VARLEN[i]
    _varlen_case(B, Hq, Hkv, S, d, lens, max_len, cap, 0xE2D25300 + i)
