"""The closed-form mask intervals of the kernels' schedule (csrc/schedule.h), built
into a small host program, against the oracle's explicit masks: for every query row,
the allowed keys of each source; for every key, the query rows that allow it (the
backward pass walks these); and the union / common rows of key spans.  CPU only."""
import os
import shutil
import subprocess

import numpy as np
import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "masked_attention_amd", "csrc")
PROBE = os.path.join(ROOT, "tests", "native", "schedule_probe.cpp")


@pytest.fixture(scope="module")
def probe(tmp_path_factory):
    cxx = shutil.which("g++") or shutil.which("c++")
    if cxx is None:
        pytest.skip("no host C++ compiler")
    exe = str(tmp_path_factory.mktemp("probe") / "schedule_probe")
    subprocess.run([cxx, "-std=c++17", "-O1", "-I", CSRC, PROBE, "-o", exe], check=True)
    return exe


def _run(exe, kind, src, L, S):
    out = subprocess.run([exe, str(kind), str(src), str(L), str(S)], check=True,
                         capture_output=True, text=True).stdout.split("\n")
    rows, cols, spans = {}, {}, []
    for line in out:
        f = line.split()
        if not f:
            continue
        if f[0] == "row":
            rows[int(f[1])] = (int(f[2]), int(f[3]))
        elif f[0] == "col":
            cols[int(f[1])] = (int(f[2]), int(f[3]))
        else:
            spans.append(tuple(int(x) for x in f[1:]))
    return rows, cols, spans


def _as_interval(mask_vec):
    idx = np.flatnonzero(mask_vec)
    return (int(idx[0]), int(idx[-1]) + 1) if len(idx) else None


KINDS = [(0, 0), (1, 0), (1, 1)]  # (ENC, clean), (DEC, clean), (DEC, noised)


@pytest.mark.parametrize("L,S", [(64, 8), (37, 5), (16, 1), (20, 20), (33, 16), (7, 3)])
@pytest.mark.parametrize("kind,src", KINDS)
def test_intervals_match_oracle_masks(probe, kind, src, L, S):
    if kind == 0:
        m = oracle.encoder_mask(L, S)
    else:
        full = oracle.decoder_mask(L, S)
        m = full[:, :L] if src == 0 else full[:, L:]
    rows, cols, spans = _run(probe, kind, src, L, S)
    for i in range(L):
        want = _as_interval(m[i])
        lo, hi = rows[i]
        assert (want is None and hi <= lo) or want == (lo, hi), ("row", i, want, (lo, hi))
    for j in range(L):
        want = _as_interval(m[:, j])
        lo, hi = cols[j]
        assert (want is None and hi <= lo) or want == (lo, hi), ("col", j, want, (lo, hi))
    for k0, k1, ulo, uhi, clo, chi in spans:
        anyk = m[:, k0:k1 + 1].any(axis=1)
        allk = m[:, k0:k1 + 1].all(axis=1)
        u = _as_interval(anyk)
        c = _as_interval(allk)
        assert (u is None and uhi <= ulo) or u == (ulo, uhi), ("union", k0, k1)
        assert (c is None and chi <= clo) or c == (clo, chi), ("common", k0, k1)
