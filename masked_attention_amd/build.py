"""Build of the HIP libraries for gfx950 (in-tree, explicit hipcc command lines).

``libe2d2_attn.so`` is the product: the C-ABI library declared in
include/e2d2_attn.h.  ``synth/libe2d2_synth.so`` is the device twin of the input
generator used by the tests and the bench.  Sources compile in parallel to objects
under ``_build/`` and link into the shared libraries next to their Python wrappers.
"""
from __future__ import annotations

import concurrent.futures
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "masked_attention_amd")
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libe2d2_attn.so")
SYNTH_SRC = os.path.join(ROOT, "synth", "synth_fill.hip")
SYNTH_LIB = os.path.join(ROOT, "synth", "libe2d2_synth.so")
BUILD_DIR = os.path.join(ROOT, "_build")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
# Packed-fp32 VALU forms are disabled for all device code.
COMMON = ["--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-Wno-unused-command-line-argument"]

SOURCES = ["api.hip", "attn_train.hip", "attn_denoise.hip", "attn_bwd.hip", "linear.hip"]


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in r.stderr.splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError("command failed:\n" + " ".join(cmd) + "\n" + err)
    return err


def build(verbose: bool = False) -> None:
    """Compile both libraries (always; never skips on existing outputs)."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    jobs = []
    for src in SOURCES:
        obj = os.path.join(BUILD_DIR, src.replace(".hip", ".o"))
        jobs.append((obj, [HIPCC, *COMMON, "-c", os.path.join(CSRC, src), "-o", obj]))
    synth_obj = os.path.join(BUILD_DIR, "synth_fill.o")
    jobs.append((synth_obj, [HIPCC, *COMMON, "-c", SYNTH_SRC, "-o", synth_obj]))
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(jobs))) as ex:
        futs = [ex.submit(_run, cmd) for _, cmd in jobs]
        for f in futs:
            msg = f.result()
            if verbose and msg:
                print(msg, file=sys.stderr)
    objs = [o for o, _ in jobs[:-1]]
    tmp = LIB + ".tmp"
    _run([HIPCC, *COMMON, "-shared", *objs, "-o", tmp])
    os.replace(tmp, LIB)
    tmp = SYNTH_LIB + ".tmp"
    _run([HIPCC, *COMMON, "-shared", synth_obj, "-o", tmp])
    os.replace(tmp, SYNTH_LIB)


if __name__ == "__main__":
    build(verbose=True)
    print("built", LIB, SYNTH_LIB)
