"""Build of the HIP libraries for gfx950 (in-tree, explicit hipcc command lines).

``libe2d2_attn.so`` is the product: the C-ABI library declared in
include/e2d2_attn.h.  ``synth/libe2d2_synth.so`` is the device twin of the input
generator used by the tests and the bench.  Sources compile in parallel to objects
under ``_build/`` and link into the shared libraries next to their Python wrappers.
"""
from __future__ import annotations

import concurrent.futures
import os
import re
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


# ---- m0 guard.  dma_lds16 / dma_lds4 (device_common.h) write m0, the LDS base of a
# buffer_load ... lds, from inline asm, which the compiler cannot be told about (it
# reserves m0).  That is sound only in a kernel where the compiler itself emits no m0
# access.  Every kernel's generated AMD assembly is checked: in a kernel holding such an
# asm block, each m0-writing block must be exactly the helper's sequence, and no other
# instruction may name m0 or read it implicitly.
_ASM_BLOCK = re.compile(r";;#ASMSTART\n(.*?)\n\s*;;#ASMEND", re.S)
_DMA_SEQ = re.compile(r"\s*s_mov_b32 m0, s\d+\s*\n\s*s_nop 0\s*\n"
                      r"\s*buffer_load_dword(x4)? v\d+, s\[\d+:\d+\], s\d+ offen lds\s*$")
# instructions that read m0 without naming it
_M0_IMPLICIT = re.compile(r"\b(s_sendmsg\w*|s_movrel\w*|v_movrel\w*|ds_gws\w*|ds_append|"
                          r"ds_consume|ds_\w*addtid\w*|v_interp\w*|global_load_lds\w*)\b|"
                          r"\slds\s*$")


def check_m0(asm: str, what: str) -> int:
    """Raise when a kernel of ``asm`` mixes the asm m0 writes with any other m0 use.
    Returns the number of kernels holding the asm sequence."""
    n = 0
    starts = [mm.start() for mm in re.finditer(r"^\S+:\s*;\s*@", asm, re.M)] + [len(asm)]
    for a, b in zip(starts, starts[1:]):
        body = asm[a:b]
        name = body.split(":", 1)[0]
        blocks = [x for x in _ASM_BLOCK.findall(body) if re.search(r"\bm0\b", x)]
        if not blocks:
            continue
        n += 1
        for x in blocks:
            if not _DMA_SEQ.fullmatch(x):
                raise RuntimeError(f"{what}: {name}: unexpected m0 asm block:\n{x}")
        for line in _ASM_BLOCK.sub("", body).splitlines():
            code = line.split(";", 1)[0]
            if re.search(r"\bm0\b", code) or _M0_IMPLICIT.search(code):
                raise RuntimeError(f"{what}: {name} writes m0 from asm and also has the "
                                   f"compiler's m0 use: {line.strip()}")
    return n


def build(verbose: bool = False) -> None:
    """Compile both libraries (always; never skips on existing outputs)."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    jobs = []
    for src in SOURCES:
        obj = os.path.join(BUILD_DIR, src.replace(".hip", ".o"))
        jobs.append((obj, [HIPCC, *COMMON, "-c", os.path.join(CSRC, src), "-o", obj]))
    synth_obj = os.path.join(BUILD_DIR, "synth_fill.o")
    jobs.append((synth_obj, [HIPCC, *COMMON, "-c", SYNTH_SRC, "-o", synth_obj]))
    asm_jobs = []
    for src in SOURCES:
        out = os.path.join(BUILD_DIR, src.replace(".hip", ".s"))
        asm_jobs.append((out, [HIPCC, *COMMON, "--cuda-device-only", "-S",
                               os.path.join(CSRC, src), "-o", out]))
    with concurrent.futures.ThreadPoolExecutor(max_workers=8) as ex:
        futs = [ex.submit(_run, cmd) for _, cmd in jobs + asm_jobs]
        for f in futs:
            msg = f.result()
            if verbose and msg:
                print(msg, file=sys.stderr)
    n_dma = 0
    for out, _ in asm_jobs:
        with open(out) as f:
            n_dma += check_m0(f.read(), os.path.basename(out))
    if n_dma == 0:
        raise RuntimeError("m0 guard found no kernel with the asm LDS-DMA sequence; "
                           "the assembly format it parses may have changed")
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
