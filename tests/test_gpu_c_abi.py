"""The C ABI from a plain C++ program (needs an MI355X): tests/native/abi_c_caller.cpp
allocates with hipMalloc, calls the library on the null stream with no Python or torch
in the process, and checks argument validation, closed forms of the encoder, decoder
and denoising attentions (all-zero queries: each row is the mean of the value rows its
mask allows, LSE = ln(count)) and the bitwise KV-cache append.  The program is built
with the host compiler against include/e2d2_attn.h and the in-tree library."""
import os
import shutil
import subprocess

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "tests", "native", "abi_c_caller.cpp")
LIB_DIR = os.path.join(ROOT, "masked_attention_amd")


def test_c_abi_from_a_plain_cpp_caller(tmp_path):
    cxx = shutil.which("g++") or shutil.which("c++")
    if cxx is None:
        pytest.skip("no host C++ compiler")
    if not os.path.exists(os.path.join(LIB_DIR, "libe2d2_attn.so")):
        raise RuntimeError("libe2d2_attn.so is not built: run python -m masked_attention_amd.build")
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    exe = str(tmp_path / "abi_c_caller")
    subprocess.run([cxx, "-std=c++17", "-O1", "-D__HIP_PLATFORM_AMD__", f"-I{rocm}/include",
                    "-I", os.path.join(ROOT, "include"), SRC, f"-L{LIB_DIR}", "-le2d2_attn",
                    f"-L{rocm}/lib", "-lamdhip64", f"-Wl,-rpath,{LIB_DIR}:{rocm}/lib", "-o", exe],
                   check=True)
    run = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    print(run.stdout)
    assert run.returncode == 0, run.stdout + run.stderr
    assert " 0 failures" in run.stdout, run.stdout
