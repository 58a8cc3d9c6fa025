"""The build's m0 guard (masked_attention_amd.build.check_m0), without a GPU: it accepts
the LDS-DMA asm sequence on its own, and rejects a kernel that mixes it with any other
m0 use (a compiler-emitted m0 write, a builtin direct-to-LDS load, an m0-indexed
move) or with an altered asm block.  Also run over the real assembly of the two
sources that use the sequence."""
import os
import subprocess

import pytest

from masked_attention_amd import build

SEQ = (";;#ASMSTART\n\ts_mov_b32 m0, s48\n\ts_nop 0\n"
       "\tbuffer_load_dwordx4 v84, s[8:11], s12 offen lds\n\t;;#ASMEND\n")


def kernel(body, name="_Z6kernelv"):
    return f"{name}:                         ; @{name}\n{body}\t s_endpgm\n.Lfunc_end0:\n"


def test_accepts_the_sequence_alone():
    assert build.check_m0(kernel("\tv_mov_b32 v1, 0\n" + SEQ + SEQ), "t") == 1


def test_kernel_without_the_sequence_may_use_m0():
    asm = kernel("\ts_mov_b32 m0, s2\n\tbuffer_load_dword v1, s[0:3], 0 offen lds\n")
    assert build.check_m0(asm, "t") == 0


@pytest.mark.parametrize("extra", [
    "\ts_mov_b32 m0, s2\n",                                # compiler's own m0 write
    "\ts_add_i32 m0, s2, 0x1000\n",
    "\tbuffer_load_dwordx4 v1, s[0:3], 0 offen lds\n",     # builtin LDS-DMA (reads m0)
    "\tglobal_load_lds_dwordx4 v[2:3], off\n",
    "\tv_movrels_b32 v0, v1\n",                            # m0-indexed register move
    "\ts_sendmsg sendmsg(MSG_GS_DONE)\n",
])
def test_rejects_other_m0_users_beside_the_sequence(extra):
    with pytest.raises(RuntimeError):
        build.check_m0(kernel(SEQ + extra), "t")


def test_rejects_an_altered_sequence():
    bad = SEQ.replace("\ts_nop 0\n", "")
    with pytest.raises(RuntimeError):
        build.check_m0(kernel(bad), "t")


def test_other_kernels_in_the_file_are_independent():
    a = kernel(SEQ, "_Z1av")
    b = kernel("\ts_mov_b32 m0, s2\n\tbuffer_load_dword v1, s[0:3], 0 offen lds\n", "_Z1bv")
    assert build.check_m0(a + b, "t") == 1


@pytest.mark.parametrize("src,kernels", [("attn_bwd.hip", 3), ("linear.hip", 2)])
def test_real_assembly_passes(tmp_path, src, kernels):
    out = os.path.join(tmp_path, "k.s")
    cmd = [build.HIPCC, *build.COMMON, "--cuda-device-only", "-S", os.path.join(build.CSRC, src),
           "-o", out]
    subprocess.run(cmd, check=True, capture_output=True)
    with open(out) as f:
        assert build.check_m0(f.read(), src) == kernels
