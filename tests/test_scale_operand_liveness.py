"""Every scaled MFMA in the built kernels keeps its E8M0 scale registers until the instruction is
known to be complete (CPU: compiles the kernel sources to gfx950 assembly with the library's own
flags and walks it; tests/hw/scale_hazard.py states the hazard and the rule).  The checker is pinned
on hand-written assembly first: one sequence that overwrites a scale register right after the
instruction, and the same sequence with the result read before the write."""
import functools
import os
import re
import subprocess
import tempfile

import pytest

from hw import scale_hazard as sh
from mxfp8_block_scaled_flash_amd import build as bld

BAD = """
  v_mfma_scale_f32_32x32x64_f8f6f4 v[0:15], v[16:23], v[24:31], v[0:15], v40, v41 op_sel_hi:[0,0,0]
  v_mov_b32_e32 v40, 0
  v_add_f32_e32 v50, v0, v1
"""
GOOD = """
  v_mfma_scale_f32_32x32x64_f8f6f4 v[0:15], v[16:23], v[24:31], v[0:15], v40, v41 op_sel_hi:[0,0,0]
  v_mfma_scale_f32_32x32x64_f8f6f4 v[60:75], v[16:23], v[24:31], v[60:75], v42, v43 op_sel_hi:[0,0,0]
  s_nop 7
  v_add_f32_e32 v50, v60, v61
  v_mov_b32_e32 v40, 0
"""


def test_checker_flags_an_early_write_and_clears_a_read_first():
    assert len(sh.violations(BAD)) == 1
    assert sh.violations(GOOD) == []          # a later MFMA's result read: the first one is done too
    assert sh.violations(BAD.replace("v40, 0", "v44, 0")) == []


@functools.lru_cache(maxsize=None)
def _device_asm(src):
    path = os.path.join(bld.CSRC, src)
    with tempfile.TemporaryDirectory() as d:
        out = os.path.join(d, "k.s")
        cmd = [bld.HIPCC, *[f for f in bld.FLAGS if f != "-fPIC"], *bld.FILE_FLAGS.get(src, []), "--cuda-device-only",
               "-S", path, "-o", out]
        r = subprocess.run(cmd, capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-2000:]
        return open(out).read()


@pytest.mark.parametrize("src", ["attn_fwd.hip", "attn_bwd.hip", "gemm_quant.hip"])
def test_kernels_keep_scale_registers_until_complete(src):
    asm = _device_asm(src)
    assert "v_mfma_scale" in asm
    bad = sh.violations(asm)
    assert not bad, bad[:5]


@pytest.mark.parametrize("src", ["attn_fwd.hip", "gemm_quant.hip"])
def test_forward_and_gemm_kernels_use_no_scratch_memory(src):
    """The forward and GEMM kernels keep everything in registers and LDS: a private segment there
    means spilled registers or an array the compiler could not keep in registers, each access a
    memory round trip inside the main loop."""
    asm = _device_asm(src)
    sizes = re.findall(r"\.name:\s+(\S+)\s+\.private_segment_fixed_size:\s+(\d+)", asm)
    assert sizes, "no kernel metadata found"
    used = [(n, int(b)) for n, b in sizes if int(b) != 0]
    assert not used, used
