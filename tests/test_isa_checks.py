"""Checks on the gfx950 assembly the attention kernels compile to (CPU only).

hipcc cross-compiles here, so properties of the generated code can be checked
without a GPU:

* The score contraction runs on v_mfma_f32_32x32x16_f16 and the value
  contraction on v_mfma_f32_32x32x16_bf16.
* No vector-register spills, no scratch memory and no packed-fp32
  instructions.  (Scalar spills go to vector-register lanes, not memory.)
* If a v_dot2 chain appears, no accumulator is fed the same source register
  twice in a row: this toolchain miscompiles a dot2 whose source is an element
  of a 128-bit vector (it reads element 0 every time).
"""

import os
import re
import subprocess

import pytest

from joint_sequence_attention_amd import build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def isa(tmp_path_factory):
    out = tmp_path_factory.mktemp("isa") / "attn.s"
    cmd = [build.hipcc(), "--offload-arch=gfx950", "-O3", "-std=c++17", "-Xclang", "-target-feature", "-Xclang",
           "-packed-fp32-ops", "-I", os.path.join(ROOT, "include"), "-I", build.CSRC, "-S", "--cuda-device-only",
           os.path.join(build.CSRC, "attn_kernels.hip"), "-o", str(out)]
    proc = subprocess.run(cmd, capture_output=True, text=True)
    assert proc.returncode == 0, proc.stderr
    return out.read_text()


def test_mfma_instructions(isa):
    assert "v_mfma_f32_32x32x16_f16" in isa
    assert "v_mfma_f32_32x32x16_bf16" in isa


def test_dot2_chains_read_distinct_sources(isa):
    ops = re.findall(r"v_dot2c_f32_bf16_e32\s+(v\d+),\s*([^,\s]+),\s*(v\d+)", isa)
    for (acc0, _, src0), (acc1, _, src1) in zip(ops, ops[1:]):
        assert not (acc0 == acc1 and src0 == src1), f"dot2 chain on {acc0} reads {src0} twice in a row"


def test_no_spills_and_no_packed_fp32(isa):
    counts = re.findall(r"\.vgpr_spill_count:\s+(\d+)", isa)
    assert counts and all(int(c) == 0 for c in counts)
    scratch = re.findall(r"\.private_segment_fixed_size:\s+(\d+)", isa)
    assert scratch and all(int(c) == 0 for c in scratch)
    assert not re.search(r"\bv_pk_(add|mul|fma)_f32\b", isa)
