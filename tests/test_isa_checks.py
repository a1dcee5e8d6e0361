"""Checks on the gfx950 assembly the attention kernels compile to (CPU only).

hipcc cross-compiles here, so properties of the generated code can be checked
without a GPU:

* The row sums use v_dot2c_f32_bf16 over packed bf16 probabilities.  This
  toolchain miscompiles a dot2 whose source is an element of a 128-bit vector:
  it reads element 0 for every call, so one pair is counted four times.  The
  kernel avoids that form; this test fails if such a chain (the same
  accumulator fed the same source register twice in a row) reappears.
* No scratch (register spills) and no packed-fp32 instructions.
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


def test_dot2_chains_read_distinct_sources(isa):
    ops = re.findall(r"v_dot2c_f32_bf16_e32\s+(v\d+),\s*([^,\s]+),\s*(v\d+)", isa)
    assert ops, "expected dot2 row sums in the attention kernel"
    for (acc0, _, src0), (acc1, _, src1) in zip(ops, ops[1:]):
        assert not (acc0 == acc1 and src0 == src1), f"dot2 chain on {acc0} reads {src0} twice in a row"


def test_no_spills_and_no_packed_fp32(isa):
    for m in re.finditer(r"\.(?:vgpr|sgpr)_spill_count:\s+(\d+)", isa):
        assert int(m.group(1)) == 0
    assert not re.search(r"\bv_pk_(add|mul|fma)_f32\b", isa)
