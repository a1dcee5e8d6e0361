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
* The FP8 mode runs both contractions on v_mfma_scale_f32_32x32x64_f8f6f4, has
  no packed-fp32 instructions, and its main loop writes no scratch and copies
  no register blocks.  It may reload a few loop-invariant values, at most
  eight dwords per pass of the eight-times unrolled loop; the other spills
  the compiler leaves sit in the once-per-workgroup last iteration.
"""

import os
import re
import subprocess

import pytest

from joint_sequence_attention_amd import build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _compile(tmp_path_factory, source):
    out = tmp_path_factory.mktemp("isa") / (source + ".s")
    cmd = [build.hipcc(), "--offload-arch=gfx950", "-O3", "-std=c++17", "-Xclang", "-target-feature", "-Xclang",
           "-packed-fp32-ops", "-I", os.path.join(ROOT, "include"), "-I", build.CSRC, "-S", "--cuda-device-only",
           os.path.join(build.CSRC, source), "-o", str(out)]
    proc = subprocess.run(cmd, capture_output=True, text=True)
    assert proc.returncode == 0, proc.stderr
    return out.read_text()


@pytest.fixture(scope="module")
def isa(tmp_path_factory):
    return _compile(tmp_path_factory, "attn_kernels.hip")


@pytest.fixture(scope="module")
def isa_fp8(tmp_path_factory):
    return _compile(tmp_path_factory, "attn_fp8.hip")


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


def _loop_blocks(isa_text, kernel_substring):
    """Basic blocks of the kernel's loop body (the compiler marks them 'in Loop' / 'Loop Header')."""
    start = isa_text.index(kernel_substring)
    end = isa_text.index(".Lfunc_end", start)
    blocks, cur, in_loop = [], [], False
    for ln in isa_text[start:end].split("\n"):
        if ln.startswith(".LBB") or ln.startswith("; %bb"):
            if in_loop:
                blocks.append(cur)
            cur, in_loop = [], ("Loop" in ln)
        cur.append(ln)
    if in_loop:
        blocks.append(cur)
    return blocks


def test_fp8_mfma_and_no_packed_fp32(isa_fp8):
    assert "v_mfma_scale_f32_32x32x64_f8f6f4" in isa_fp8
    assert not re.search(r"\bv_pk_(add|mul|fma)_f32\b", isa_fp8)


SKIP_INSTANCE = "attn_fwd_fp8_kernelILb1ELb0E"


@pytest.mark.parametrize("instance", ["attn_fwd_fp8_kernelILb0ELb0E", "attn_fwd_fp8_kernelILb0ELb1E", SKIP_INSTANCE])
def test_fp8_main_loop_has_no_spills_or_block_copies(isa_fp8, instance):
    # every instance (dense with the early or the late reference form, and with Skip-Softmax)
    # stores nothing to scratch in the loop and reloads at most eight dwords per pass of the
    # unrolled loop
    blocks = _loop_blocks(isa_fp8, instance)
    assert len(blocks) >= 8
    reloads = 0
    for bl in blocks:
        text = "\n".join(bl)
        assert "scratch_store" not in text
        reloads += text.count("scratch_load")
    assert reloads <= 8
    if instance == SKIP_INSTANCE:
        return
    # The dense instances, the hot path: register-to-register moves, per tile (one MFMA block of the
    # loop per tile), stay at a handful -- the start value of the score chains -- where copying an
    # accumulator block from one set of registers to another on every tile would take 16 or more.
    mfma_blocks = [bl for bl in blocks if any("v_mfma" in ln for ln in bl)]
    assert len(mfma_blocks) >= 8
    moves = 0
    for bl in mfma_blocks:
        for ln in bl:
            mv = re.match(r"\s+v_mov_b(32|64)_e32\s+v[\[\d:\]]+,\s*v", ln)
            if mv:
                moves += 2 if mv.group(1) == "64" else 1
    assert moves / len(mfma_blocks) <= 8, moves / len(mfma_blocks)
