"""The parity bars themselves, on the CPU: they accept a correctly rounded result and reject wrong ones.

At the 1344x768 shape (130,048 keys per row) a row's output is an average of
many values and is small, so an absolute bar alone says little there.  These
tests take oracle rows of that workload and show that the comparison the GPU
tests use passes the oracle's own output rounded to bf16, and fails an
all-zero output and an output formed with the values of other keys (V rows
permuted inside the segment).
"""

import numpy as np
import pytest

import oracle
from helpers import compare, row_relative_error
from joint_sequence_attention_amd import workloads as wl


def _bf16_round(x):
    return wl.bf16_bits_to_f32(wl._round_bf16_bits(np.asarray(x, dtype=np.float32))).astype(np.float64)


@pytest.fixture(scope="module")
def rows_1344():
    cfg = wl.config("1344x768")
    cu, pos = oracle.layout(cfg["segments"])
    N, H = int(cu[-1]), cfg["heads"]
    qb, kb, vb = wl.random_qkv(N, H, cfg["seed"])
    q, k, v = (wl.bf16_bits_to_f32(b).astype(np.float64) for b in (qb, kb, vb))
    rows = np.sort(np.random.default_rng(5).choice(N, size=6, replace=False))
    o, l = oracle.attention_rows(q, k, v, cu, pos, rows)
    perm = np.random.default_rng(6).permutation(N)
    o_perm, _ = oracle.attention_rows(q, k, v[perm], cu, pos, rows)
    return o, l, o_perm


def test_rounded_oracle_output_passes(rows_1344):
    o, l, _ = rows_1344
    stats = compare(_bf16_round(o), l.astype(np.float32).astype(np.float64), o, l, label="bf16-rounded oracle")
    assert stats["out_rel_max"] < 5e-3


def test_zero_output_fails(rows_1344):
    o, l, _ = rows_1344
    assert row_relative_error(np.zeros_like(o), o).min() == pytest.approx(1.0)
    with pytest.raises(AssertionError):
        compare(np.zeros_like(o), l, o, l, label="zeros")


def test_output_from_permuted_values_fails(rows_1344):
    o, l, o_perm = rows_1344
    rel = row_relative_error(o_perm, o)
    assert rel.min() > 0.5
    with pytest.raises(AssertionError):
        compare(_bf16_round(o_perm), l, o, l, label="permuted values")
