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
from helpers import FP8_EXACT_REL, compare, compare_fp8, row_relative_error
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
    # the FP8 mode's own result (P rounded) and its quantized reference (P unrounded, with scales)
    o8, l8 = oracle.sage_attention_rows(q, k, v, cu, pos, rows)
    o8u, l8u, es = oracle.sage_attention_rows(q, k, v, cu, pos, rows, quantize_p=False, error_scales=True)
    return o, l, o_perm, (o8, l8, o8u, l8u, es)


def test_rounded_oracle_output_passes(rows_1344):
    o, l, _, _ = rows_1344
    stats = compare(_bf16_round(o), l.astype(np.float32).astype(np.float64), o, l, label="bf16-rounded oracle")
    assert stats["out_rel_max"] < 5e-3


def test_zero_output_fails(rows_1344):
    o, l, _, _ = rows_1344
    assert row_relative_error(np.zeros_like(o), o).min() == pytest.approx(1.0)
    with pytest.raises(AssertionError):
        compare(np.zeros_like(o), l, o, l, label="zeros")


def test_output_from_permuted_values_fails(rows_1344):
    o, l, o_perm, _ = rows_1344
    rel = row_relative_error(o_perm, o)
    assert rel.min() > 0.5
    with pytest.raises(AssertionError):
        compare(_bf16_round(o_perm), l, o, l, label="permuted values")


def _fp8_compare(out, lse, rows_1344):
    o, l, _, (o8, l8, o8u, l8u, es) = rows_1344
    return compare_fp8(out, lse, o8u, l8u, es, o, l, label="fp8 bar")


def test_fp8_mode_output_passes_its_bars(rows_1344):
    # the FP8 mode's own float64 result (P rounded to e4m3, bf16 output rounding) passes both the
    # quantized-oracle bars and the quality bar against exact softmax, well inside the latter
    _, _, _, (o8, l8, _, _, _) = rows_1344
    stats = _fp8_compare(_bf16_round(o8), l8.astype(np.float32).astype(np.float64), rows_1344)
    assert stats["exact_rel_max"] < FP8_EXACT_REL / 2


def test_fp8_bar_rejects_zero_and_permuted_values(rows_1344):
    o, l, o_perm, (o8, l8, _, _, _) = rows_1344
    with pytest.raises(AssertionError):
        _fp8_compare(np.zeros_like(o8), l8, rows_1344)
    with pytest.raises(AssertionError):
        _fp8_compare(_bf16_round(o_perm), l8, rows_1344)
    # and on its own the relative quality bar rejects both, where the absolute ones would not
    assert row_relative_error(np.zeros_like(o8), o).min() > FP8_EXACT_REL
    assert row_relative_error(o_perm, o).min() > FP8_EXACT_REL
    assert np.abs(o).max() < 0.5 and np.abs(o).mean() < 2e-2
