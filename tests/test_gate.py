"""Skip-Softmax timestep gate: the oracle against the pages' worked example, the C ABI against the oracle.

CPU only: h3attn_skip_gate is host logic and makes no device call.
"""

import json
import os

import numpy as np
import pytest

import oracle
from joint_sequence_attention_amd import h3attn as H

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "skip_gate_counts.json")


@pytest.fixture(scope="module")
def golden():
    with open(GOLDEN) as f:
        return json.load(f)


def _dense_prefix(gate, sigmas):
    dense = [gate(s) == 0.0 for s in sigmas]
    n = 0
    while n < len(dense) and dense[n]:
        n += 1
    assert not any(dense[n:]), "the dense steps form a prefix"
    return n


def test_flow_shift_closed_forms():
    s = np.linspace(0, 1, 101)
    assert oracle.flow_shift(0.0, 12.0) == 0.0 and oracle.flow_shift(1.0, 12.0) == 1.0
    assert np.allclose(oracle.flow_shift(s, 1.0), s, rtol=0, atol=0)            # shift 1: identity
    assert np.all(np.diff(oracle.flow_shift(s, 12.0)) > 0)                       # order kept
    # sigma = 1/2 -> s / (s + 1); the shift inverts as 1/s
    assert oracle.flow_shift(0.5, 12.0) == pytest.approx(12.0 / 13.0, rel=1e-15)
    assert np.allclose(oracle.flow_shift(oracle.flow_shift(s, 12.0), 1.0 / 12.0), s, rtol=0, atol=1e-14)


def test_oracle_gate_matches_worked_example(golden):
    sig = oracle.forward_sigmas(golden["steps"], golden["shift"])
    assert len(sig) == golden["forwards"]
    for cut, n in golden["dense_prefix"].items():
        assert _dense_prefix(lambda s: oracle.skip_threshold_at(0.05, float(cut), s), sig) == n, cut


def test_abi_gate_matches_worked_example(golden):
    sig = oracle.forward_sigmas(golden["steps"], golden["shift"])
    for cut, n in golden["dense_prefix"].items():
        assert _dense_prefix(lambda s: H.h3attn_skip_gate(0.05, float(cut), s), sig) == n, cut


def test_abi_gate_equals_oracle():
    rng = np.random.default_rng(5)
    sig = np.concatenate([rng.uniform(0, 1, 200), [0.0, 1.0, 0.97, np.float32(0.97)]]).astype(np.float32)
    for thr in (0.0, 0.05, 0.5):
        for cut in (0.0, 0.5, 0.97, 1.0):
            for s in sig:
                # both sides compare the float32 values the C function receives
                want = oracle.skip_threshold_at(float(np.float32(thr)), float(np.float32(cut)), float(s))
                assert H.h3attn_skip_gate(thr, cut, float(s)) == pytest.approx(want, rel=0, abs=0)


@pytest.mark.parametrize("args", [(-0.1, 0.97, 0.5), (1.0, 0.97, 0.5), (float("nan"), 0.97, 0.5),
                                  (0.05, float("nan"), 0.5), (0.05, 0.97, float("nan"))])
def test_abi_gate_rejects_bad_arguments(args):
    with pytest.raises(H.H3AttnError):
        H.h3attn_skip_gate(*args)
