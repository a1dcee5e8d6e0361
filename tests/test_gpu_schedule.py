"""The segment order the K/V prologues write for the attention grid.

Both attention kernels walk their grid as (query tile, head, segment rank). The rank order sits at
the end of the workspace, one int32 per segment, and the prologue fills it. It must be a
permutation of the segments by length, longest first, with equal lengths in index order.

The order changes only which workgroup starts when, never what a workgroup computes. These tests
check the order itself against a host sort of the lengths, and check that a batch full of ties and
empty segments still matches the float64 oracle.
"""
import numpy as np
import pytest

from joint_sequence_attention_amd import h3attn as H
from joint_sequence_attention_amd import workloads as wl

from helpers import Case, compare, device_to_f64, ragged_segments, say

pytestmark = pytest.mark.gpu


def _ties_segments():
    """Lengths 64, 0, 64, 300, 0, 1, 300, 65: equal pairs, two empty segments."""
    return [[wl.text(64)], [], [wl.text(64)], [wl.text(300)], [], [wl.text(1)], [wl.text(300)], [wl.text(65)]]


CASES = {
    "ties": (_ties_segments, 2),
    "ragged": (ragged_segments, 3),
    "refiner": (lambda: wl.config("refiner")["segments"], 4),
}


def _longest_first(lens):
    return sorted(range(len(lens)), key=lambda s: (-int(lens[s]), s))


@pytest.mark.parametrize("fp8", [False, True], ids=["exact", "fp8"])
@pytest.mark.parametrize("name", list(CASES))
def test_prologue_orders_segments_longest_first(gpu, name, fp8):
    import torch

    segments, heads = CASES[name]
    c = Case(segments(), heads, seed=11)
    say(f"segment order, {name} ({'fp8' if fp8 else 'exact'}): lens={c.lens.tolist()}")
    ns = len(c.lens)
    size = H.h3attn_varlen_fwd_fp8_workspace_size if fp8 else H.h3attn_varlen_fwd_workspace_size
    nbytes = size(c.N, heads, 128, ns)
    ws = H.alloc_workspace(c.N, heads, ns, fp8=fp8)
    ws.fill_(0xA5)  # stale contents must not survive
    prologue = H.h3attn_varlen_kv_prologue_fp8 if fp8 else H.h3attn_varlen_kv_prologue
    prologue(c.k, c.v, c.cu_d, c.pos_d, c.max_seqlen, ws)
    torch.cuda.synchronize()
    order = ws[nbytes - 4 * ns:nbytes].cpu().numpy().view(np.int32)
    assert order.tolist() == _longest_first(c.lens), (order.tolist(), c.lens.tolist())


def test_ties_and_empty_segments_match_the_oracle(gpu):
    c = Case(_ties_segments(), 2, seed=12)
    say(f"ties and empty segments: lens={c.lens.tolist()}")
    out, lse = c.run()
    out_ref, lse_ref = c.oracle_full()
    compare(device_to_f64(out), device_to_f64(lse), out_ref, lse_ref, label="ties")
