"""The no-allocation entry point (h3attn_varlen_fwd_noalloc) through the C ABI, on the GPU.

It runs the exact path's kernels on the library's own scratch array, so its
results must equal h3attn_varlen_fwd's (with a caller workspace) bit for bit.
Two calls in a row, the second on a smaller input, check that what the first
left in the shared array does not leak into the second.
"""

import numpy as np
import pytest

from helpers import Case, bf16_bits, compare, device_to_f64, ragged_segments, say
from joint_sequence_attention_amd import h3attn as H
from joint_sequence_attention_amd import workloads as wl

pytestmark = pytest.mark.gpu


def _same(c, label):
    import torch
    out_n, lse_n = H.h3attn_varlen_fwd_noalloc(c.q, c.k, c.v, c.cu_d, c.pos_d, c.max_seqlen)
    out_w, lse_w = H.h3attn_varlen_fwd(c.q, c.k, c.v, c.cu_d, c.pos_d, c.max_seqlen)
    torch.cuda.synchronize()
    say(f"noalloc {label}: N={c.N} H={c.heads} segments={len(c.lens)}")
    assert np.array_equal(bf16_bits(out_n), bf16_bits(out_w))
    assert np.array_equal(lse_n.cpu().numpy(), lse_w.cpu().numpy())
    return out_n, lse_n


def test_noalloc_equals_workspace_call_twice_second_smaller(gpu):
    cfg = wl.config("480p")                       # 7,936 tokens x 24 heads: 98 MB of the 128 MiB array
    big = Case(cfg["segments"], cfg["heads"], cfg["seed"])
    _same(big, "480p")
    small = Case(ragged_segments(), 3, 77)        # then a smaller, ragged batch on the same array
    out, lse = _same(small, "ragged")
    o_ref, l_ref = small.oracle_full()
    compare(device_to_f64(out), device_to_f64(lse), o_ref, l_ref, label="noalloc ragged vs oracle")


def test_noalloc_refuses_a_call_beyond_its_array(gpu):
    cfg = wl.config("1344x768")                   # 333 MB of workspace: refused before any launch
    c = Case(cfg["segments"], cfg["heads"], cfg["seed"])
    with pytest.raises(H.H3AttnError) as err:
        H.h3attn_varlen_fwd_noalloc(c.q, c.k, c.v, c.cu_d, c.pos_d, c.max_seqlen)
    assert err.value.status == H.H3ATTN_ERR_UNSUPPORTED and "128 MiB" in str(err.value)
