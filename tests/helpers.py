"""Shared helpers for the GPU parity tests: inputs onto the device, oracle on the host, comparisons."""

from __future__ import annotations

import sys

import numpy as np

import oracle
from joint_sequence_attention_amd import h3attn as H
from joint_sequence_attention_amd import workloads as wl

# Parity bar for bf16-in / fp32-accumulate attention against the float64 oracle.
OUT_MAX_ABS = 1e-2
OUT_MEAN_ABS = 1e-3
LSE_MAX_ABS = 1e-3
# Per (row, head): |out - out_ref|_2 <= OUT_REL_L2 * |out_ref|_2.  On long segments a row's output
# is an average of many values and is small (|out| ~ sqrt(D / S), 0.03 at 130k keys), so the
# absolute bars alone would pass an all-zero output there.  Expected relative error: the bf16
# rounding of out (RMS about 2^-8 / sqrt(3) of each element), the bf16 rounding of P (the same
# share of the weighted sum) and the fp16 score operands (logits off by ~2^-11 of their summed
# magnitudes, a few 1e-3): together about 5e-3 per row; the bar is four times that.  A zeroed
# output is off by 1, values taken from the wrong keys by about sqrt(2).
OUT_REL_L2 = 2e-2
# Query rows per attention workgroup: the sampled full-size checks take one row of every
# (segment, 256-row query tile), with every head.
WG_QUERY_ROWS = 256


def say(msg: str):
    print(msg, flush=True)
    sys.stdout.flush()


def bits_to_device(bits: np.ndarray, device="cuda"):
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(device)


def device_to_f64(t) -> np.ndarray:
    import torch
    if t.dtype == torch.bfloat16:
        u = t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
        return wl.bf16_bits_to_f32(u).astype(np.float64)
    return t.detach().cpu().numpy().astype(np.float64)


def bf16_bits(t) -> np.ndarray:
    import torch
    assert t.dtype == torch.bfloat16
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def widen(bits: np.ndarray) -> np.ndarray:
    return wl.bf16_bits_to_f32(bits).astype(np.float64)


class Case:
    """One packed batch: layout from the library's host builder, inputs from the seed."""

    def __init__(self, segments, heads, seed, qscale=1.0, device="cuda"):
        import torch
        self.segments = segments
        self.heads = heads
        self.cu, self.pos = H.h3attn_build_layout(segments)
        cu_o, pos_o = oracle.layout(segments)
        assert np.array_equal(self.cu, cu_o) and np.array_equal(self.pos.view(np.uint32), pos_o.view(np.uint32))
        self.N = int(self.cu[-1])
        self.lens = np.diff(self.cu.astype(np.int64))
        self.max_seqlen = int(self.lens.max()) if len(self.lens) else 0
        self.qb, self.kb, self.vb = wl.random_qkv(self.N, heads, seed, scale=(qscale, 1.0, 1.0))
        self.q = bits_to_device(self.qb, device)
        self.k = bits_to_device(self.kb, device)
        self.v = bits_to_device(self.vb, device)
        self.cu_d = torch.from_numpy(self.cu).to(device)
        self.pos_d = torch.from_numpy(np.ascontiguousarray(self.pos)).to(device)

    def run(self, **kw):
        import torch
        out, lse = H.h3attn_varlen_fwd(self.q, self.k, self.v, self.cu_d, self.pos_d, self.max_seqlen, **kw)
        torch.cuda.synchronize()
        return out, lse

    def run_fp8(self, max_seqlen=None, **kw):
        import torch
        ms = self.max_seqlen if max_seqlen is None else max_seqlen
        out, lse = H.h3attn_varlen_fwd_fp8(self.q, self.k, self.v, self.cu_d, self.pos_d, ms, **kw)
        torch.cuda.synchronize()
        return out, lse

    def sage_rows(self, rows=None, **kw):
        """Block-quantized oracle with P unrounded, and its error scales: (out, lse, {"sigma", "zabs"})."""
        return oracle.sage_attention_rows(widen(self.qb), widen(self.kb), widen(self.vb), self.cu, self.pos, rows,
                                          quantize_p=False, error_scales=True, **kw)

    def oracle_full(self, **kw):
        return oracle.attention(widen(self.qb), widen(self.kb), widen(self.vb), self.cu, self.pos, **kw)

    def oracle_rows(self, rows, heads=None, **kw):
        return oracle.attention_rows(widen(self.qb), widen(self.kb), widen(self.vb), self.cu, self.pos, rows, heads,
                                     **kw)

    def sample_rows(self, n_random=128, seed=0):
        """Rows that exercise tile edges, segment edges, the audio tail and a random spread."""
        rng = np.random.default_rng(seed)
        rows = set()
        for s in range(len(self.lens)):
            a, b = int(self.cu[s]), int(self.cu[s + 1])
            if a == b:
                continue
            for off in (0, 1, 31, 32, 63, 64, 127, 128, 255, 256, 257, 511, 512):
                if a + off < b:
                    rows.add(a + off)
            for off in (1, 2, 3, 64, 200, 256):
                if b - off >= a:
                    rows.add(b - off)
        rows.update(int(r) for r in rng.integers(0, self.N, size=n_random))
        return np.array(sorted(rows), dtype=np.int64)

    def workgroup_rows(self, seed=0):
        """One random row of every (segment, 256-row query tile), plus the edge rows of sample_rows."""
        rng = np.random.default_rng(seed)
        rows = set(int(r) for r in self.sample_rows(n_random=0, seed=seed))
        for s in range(len(self.lens)):
            a, b = int(self.cu[s]), int(self.cu[s + 1])
            for t0 in range(a, b, WG_QUERY_ROWS):
                rows.add(int(rng.integers(t0, min(b, t0 + WG_QUERY_ROWS))))
        return np.array(sorted(rows), dtype=np.int64)


def row_relative_error(out_gpu, out_ref):
    """Per (row, head): |out_gpu - out_ref|_2 / |out_ref|_2 over the head dimension, [R, H]."""
    num = np.sqrt(np.sum((out_gpu - out_ref) ** 2, axis=-1))
    den = np.sqrt(np.sum(out_ref ** 2, axis=-1))
    return num / np.maximum(den, 1e-30)


def compare(out_gpu, lse_gpu, out_ref, lse_ref, out_max=OUT_MAX_ABS, out_mean=OUT_MEAN_ABS, lse_max=LSE_MAX_ABS,
            label="", out_rel=OUT_REL_L2):
    """out_rel: the per-row relative bar (None for stress cases whose absolute bars are widened)."""
    err = np.abs(out_gpu - out_ref)
    lerr = np.abs(lse_gpu - lse_ref)
    rel = row_relative_error(out_gpu, out_ref) if out_gpu.size else np.zeros(1)
    stats = dict(out_max=float(err.max()), out_mean=float(err.mean()), lse_max=float(lerr.max()),
                 out_rel_max=float(rel.max()))
    say(f"{label} parity: out max {stats['out_max']:.3e} mean {stats['out_mean']:.3e} lse max {stats['lse_max']:.3e} "
        f"row-relative out max {stats['out_rel_max']:.3e}")
    assert np.all(np.isfinite(out_gpu)) and np.all(np.isfinite(lse_gpu))
    assert stats["out_max"] <= out_max, (label, stats, np.unravel_index(err.argmax(), err.shape))
    assert stats["out_mean"] <= out_mean, (label, stats)
    assert stats["lse_max"] <= lse_max, (label, stats, np.unravel_index(lerr.argmax(), lerr.shape))
    if out_rel is not None:
        assert stats["out_rel_max"] <= out_rel, (label, stats, np.unravel_index(rel.argmax(), rel.shape))
    return stats


def ragged_segments():
    """Segment lengths 1, 127, 129, 255, 0, 64, 300, 2 built from grids and audio runs."""
    return [
        [wl.visual(1, 1, 1)],
        [wl.visual(1, 7, 17), wl.audio(8, 1, attached=True)],
        [wl.visual(2, 8, 8), wl.audio(1, 2, attached=True)],
        [wl.visual(3, 9, 9), wl.audio(12, 3, attached=True, rule="round")],
        [],
        [wl.visual(1, 8, 8)],
        [wl.visual(2, 10, 14), wl.audio(20, 2, attached=True)],
        [wl.audio(2, 1.0, attached=False)],
    ]


# Bar for the lossy FP8 mode.
#
# Against the block-quantized oracle (oracle.sage with P left unrounded), the
# kernel differs by:
#   * the e4m3 rounding of its probabilities: per output element a sum of
#     independent roundings whose standard deviation the oracle reports
#     ("sigma").  Bound: 6 sigma, plus the bf16 rounding of out (2^-8 of
#     |out|), plus 1e-4 for fp32 accumulation order.
#   * evaluation of the scores: the scaled fp8 products are summed by the matrix
#     core, whose accumulation is not exact fp32: on logits of several hundred
#     (q x 64) lse moved by up to 2^-15.8 of the row's largest sum of absolute
#     products ("zabs" per row).  Bound: lse within 2^-14 zabs + 1e-5, the same
#     evaluation error the oracle allows each logit for Skip-Softmax decisions.
#   * rounding decisions: the kernel rotates in fp32 arithmetic of its own and
#     the oracle rounds the float64 rotation to fp32; where an e4m3 rounding
#     midpoint (or a block-scale boundary) lies within their error window, both
#     roundings are valid.  The oracle reports how far such elements can move
#     lse and out ("lse_flip", "out_flip", zero for almost every row), and both
#     bounds include it.
#
# Against the exact float64 oracle: the quality of the mode itself, on the
# N(0, 1) workloads.  Rounding Q and K to 3-bit mantissas (relative error up to
# 2^-4 each, standard deviation about 2^-4 / sqrt(3)) moves a logit by
# sigma_z = scale sqrt(2/3) 2^-4 |q * k|_2, about 0.05 for N(0, 1) rows.  A row
# dominated by one key moves its lse by sigma_z: 5 sigma_z = 0.25.  Its output
# moves by p (1 - p) sigma_z |v_a - v_b| for two competing keys, at most
# 1/4 x 0.05 x 8 (4-sigma values of v) x 5 = 0.5; rounding V adds 2^-4 of
# |v| on such rows.  Averaged over all outputs the error stays far smaller:
# mean-abs 2e-2.
# Per (row, head) the relative L2 error |out - out_exact|_2 / |out_exact|_2 is
# what stays meaningful on long rows, whose outputs are small averages: the
# logit noise moves out by about sigma_z of itself, and the roundings of V and
# P by about 2^-4 / sqrt(3) = 0.036 each, so sqrt(0.05^2 + 2 x 0.036^2) = 0.07;
# the bar is four times that, 0.3 (measured on the float64 modes at 1344x768:
# 0.053 mean, 0.068 largest of 200 row-heads).  A zeroed output is off by 1,
# values taken from other keys by about 1.4.  Wider inputs (the peaky case) are
# checked against the quantized oracle only; their distance from exact softmax
# grows with the logits and is reported.
FP8_SIGMAS = 6.0
FP8_LSE_REL = 2.0 ** -14
FP8_LSE_ABS = 1e-5
FP8_EXACT_OUT_MAX = 0.5
FP8_EXACT_OUT_MEAN = 2e-2
FP8_EXACT_LSE_MAX = 0.25
FP8_EXACT_REL = 0.3


def compare_fp8(out_gpu, lse_gpu, out_sage, lse_sage, scales, out_exact, lse_exact, label="", exact_bars=True):
    """exact_bars: also hold the mode to its quality bar against exact softmax (N(0, 1) inputs)."""
    sigma, zabs = scales["sigma"], scales["zabs"]
    d = np.abs(out_gpu - out_sage)
    bound = FP8_SIGMAS * sigma + 2.0 ** -8 * np.abs(out_sage) + 1e-4 + scales["out_flip"]
    ld = np.abs(lse_gpu - lse_sage)
    lbound = FP8_LSE_REL * zabs + FP8_LSE_ABS + scales["lse_flip"]
    ex = np.abs(out_gpu - out_exact)
    lex = np.abs(lse_gpu - lse_exact)
    rel = row_relative_error(out_gpu, out_exact)
    stats = dict(max_over_bound=float((d / bound).max()), rms_over_sigma=float(np.sqrt(np.mean((d / sigma) ** 2))),
                 lse_max=float(ld.max()), lse_max_over_bound=float((ld / lbound).max()),
                 rows_with_alternatives=int(np.count_nonzero(scales["lse_flip"])),
                 exact_out_max=float(ex.max()), exact_out_mean=float(ex.mean()), exact_lse_max=float(lex.max()),
                 exact_rel_max=float(rel.max()))
    say(f"{label} fp8: vs quantized oracle: max err/bound {stats['max_over_bound']:.3f}, rms err/sigma "
        f"{stats['rms_over_sigma']:.3f}, lse max {stats['lse_max']:.2e} (max err/bound {stats['lse_max_over_bound']:.3f}, "
        f"rows with alternative roundings {stats['rows_with_alternatives']}); "
        f"vs exact: out max {stats['exact_out_max']:.3e} mean {stats['exact_out_mean']:.3e} lse max "
        f"{stats['exact_lse_max']:.3e} row-relative max {stats['exact_rel_max']:.3e}")
    assert np.all(np.isfinite(out_gpu)) and np.all(np.isfinite(lse_gpu))
    assert stats["max_over_bound"] <= 1.0, (label, stats, np.unravel_index((d / bound).argmax(), d.shape))
    assert stats["lse_max_over_bound"] <= 1.0, (label, stats, np.unravel_index((ld / lbound).argmax(), ld.shape))
    if exact_bars:
        assert stats["exact_out_max"] <= FP8_EXACT_OUT_MAX, (label, stats)
        assert stats["exact_out_mean"] <= FP8_EXACT_OUT_MEAN, (label, stats)
        assert stats["exact_lse_max"] <= FP8_EXACT_LSE_MAX, (label, stats)
        assert stats["exact_rel_max"] <= FP8_EXACT_REL, (label, stats, np.unravel_index(rel.argmax(), rel.shape))
    return stats


BF16_NAN = 0x7FC0
BF16_INF = 0x7F80


def nonfinite_isolation(c, run, segments_poisoned=(1, 3, 6), same_row_heads=True, near=(1e-2, 1e-3)):
    """Non-finite inputs stay where they are.

    On a case built from ragged_segments(), poisons head 0 of one query row of segment 1 (NaN),
    one key of segment 3 (+inf) and one value of segment 6 (NaN, value dim 100), and checks
    against a clean run: every row of every other segment, and every other head, comes out bit
    for bit the same; so does every other value dim of segment 6; the poisoned query row and
    value dim do come out non-finite.  The other rows of the query's segment come out bit for bit
    the same where the kernel decides everything per row (same_row_heads), else finite and within
    near = (out, lse) max-abs of the clean run: a kernel that moves the softmax reference of a
    whole wave at once may then round them against another valid reference.
    run(c) -> (out, lse) on the case's current inputs.
    """
    sq, sk, sv = segments_poisoned
    out0, lse0 = run(c)
    o0, l0 = bf16_bits(out0), lse0.cpu().numpy()
    rq, rk, rv = int(c.cu[sq]) + 5, int(c.cu[sk]) + 17, int(c.cu[sv]) + 40
    assert rq < c.cu[sq + 1] and rk < c.cu[sk + 1] and rv < c.cu[sv + 1]
    c.qb = c.qb.copy()
    c.kb = c.kb.copy()
    c.vb = c.vb.copy()
    c.qb[rq, 0, 3] = BF16_NAN
    c.kb[rk, 0, 10] = BF16_INF
    c.vb[rv, 0, 100] = BF16_NAN
    dev = c.q.device
    c.q, c.k, c.v = bits_to_device(c.qb, dev), bits_to_device(c.kb, dev), bits_to_device(c.vb, dev)
    out1, lse1 = run(c)
    o1, l1 = bf16_bits(out1), lse1.cpu().numpy()
    seg_of = np.searchsorted(c.cu, np.arange(c.N), side="right") - 1
    clean = ~np.isin(seg_of, segments_poisoned)
    assert np.array_equal(o1[clean], o0[clean]) and np.array_equal(l1[:, clean], l0[:, clean])
    assert np.array_equal(o1[:, 1:], o0[:, 1:]) and np.array_equal(l1[1:], l0[1:])  # other heads
    seg_v = seg_of == sv
    keep = np.ones(o0.shape[2], dtype=bool)
    keep[100] = False
    assert np.array_equal(o1[seg_v][:, 0][:, keep], o0[seg_v][:, 0][:, keep])
    f1 = widen(o1)
    assert not np.all(np.isfinite(f1[rq, 0])) and not np.isfinite(l1[0, rq])
    assert not np.all(np.isfinite(f1[seg_v, 0, 100]))
    rows_q = (seg_of == sq) & (np.arange(c.N) != rq)
    if same_row_heads:
        # the other rows of the query's segment do not see its query at all
        assert np.array_equal(o1[rows_q], o0[rows_q]) and np.array_equal(l1[:, rows_q], l0[:, rows_q])
    else:
        d_out = float(np.abs(widen(o1[rows_q]) - widen(o0[rows_q])).max())
        d_lse = float(np.abs(l1[:, rows_q] - l0[:, rows_q]).max())
        say(f"non-finite inputs: other rows of the query's segment moved by out {d_out:.3e}, lse {d_lse:.3e}")
        assert d_out <= near[0] and d_lse <= near[1], (d_out, d_lse)
    say(f"non-finite inputs: {int(clean.sum())} rows of untouched segments and heads 1.. bit for bit unchanged; "
        f"poisoned row lse {l1[0, rq]}")
