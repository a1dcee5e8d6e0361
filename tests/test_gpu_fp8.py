"""GPU parity of the lossy FP8 mode (h3attn_varlen_fwd_fp8) through the C ABI.

Bars (tests/helpers.py, compare_fp8): against the block-quantized float64
oracle (oracle.sage, P unrounded) every output element within 6 standard
deviations of the P rounding the oracle predicts, plus the bf16 rounding of
out; lse within fp32 score evaluation error (2^-16 of the row's largest sum
of absolute products); both plus what the oracle reports alternative
roundings next to an e4m3 midpoint can change; against
the exact float64 oracle the mode's own quality bar on N(0, 1) inputs (out
max-abs 0.5, mean-abs 2e-2, lse max-abs 0.25, and per (row, head) a relative
L2 error of at most 0.3).  Small cases are compared in full, the workloads on
one row of every attention workgroup in the launch configuration the bench
times.  Skip-Softmax decisions are per row; the kernel's count of left-out
(row, tile) pairs is held to the oracle's, up to decisions next to the
threshold, on full cases and on every row of one head of the configuration
the bench times.
"""

import numpy as np
import pytest

from helpers import (Case, bf16_bits, compare_fp8, device_to_f64, nonfinite_isolation, ragged_segments, say,
                     widen)
from joint_sequence_attention_amd import h3attn as H
from joint_sequence_attention_amd import workloads as wl

pytestmark = pytest.mark.gpu

# The dense kernel moves its softmax reference in one of two forms, chosen per launch by
# max_seqlen: early below 65,536 keys, late from there on.  The small cases run in both: for the
# late form one 65,536-token segment follows them in the same launch, and only their own rows
# are compared (the long segment's rows are checked for being finite).
FORMS = ["early", "late"]
FILLER = [wl.visual(16, 64, 64)]  # 65,536 tokens


def _segments(segments, form):
    return list(segments) + [FILLER] if form == "late" else list(segments)


def _n_rows(c, n_segments):
    """Rows of the first n_segments segments of a case."""
    return int(c.cu[n_segments])


def _full(c, label, exact_bars=True, scale=None, n_rows=None, max_seqlen=None, **kw):
    out, lse = c.run_fp8(max_seqlen=max_seqlen, softmax_scale=scale or 0.0, **kw)
    out64, lse64 = device_to_f64(out), device_to_f64(lse)
    if n_rows is None or n_rows == c.N:
        o_s, l_s, es = c.sage_rows(scale=scale, **kw)
        o_e, l_e = c.oracle_full(scale=scale, **kw)
    else:
        assert np.all(np.isfinite(out64[n_rows:])) and np.all(np.isfinite(lse64[:, n_rows:]))
        rows = np.arange(n_rows)
        o_s, l_s, es = c.sage_rows(rows, scale=scale, **kw)
        o_e, l_e = c.oracle_rows(rows, scale=scale, **kw)
        out64, lse64 = out64[:n_rows], lse64[:, :n_rows]
    return compare_fp8(out64, lse64, o_s, l_s, es, o_e, l_e, label=label, exact_bars=exact_bars)


def _form_case(segments, heads, seed, form, **kw):
    """(case, rows to compare) for the small segments in the given form."""
    c = Case(_segments(segments, form), heads, seed, **kw)
    return c, _n_rows(c, len(segments))


@pytest.mark.parametrize("form", FORMS)
@pytest.mark.parametrize("seed", [1, 1001])
def test_fp8_tiny_full(gpu, seed, form):
    cfg = wl.config("tiny")
    c, n = _form_case(cfg["segments"], cfg["heads"], seed, form)
    say(f"fp8 tiny seed {seed} ({form}): N={c.N} H={c.heads}")
    _full(c, f"tiny/{seed}/{form}", n_rows=n)


@pytest.mark.parametrize("form", FORMS)
@pytest.mark.parametrize("heads", [1, 3])
def test_fp8_ragged_segments_full(gpu, heads, form):
    c, n = _form_case(ragged_segments(), heads, 140 + heads, form)
    say(f"fp8 ragged ({form}): lens={c.lens.tolist()} H={heads}")
    _full(c, f"ragged/{form}", n_rows=n)


@pytest.mark.parametrize("form", FORMS)
def test_fp8_peaky_softmax_full(gpu, form):
    # q x 4: logits four times wider; checked against the quantized oracle (the
    # distance from exact softmax grows with the logits and is only reported).
    c, n = _form_case(ragged_segments(), 2, 150, form, qscale=4.0)
    say(f"fp8 peaky ({form}): lens={c.lens.tolist()}")
    _full(c, f"peaky/{form}", exact_bars=False, n_rows=n)


@pytest.mark.parametrize("name", ["480p", "packed", "1344x768", "ref2va", "long300"])
@pytest.mark.parametrize("seed_offset", [0, wl.ROBUSTNESS_SEED_OFFSET])
def test_fp8_workload_sampled_rows(gpu, name, seed_offset):
    cfg = wl.config(name)
    seed = cfg["seed"] + seed_offset
    c = Case(cfg["segments"], cfg["heads"], seed)
    say(f"fp8 {name} seed {seed}: N={c.N} H={c.heads} segments={len(c.lens)}")
    out, lse = c.run_fp8()
    out64, lse64 = device_to_f64(out), device_to_f64(lse)
    assert np.all(np.isfinite(out64)) and np.all(np.isfinite(lse64))
    rows = c.workgroup_rows(seed=seed)
    o_s, l_s, es = c.sage_rows(rows)
    o_e, l_e = c.oracle_rows(rows)
    compare_fp8(out64[rows], lse64[:, rows], o_s, l_s, es, o_e, l_e,
                label=f"{name}/{seed} ({len(rows)} rows, every query tile)")


@pytest.mark.parametrize("form", FORMS)
def test_fp8_explicit_scale_and_rope_config(gpu, form):
    c, n = _form_case(ragged_segments(), 2, 164, form)
    say(f"fp8 explicit scale / rope config ({form})")
    _full(c, f"scale/theta/{form}", scale=0.05, theta=500.0, dims=(64, 32, 32), n_rows=n)


def test_fp8_two_stages_equal_fused_call_and_deterministic(gpu):
    import torch
    c = Case(ragged_segments(), 3, 161)
    out, lse = c.run_fp8()
    ws = H.alloc_workspace(c.N, 3, len(c.lens), fp8=True)
    H.h3attn_varlen_kv_prologue_fp8(c.k, c.v, c.cu_d, c.pos_d, c.max_seqlen, ws)
    out2, lse2 = H.h3attn_varlen_attention_fp8(c.q, c.cu_d, c.pos_d, c.max_seqlen, ws)
    torch.cuda.synchronize()
    assert np.array_equal(bf16_bits(out), bf16_bits(out2))
    assert np.array_equal(lse.cpu().numpy(), lse2.cpu().numpy())
    out3, lse3 = c.run_fp8()
    assert np.array_equal(bf16_bits(out), bf16_bits(out3))
    assert np.array_equal(lse.cpu().numpy(), lse3.cpu().numpy())


def test_fp8_segment_isolation_bitwise(gpu):
    import torch
    segs = [[wl.visual(T, 6, 10), wl.audio(32 * T // 4, T, attached=True)] for T in (3, 5, 2)]
    c = Case(segs, 2, 163)
    out, lse = c.run_fp8()
    for s in range(len(segs)):
        a, b = int(c.cu[s]), int(c.cu[s + 1])
        cu1 = torch.tensor([0, b - a], dtype=torch.int32, device="cuda")
        o1, l1 = H.h3attn_varlen_fwd_fp8(c.q[a:b].contiguous(), c.k[a:b].contiguous(), c.v[a:b].contiguous(), cu1,
                                         c.pos_d[a:b].contiguous(), b - a)
        torch.cuda.synchronize()
        assert np.array_equal(bf16_bits(out[a:b]), bf16_bits(o1))
        assert np.array_equal(lse[:, a:b].cpu().numpy(), l1.cpu().numpy())


@pytest.mark.parametrize("form", FORMS)
def test_fp8_length_one_and_empty_segments(gpu, form):
    segs = [[], [wl.visual(1, 1, 1)], [], [wl.audio(1, 1.0, attached=False)], [wl.visual(1, 5, 7)], []]
    c, n = _form_case(segs, 2, 166, form)
    _full(c, f"length-1/empty/{form}", n_rows=n, max_seqlen=c.N)  # generous max_seqlen


def test_fp8_zero_tokens_noop(gpu):
    import torch
    q = torch.empty((0, 2, 128), dtype=torch.bfloat16, device="cuda")
    cu = torch.zeros(2, dtype=torch.int32, device="cuda")
    pos = torch.empty((0, 3), dtype=torch.float32, device="cuda")
    ws = torch.empty(256, dtype=torch.uint8, device="cuda")
    out, lse = H.h3attn_varlen_fwd_fp8(q, q, q, cu, pos, 0, workspace=ws)
    torch.cuda.synchronize()
    assert out.shape == (0, 2, 128) and lse.shape == (2, 0)


# ---- limits of the launch shape --------------------------------------------------------------


def test_fp8_long_single_segment_sampled_rows(gpu):
    segs = [[wl.visual(64, 64, 64)]]
    c = Case(segs, 1, seed=171)
    say(f"fp8 long segment: N={c.N} H=1")
    out, lse = c.run_fp8()
    out64, lse64 = device_to_f64(out), device_to_f64(lse)
    assert np.all(np.isfinite(out64)) and np.all(np.isfinite(lse64))
    rows = c.sample_rows(n_random=24, seed=171)
    o_s, l_s, es = c.sage_rows(rows)
    o_e, l_e = c.oracle_rows(rows)
    compare_fp8(out64[rows], lse64[:, rows], o_s, l_s, es, o_e, l_e, label=f"long segment ({len(rows)} rows)")


def test_fp8_two_thousand_short_segments_full(gpu):
    rng = np.random.default_rng(172)
    lengths = rng.integers(0, 65, size=2000)
    segs = [[wl.visual(1, 1, int(n))] if n else [] for n in lengths]
    c = Case(segs, 2, seed=172)
    say(f"fp8 2000 segments: N={c.N} H=2, empty={int((lengths == 0).sum())}")
    _full(c, "2000 segments")


def test_fp8_many_heads_full(gpu):
    c = Case([[wl.visual(2, 16, 16)]], 128, seed=173)
    say(f"fp8 128 heads: N={c.N} H=128")
    _full(c, "128 heads")


@pytest.mark.parametrize("form", FORMS)
def test_fp8_refiner_full(gpu, form):
    cfg = wl.config("refiner")
    c, n = _form_case(cfg["segments"], cfg["heads"], cfg["seed"], form)
    say(f"fp8 refiner ({form}): N={c.N} H={c.heads}")
    _full(c, f"refiner/{form}", n_rows=n)


# ---- Skip-Softmax ------------------------------------------------------------------------------


def _local_case(n_tokens, heads, seed, sharp=3.0):
    """A sequence whose attention is local: q_i . k_j peaks at i = j (features cos/sin of i w_m),
    positions zero (identity rotation), so tiles far after a block's own keys carry almost no weight."""
    from helpers import bits_to_device
    rng = np.random.default_rng(seed)
    w = 0.5 * np.power(10.0, -np.arange(64) / 64.0)
    ang = np.arange(n_tokens)[:, None] * w[None, :]
    f = np.concatenate([np.cos(ang), np.sin(ang)], axis=1) * sharp / 1.5
    def bits(x):
        return wl._round_bf16_bits(np.ascontiguousarray(x, dtype=np.float32))
    q = f[:, None, :] + 0.3 * rng.standard_normal((n_tokens, heads, 128))
    k = f[:, None, :] + 0.3 * rng.standard_normal((n_tokens, heads, 128))
    v = rng.standard_normal((n_tokens, heads, 128))
    c = Case([[wl.visual(1, 1, n_tokens)]], heads, seed)
    c.qb, c.kb, c.vb = bits(q), bits(k), bits(v)
    dev = c.q.device
    c.q, c.k, c.v = bits_to_device(c.qb, dev), bits_to_device(c.kb, dev), bits_to_device(c.vb, dev)
    c.pos = np.zeros_like(c.pos)
    c.pos_d = c.pos_d.zero_()
    return c


def _skip_run(c, thr, rows=None, label=""):
    """Kernel with Skip-Softmax against the oracle's rule; returns the kernel's (row, tile) counts and
    the oracle's error scales (per-row left-out and ambiguous counts)."""
    import torch
    stats = torch.zeros(2, dtype=torch.int64, device="cuda")
    out, lse = c.run_fp8(skip_threshold=thr, skip_stats=stats)
    o64, l64 = device_to_f64(out), device_to_f64(lse)
    o_s, l_s, es = c.sage_rows(rows, skip_threshold=thr)
    o_e, l_e = (c.oracle_full() if rows is None else c.oracle_rows(rows))
    if rows is not None:
        o64, l64 = o64[rows], l64[:, rows]
    compare_fp8(o64, l64, o_s, l_s, es, o_e, l_e, label=label, exact_bars=False)
    seen, skipped = (int(x) for x in stats.cpu().numpy())
    say(f"{label}: kernel left out {skipped} of {seen} (row, tile) pairs; oracle on its rows: "
        f"{int(es['skipped'].sum())} of {int(c.heads * es['tiles'].sum())}, "
        f"{int(es['skip_ambiguous'].sum())} decisions could go either way")
    # every row of every head counts each key tile of its segment once
    assert seen == c.heads * int(np.sum(c.lens * ((c.lens + 63) // 64)))
    if rows is None:
        want, slack = int(es["skipped"].sum()), int(es["skip_ambiguous"].sum())
        assert abs(skipped - want) <= slack, (skipped, want, slack)
    return seen, skipped, es


def test_fp8_skip_negligible_threshold_leaves_nothing_out(gpu):
    # A threshold of 1e-30 leaves no tile out: the result is the dense mode's, within the same bars
    # (the skip instance rounds P against the exact running maximum, the dense one against a lazily
    # moved reference within a factor 1.75 of it, so the two are not bit for bit the same).
    import torch
    c = Case(ragged_segments(), 3, 180)
    stats = torch.zeros(2, dtype=torch.int64, device="cuda")
    out, lse = c.run_fp8(skip_threshold=1e-30, skip_stats=stats)
    seen, skipped = (int(x) for x in stats.cpu().numpy())
    assert skipped == 0 and seen == 3 * int(np.sum(c.lens * ((c.lens + 63) // 64)))
    o_s, l_s, es = c.sage_rows()
    o_e, l_e = c.oracle_full()
    compare_fp8(device_to_f64(out), device_to_f64(lse), o_s, l_s, es, o_e, l_e, label="skip 1e-30")


def test_fp8_skip_local_attention_full(gpu):
    # local attention: most (row, tile) pairs are negligible; every row checked against the oracle's
    # rule, and the kernel leaves out exactly the oracle's count up to decisions next to the threshold
    c = _local_case(1000, 2, 181)
    say(f"fp8 skip local: N={c.N} H=2")
    seen, skipped, es = _skip_run(c, 0.05, label="skip local")
    assert skipped > seen // 3                    # the case really exercises skipping


def test_fp8_skip_peaky_ragged_full(gpu):
    c = Case(ragged_segments(), 2, 182, qscale=4.0)
    say(f"fp8 skip peaky: lens={c.lens.tolist()}")
    _skip_run(c, 0.05, label="skip peaky")


def test_fp8_skip_workload_sampled_rows(gpu):
    # N(0, 1) inputs: diffuse attention, where the rule leaves out little
    cfg = wl.config("1344x768")
    c = Case(cfg["segments"], cfg["heads"], cfg["seed"])
    rows = c.sample_rows(n_random=16, seed=183)
    say(f"fp8 skip 1344x768: N={c.N} H={c.heads}, {len(rows)} rows")
    _skip_run(c, 0.05, rows=rows, label="skip 1344x768")


def _local_workload_case(name, heads=None, amp=20.0):
    """The workload's layout with the local-attention inputs bench.py times Skip-Softmax on."""
    from helpers import bits_to_device
    cfg = wl.config(name)
    c = Case(cfg["segments"], cfg["heads"], cfg["seed"])
    c.qb, c.kb, c.vb = wl.local_qkv(c.N, cfg["heads"], cfg["seed"], amp)
    if heads is not None:
        c.qb, c.kb, c.vb = (np.ascontiguousarray(x[:, :heads]) for x in (c.qb, c.kb, c.vb))
        c.heads = heads
    dev = c.q.device
    c.q, c.k, c.v = bits_to_device(c.qb, dev), bits_to_device(c.kb, dev), bits_to_device(c.vb, dev)
    return c


def test_fp8_skip_timed_workload(gpu):
    # The configuration bench.py times: the 1344x768 layout, local-attention inputs of amplitude 20,
    # threshold 0.05, all five heads.  Every attention workgroup's rows sampled against the oracle's
    # rule and outputs; the left-out share reported for all heads.
    c = _local_workload_case("1344x768")
    rows = c.workgroup_rows(seed=184)
    say(f"fp8 skip timed workload: N={c.N} H={c.heads}, {len(rows)} rows")
    seen, skipped, es = _skip_run(c, 0.05, rows=rows, label="skip timed workload")
    share = skipped / seen
    oracle_share = float(es["skipped"].sum()) / float(c.heads * es["tiles"].sum())
    say(f"skip timed workload: kernel share {share:.4f} over every row, oracle {oracle_share:.4f} on the sample")
    assert 0.5 < share < 1.0
    assert abs(share - oracle_share) < 0.02


def test_fp8_skip_timed_workload_head0_counts(gpu):
    # The same configuration, one head, every row: the kernel's count of left-out (row, tile) pairs
    # equals the oracle's (130,048 rows x 2,032 tiles), up to the decisions an evaluation error
    # could flip.
    import torch
    from oracle import sage
    c = _local_workload_case("1344x768", heads=1)
    stats = torch.zeros(2, dtype=torch.int64, device="cuda")
    out, lse = c.run_fp8(skip_threshold=0.05, skip_stats=stats)
    seen, skipped = (int(x) for x in stats.cpu().numpy())
    say(f"skip timed workload head 0: kernel left out {skipped} of {seen}; running the oracle on every row")
    left, amb = sage.skip_counts(widen(c.qb), widen(c.kb), c.cu, c.pos, 0.05)
    want, slack = int(left.sum()), int(amb.sum())
    say(f"skip timed workload head 0: oracle {want} +- {slack}, kernel {skipped} (share {skipped / seen:.4f})")
    assert seen == c.N * ((c.N + 63) // 64)
    assert abs(skipped - want) <= slack, (skipped, want, slack)
    assert np.all(np.isfinite(device_to_f64(out))) and np.all(np.isfinite(device_to_f64(lse)))


# ---- Running maximum that moves on every tile ----------------------------------------------------


def _rising_case(n_tokens, heads, seed, top=40.0, form=None):
    """Keys that line up with the queries and grow along the sequence: every 64-key tile holds
    larger logits than the one before, so the running maximum moves on every tile (up to ~top
    natural units), with ragged segment lengths.  With a form, returns (case, rows of these
    segments), the late form's long segment after them with N(0, 1) rows."""
    from helpers import bits_to_device
    rng = np.random.default_rng(seed)
    c = rng.standard_normal((heads, 128))
    c /= np.linalg.norm(c, axis=1, keepdims=True)
    ramp = np.linspace(0.0, 1.0, n_tokens)[:, None, None]
    q = 3.0 * c[None] + 0.3 * rng.standard_normal((n_tokens, heads, 128))
    k = (top * np.sqrt(128) / 3.0) * ramp * c[None] + 0.3 * rng.standard_normal((n_tokens, heads, 128))
    v = rng.standard_normal((n_tokens, heads, 128))

    def bits(x):
        return wl._round_bf16_bits(np.ascontiguousarray(x, dtype=np.float32))
    lens = [1, 63, 64, 65, 200, n_tokens - 393]
    segs = [[wl.visual(1, 1, n)] for n in lens]
    c0 = Case(_segments(segs, form), heads, seed)
    extra = c0.N - n_tokens
    if extra:
        q, k, v = (np.concatenate([x, rng.standard_normal((extra, heads, 128))]) for x in (q, k, v))
    c0.qb, c0.kb, c0.vb = bits(q), bits(k), bits(v)
    dev = c0.q.device
    c0.q, c0.k, c0.v = bits_to_device(c0.qb, dev), bits_to_device(c0.kb, dev), bits_to_device(c0.vb, dev)
    return c0 if form is None else (c0, n_tokens)


@pytest.mark.parametrize("form", FORMS)
def test_fp8_running_maximum_moves_every_tile(gpu, form):
    c, n = _rising_case(1200, 2, 190, form=form)
    say(f"fp8 rising logits ({form}): lens={c.lens.tolist()}")
    _full(c, f"rising/{form}", exact_bars=False, n_rows=n)


@pytest.mark.parametrize("form", FORMS)
def test_fp8_very_large_logits(gpu, form):
    # q x 64: logits of several hundred, far past exp2's range without a reference; every row
    # must still come out finite and match the oracle
    c, n = _form_case(ragged_segments(), 2, 191, form, qscale=64.0)
    say(f"fp8 very large logits ({form}): lens={c.lens.tolist()}")
    out, lse = c.run_fp8()
    assert np.all(np.isfinite(device_to_f64(out))) and np.all(np.isfinite(device_to_f64(lse)))
    _full(c, f"large logits/{form}", exact_bars=False, n_rows=n)


@pytest.mark.parametrize("form", FORMS + ["skip"])
def test_fp8_nonfinite_inputs_stay_in_their_segment(gpu, form):
    # as for the exact path; the late form and Skip-Softmax decide some steps per wave, so there
    # the other rows of the NaN query's wave may round differently and only other segments and
    # heads are compared
    c, _ = _form_case(ragged_segments(), 2, 178, "late" if form == "late" else "early")
    thr = 0.05 if form == "skip" else 0.0
    say(f"fp8 non-finite inputs ({form})")
    nonfinite_isolation(c, lambda c: c.run_fp8(skip_threshold=thr), same_row_heads=(form == "early"),
                        near=(0.05, 1e-2))
