"""GPU parity of the lossy FP8 mode (h3attn_varlen_fwd_fp8) through the C ABI.

Bars (tests/helpers.py, compare_fp8): against the block-quantized float64
oracle (oracle.sage, P unrounded) every output element within 6 standard
deviations of the P rounding the oracle predicts, plus the bf16 rounding of
out; lse within fp32 score evaluation error (2^-16 of the row's largest sum
of absolute products); both plus what the oracle reports alternative
roundings next to an e4m3 midpoint can change; against
the exact float64 oracle the mode's own quality bar on N(0, 1) inputs (out
max-abs 0.5, mean-abs 2e-2, lse max-abs 0.25).  Small cases are compared in full,
the workloads on sampled rows in the launch configuration the bench times.
"""

import numpy as np
import pytest

from helpers import Case, bf16_bits, compare_fp8, device_to_f64, ragged_segments, say
from joint_sequence_attention_amd import h3attn as H
from joint_sequence_attention_amd import workloads as wl

pytestmark = pytest.mark.gpu


def _full(c, label, exact_bars=True, scale=None, **kw):
    out, lse = c.run_fp8(softmax_scale=scale or 0.0, **kw)
    o_s, l_s, es = c.sage_rows(scale=scale, **kw)
    o_e, l_e = c.oracle_full(scale=scale, **kw)
    return compare_fp8(device_to_f64(out), device_to_f64(lse), o_s, l_s, es, o_e, l_e, label=label,
                       exact_bars=exact_bars)


@pytest.mark.parametrize("seed", [1, 1001])
def test_fp8_tiny_full(gpu, seed):
    cfg = wl.config("tiny")
    c = Case(cfg["segments"], cfg["heads"], seed)
    say(f"fp8 tiny seed {seed}: N={c.N} H={c.heads}")
    _full(c, f"tiny/{seed}")


@pytest.mark.parametrize("heads", [1, 3])
def test_fp8_ragged_segments_full(gpu, heads):
    c = Case(ragged_segments(), heads, 140 + heads)
    say(f"fp8 ragged: lens={c.lens.tolist()} H={heads}")
    _full(c, "ragged")


def test_fp8_peaky_softmax_full(gpu):
    # q x 4: logits four times wider; checked against the quantized oracle (the
    # distance from exact softmax grows with the logits and is only reported).
    c = Case(ragged_segments(), 2, 150, qscale=4.0)
    say(f"fp8 peaky: lens={c.lens.tolist()}")
    _full(c, "peaky", exact_bars=False)


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
    rows = c.sample_rows(n_random=64 if c.N > 100000 else 128, seed=seed)
    o_s, l_s, es = c.sage_rows(rows)
    o_e, l_e = c.oracle_rows(rows)
    compare_fp8(out64[rows], lse64[:, rows], o_s, l_s, es, o_e, l_e, label=f"{name}/{seed} ({len(rows)} rows)")


def test_fp8_explicit_scale_and_rope_config(gpu):
    c = Case(ragged_segments(), 2, 164)
    say("fp8 explicit scale / rope config")
    _full(c, "scale/theta", scale=0.05, theta=500.0, dims=(64, 32, 32))


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


def test_fp8_length_one_and_empty_segments(gpu):
    import torch
    segs = [[], [wl.visual(1, 1, 1)], [], [wl.audio(1, 1.0, attached=False)], [wl.visual(1, 5, 7)], []]
    c = Case(segs, 2, 166)
    out, lse = H.h3attn_varlen_fwd_fp8(c.q, c.k, c.v, c.cu_d, c.pos_d, c.N)  # generous max_seqlen
    torch.cuda.synchronize()
    o_s, l_s, es = c.sage_rows()
    o_e, l_e = c.oracle_full()
    compare_fp8(device_to_f64(out), device_to_f64(lse), o_s, l_s, es, o_e, l_e, label="length-1/empty")


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


def test_fp8_refiner_full(gpu):
    cfg = wl.config("refiner")
    c = Case(cfg["segments"], cfg["heads"], cfg["seed"])
    say(f"fp8 refiner: N={c.N} H={c.heads}")
    _full(c, "refiner")


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
    say(f"{label}: kernel left out {skipped} of {seen} (block, tile) pairs; oracle share {es['skipped'].mean():.4f}")
    return seen, skipped, es


def test_fp8_skip_negligible_threshold_equals_dense(gpu):
    import torch
    c = Case(ragged_segments(), 3, 180)
    out, lse = c.run_fp8()
    stats = torch.zeros(2, dtype=torch.int64, device="cuda")
    out2, lse2 = c.run_fp8(skip_threshold=1e-30, skip_stats=stats)
    assert np.array_equal(bf16_bits(out), bf16_bits(out2))
    assert np.array_equal(lse.cpu().numpy(), lse2.cpu().numpy())
    seen, skipped = (int(x) for x in stats.cpu().numpy())
    assert skipped == 0 and seen > 0


def test_fp8_skip_local_attention_full(gpu):
    # local attention: most (block, tile) pairs are negligible; every row checked against the oracle's rule
    c = _local_case(1000, 2, 181)
    say(f"fp8 skip local: N={c.N} H=2")
    seen, skipped, es = _skip_run(c, 0.05, label="skip local")
    # the kernel skips exactly what the oracle's rule skips, up to decisions next to the threshold
    blocks = np.arange(c.N)[::32]
    n_tiles = (c.N + 63) // 64
    want = int(round(float((es["skipped"][:, blocks] * n_tiles).sum())))
    slack = int(es["skip_ambiguous"][:, blocks].sum())
    assert seen == 2 * len(blocks) * n_tiles
    assert abs(skipped - want) <= slack, (skipped, want, slack)
    assert skipped > seen // 3                    # the case really exercises skipping


def test_fp8_skip_peaky_ragged_full(gpu):
    c = Case(ragged_segments(), 2, 182, qscale=4.0)
    say(f"fp8 skip peaky: lens={c.lens.tolist()}")
    _skip_run(c, 0.05, label="skip peaky")


def test_fp8_skip_workload_sampled_rows(gpu):
    cfg = wl.config("1344x768")
    c = Case(cfg["segments"], cfg["heads"], cfg["seed"])
    rows = c.sample_rows(n_random=16, seed=183)
    say(f"fp8 skip 1344x768: N={c.N} H={c.heads}, {len(rows)} rows (whole 32-row blocks evaluated)")
    _skip_run(c, 0.05, rows=rows, label="skip 1344x768")


# ---- Running maximum that moves on every tile ----------------------------------------------------


def _rising_case(n_tokens, heads, seed, top=40.0):
    """Keys that line up with the queries and grow along the sequence: every 64-key tile holds
    larger logits than the one before, so the running maximum moves on every tile (up to ~top
    natural units), with ragged segment lengths."""
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
    c0 = Case([[wl.visual(1, 1, n)] for n in lens], heads, seed)
    c0.qb, c0.kb, c0.vb = bits(q), bits(k), bits(v)
    dev = c0.q.device
    c0.q, c0.k, c0.v = bits_to_device(c0.qb, dev), bits_to_device(c0.kb, dev), bits_to_device(c0.vb, dev)
    return c0


def test_fp8_running_maximum_moves_every_tile(gpu):
    c = _rising_case(1200, 2, 190)
    say(f"fp8 rising logits: lens={c.lens.tolist()}")
    _full(c, "rising", exact_bars=False)


def test_fp8_very_large_logits(gpu):
    # q x 64: logits of several hundred, far past exp2's range without a reference; every row
    # must still come out finite and match the oracle
    c = Case(ragged_segments(), 2, 191, qscale=64.0)
    say(f"fp8 very large logits: lens={c.lens.tolist()}")
    out, lse = c.run_fp8()
    assert np.all(np.isfinite(device_to_f64(out))) and np.all(np.isfinite(device_to_f64(lse)))
    _full(c, "large logits", exact_bars=False)
