"""GPU parity: the HIP path through the C ABI against the float64 oracle.

Bar (floating point, bf16 in / fp32 accumulate): out max-abs <= 1e-2 and
mean-abs <= 1e-3, lse max-abs <= 1e-3; layout and positions bit-exact (checked
in every Case); standalone RoPE within one bf16 ulp plus the fp32 arithmetic's
own error bound (see _rope_bound).
Every comparison also holds each (row, head) to a relative L2 bar
(helpers.OUT_REL_L2) unless a stress case widens its bars.  Small cases and
the 480p-shaped workload are compared element by element in full; the other
full-size workloads on one random row of every (segment, 256-row query tile),
i.e. of every attention workgroup, with every head, plus tile and segment
edges, in the launch configuration the bench times, and every output is
checked to be finite.
"""

import math

import numpy as np
import pytest

import oracle
from helpers import Case, bf16_bits, compare, device_to_f64, nonfinite_isolation, ragged_segments, say, widen
from joint_sequence_attention_amd import h3attn as H
from joint_sequence_attention_amd import workloads as wl

pytestmark = pytest.mark.gpu


def _ordered(bits):
    """bf16 bit patterns -> integers that are monotone in the value."""
    b = bits.astype(np.int32)
    return np.where(b & 0x8000, -(b & 0x7FFF), b & 0x7FFF)


def _round_bf16_f64(x):
    f = np.asarray(x, dtype=np.float64).astype(np.float32)
    u = f.view(np.uint32)
    return ((u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)).astype(np.uint16)


def _rope_bound(x, pos, dims=(32, 48, 48), theta=10000.0):
    """Per-element error bound for an fp32 rotation rounded to bf16.

    One bf16 ulp of the exact value for the final rounding, plus the fp32
    arithmetic before it: the frequency and the angle phi = p * omega are each
    rounded to fp32 (angle error <= |phi| 2^-23), sincos and the multiply-adds
    add a few 2^-24 relative to the pair's inputs.  Bound on that part:
    2^-22 (1 + |phi|) (|x0| + |x1|), which matters only where the rotated value
    nearly cancels and is far smaller than its inputs.
    """
    phis = []
    for axis, width in enumerate(dims):
        phis.append(np.asarray(pos, dtype=np.float64)[:, axis][:, None] * oracle.rope_frequencies(theta, width)[None, :])
    phi = np.concatenate(phis, axis=1)                      # [N, 64]
    pair = np.abs(x[..., 0::2]) + np.abs(x[..., 1::2])      # [N, H, 64]
    arith = 2.0 ** -22 * (1.0 + np.abs(phi))[:, None, :] * pair
    return np.repeat(arith, 2, axis=-1)


def _bf16_ulp(v):
    a = np.maximum(np.abs(v), 2.0 ** -126)
    return np.exp2(np.floor(np.log2(a)) - 7)


@pytest.mark.parametrize("name", ["tiny", "480p", "packed", "ref2va", "long300"])
def test_rope_apply_parity(gpu, name):
    cfg = wl.config(name)
    c = Case(cfg["segments"], cfg["heads"], cfg["seed"])
    say(f"rope_apply {name}: N={c.N} H={c.heads}")
    y = H.h3attn_rope_apply(c.q, c.pos_d)
    x = widen(c.qb)
    ref = oracle.rope(x, c.pos)
    yb = bf16_bits(y)
    d = np.abs(_ordered(yb) - _ordered(_round_bf16_f64(ref)))
    err = np.abs(widen(yb) - ref)
    bound = _bf16_ulp(ref) + _rope_bound(x, c.pos)
    say(f"rope_apply {name}: within 1 ulp of the rounded oracle: {float((d <= 1).mean()):.6f}; "
        f"max err / bound {float((err / bound).max()):.3f}")
    assert np.all(err <= bound)
    assert float((d <= 1).mean()) > 0.9999


def test_rope_apply_in_place_matches_out_of_place(gpu):
    cfg = wl.config("480p")
    c = Case(cfg["segments"], cfg["heads"], 7)
    y = H.h3attn_rope_apply(c.q, c.pos_d)
    x = c.q.clone()
    H.h3attn_rope_apply(x, c.pos_d, out=x)
    assert np.array_equal(bf16_bits(x), bf16_bits(y))


def test_rope_apply_at_the_origin_returns_its_input(gpu):
    # Every angle at position (0, 0, 0) is +0, whose sine and cosine are exactly 0 and 1, so the
    # rotation there is the identity: the output equals the input value for value. The refiner's
    # text rows all sit at the origin; the tiny workload's first video token does too, inside a
    # wave of other tokens.
    for name in ("refiner", "tiny"):
        cfg = wl.config(name)
        c = Case(cfg["segments"], cfg["heads"], cfg["seed"])
        at0 = np.all(c.pos == 0, axis=1)
        say(f"rope_apply at the origin, {name}: {int(at0.sum())} of {c.N} tokens")
        assert at0.any()
        y = widen(bf16_bits(H.h3attn_rope_apply(c.q, c.pos_d)))
        assert np.array_equal(y[at0], widen(c.qb)[at0])


@pytest.mark.parametrize("seed", [1, 1001])
def test_tiny_full(gpu, seed):
    cfg = wl.config("tiny")
    c = Case(cfg["segments"], cfg["heads"], seed)
    say(f"varlen tiny seed {seed}: N={c.N} H={c.heads}")
    out, lse = c.run()
    o_ref, l_ref = c.oracle_full()
    compare(device_to_f64(out), device_to_f64(lse), o_ref, l_ref, label=f"tiny/{seed}")


@pytest.mark.parametrize("heads", [1, 3])
def test_ragged_segments_full(gpu, heads):
    c = Case(ragged_segments(), heads, 40 + heads)
    say(f"varlen ragged: lens={c.lens.tolist()} H={heads}")
    out, lse = c.run()
    o_ref, l_ref = c.oracle_full()
    compare(device_to_f64(out), device_to_f64(lse), o_ref, l_ref, label="ragged")


def test_peaky_softmax_full(gpu):
    # q scaled by 4: scores spread ~4x wider, so the softmax concentrates on few
    # keys.  bf16 rounding of the rotated q and k (relative 2^-9 each) then moves
    # a score by ~|z| * 2^-8 ~ 1.5e-2 at the top of the range, and lse and out
    # follow the top scores: bound 5e-2 max, 5e-3 mean (lse 5e-2).
    c = Case(ragged_segments(), 2, 50, qscale=4.0)
    say(f"varlen peaky: lens={c.lens.tolist()}")
    out, lse = c.run()
    o_ref, l_ref = c.oracle_full()
    compare(device_to_f64(out), device_to_f64(lse), o_ref, l_ref, out_max=5e-2, out_mean=5e-3, lse_max=5e-2,
            label="peaky", out_rel=None)


@pytest.mark.parametrize("name", ["480p", "packed", "1344x768", "ref2va", "long300"])
@pytest.mark.parametrize("seed_offset", [0, wl.ROBUSTNESS_SEED_OFFSET])
def test_workload_sampled_rows(gpu, name, seed_offset):
    cfg = wl.config(name)
    seed = cfg["seed"] + seed_offset
    c = Case(cfg["segments"], cfg["heads"], seed)
    say(f"varlen {name} seed {seed}: N={c.N} H={c.heads} segments={len(c.lens)}")
    out, lse = c.run()
    out64 = device_to_f64(out)
    lse64 = device_to_f64(lse)
    assert np.all(np.isfinite(out64)) and np.all(np.isfinite(lse64))
    rows = c.workgroup_rows(seed=seed)
    o_ref, l_ref = c.oracle_rows(rows)
    compare(out64[rows], lse64[:, rows], o_ref, l_ref, label=f"{name}/{seed} ({len(rows)} rows, every query tile)")


def test_480p_full(gpu):
    # every row of every head of the 480p-shaped workload (7,936 tokens, 24 heads)
    cfg = wl.config("480p")
    c = Case(cfg["segments"], cfg["heads"], cfg["seed"])
    say(f"varlen 480p in full: N={c.N} H={c.heads}")
    out, lse = c.run()
    o_ref, l_ref = c.oracle_full()
    compare(device_to_f64(out), device_to_f64(lse), o_ref, l_ref, label="480p full")


def test_fused_rope_turns_like_standalone_rope(gpu):
    # Rotating q and k with h3attn_rope_apply and then attending with all
    # positions zero (a rotation by zero is exact) must agree with the fused
    # path up to the extra bf16 rounding of the rotated operands (relative
    # 2^-9 per element; on this case lse moves by < 3e-3 and out by < 1e-2).
    # A rotation that differed from the standalone one (wrong pair, sign or
    # frequency) would move scores by O(1).
    c = Case(ragged_segments(), 2, 60)
    out, lse = c.run()
    qr = H.h3attn_rope_apply(c.q, c.pos_d)
    kr = H.h3attn_rope_apply(c.k, c.pos_d)
    zero = c.pos_d.clone().zero_()
    out2, lse2 = H.h3attn_varlen_fwd(qr, kr, c.v, c.cu_d, zero, c.max_seqlen)
    compare(device_to_f64(out2), device_to_f64(lse2), device_to_f64(out), device_to_f64(lse), out_max=1e-2,
            out_mean=1e-3, lse_max=3e-3, label="fused vs standalone rope", out_rel=None)


def test_two_stages_equal_fused_call(gpu):
    import torch
    c = Case(ragged_segments(), 3, 61)
    out, lse = c.run()
    ws = H.alloc_workspace(c.N, 3, len(c.lens))
    H.h3attn_varlen_kv_prologue(c.k, c.v, c.cu_d, c.pos_d, c.max_seqlen, ws)
    out2, lse2 = H.h3attn_varlen_attention(c.q, c.cu_d, c.pos_d, c.max_seqlen, ws)
    torch.cuda.synchronize()
    assert np.array_equal(bf16_bits(out), bf16_bits(out2))
    assert np.array_equal(lse.cpu().numpy(), lse2.cpu().numpy())


def test_deterministic(gpu):
    c = Case(ragged_segments(), 2, 62)
    o1, l1 = c.run()
    o2, l2 = c.run()
    assert np.array_equal(bf16_bits(o1), bf16_bits(o2))
    assert np.array_equal(l1.cpu().numpy(), l2.cpu().numpy())


def test_segment_isolation_bitwise(gpu):
    # Each packed segment's rows equal a run of that segment alone.
    import torch
    cfg = wl.config("packed")
    segs = [[wl.visual(T, 6, 10), wl.audio(32 * T // 4, T, attached=True)] for T in (3, 5, 2)]
    c = Case(segs, 2, 63)
    out, lse = c.run()
    for s in range(len(segs)):
        a, b = int(c.cu[s]), int(c.cu[s + 1])
        cu1 = torch.tensor([0, b - a], dtype=torch.int32, device="cuda")
        o1, l1 = H.h3attn_varlen_fwd(c.q[a:b].contiguous(), c.k[a:b].contiguous(), c.v[a:b].contiguous(), cu1,
                                     c.pos_d[a:b].contiguous(), b - a)
        torch.cuda.synchronize()
        assert np.array_equal(bf16_bits(out[a:b]), bf16_bits(o1))
        assert np.array_equal(lse[:, a:b].cpu().numpy(), l1.cpu().numpy())


def test_explicit_scale_and_rope_config(gpu):
    c = Case(ragged_segments(), 2, 64)
    out, lse = c.run(softmax_scale=0.05, theta=500.0, dims=(64, 32, 32))
    o_ref, l_ref = c.oracle_full(scale=0.05, theta=500.0, dims=(64, 32, 32))
    compare(device_to_f64(out), device_to_f64(lse), o_ref, l_ref, label="scale/theta")


def test_generous_max_seqlen_and_empty_segments(gpu):
    import torch
    segs = [[], [wl.visual(1, 5, 7)], [], [wl.visual(1, 1, 3)], []]
    c = Case(segs, 2, 65)
    out, lse = H.h3attn_varlen_fwd(c.q, c.k, c.v, c.cu_d, c.pos_d, c.N)  # max_seqlen = N >= every segment
    torch.cuda.synchronize()
    o_ref, l_ref = c.oracle_full()
    compare(device_to_f64(out), device_to_f64(lse), o_ref, l_ref, label="empty segments")


def test_length_one_segment_returns_v(gpu):
    c = Case([[wl.visual(1, 1, 1)], [wl.audio(1, 1.0, attached=False)]], 4, 66)
    out, lse = c.run()
    assert np.array_equal(bf16_bits(out), c.vb)
    o_ref, l_ref = c.oracle_full()
    compare(device_to_f64(out), device_to_f64(lse), o_ref, l_ref, label="length-1")


def test_zero_tokens_noop(gpu):
    import torch
    q = torch.empty((0, 2, 128), dtype=torch.bfloat16, device="cuda")
    cu = torch.zeros(2, dtype=torch.int32, device="cuda")
    pos = torch.empty((0, 3), dtype=torch.float32, device="cuda")
    ws = torch.empty(256, dtype=torch.uint8, device="cuda")
    out, lse = H.h3attn_varlen_fwd(q, q, q, cu, pos, 0, workspace=ws)
    torch.cuda.synchronize()
    assert out.shape == (0, 2, 128) and lse.shape == (2, 0)


def test_reordered_references_change_output(gpu):
    # A different reference order moves positions on the shared clock, which
    # must show in the attention output beyond the parity tolerance.
    seg = [wl.visual(1, 4, 6), wl.visual(1, 4, 6), wl.visual(2, 4, 6), wl.audio(16, 2, attached=True)]
    swapped = [seg[2], seg[3], seg[0], seg[1]]
    c1 = Case([seg], 2, 67)
    c2 = Case([swapped], 2, 67)
    o1, _ = c1.run()
    o2, _ = c2.run()
    # same token values, different positions: outputs differ by far more than 1e-2 somewhere
    assert np.abs(device_to_f64(o1) - device_to_f64(o2)).max() > 5e-2


# ---- limits of the launch shape --------------------------------------------------------------


def test_long_single_segment_sampled_rows(gpu):
    # One 262,144-token segment (twice the 1344x768 sequence): 1,024 query tiles, 8,192 key tiles
    # per workgroup, token offsets past 2^25 elements.
    segs = [[wl.visual(64, 64, 64)]]
    c = Case(segs, 1, seed=71)
    say(f"long segment: N={c.N} H=1")
    out, lse = c.run()
    out64, lse64 = device_to_f64(out), device_to_f64(lse)
    assert np.all(np.isfinite(out64)) and np.all(np.isfinite(lse64))
    rows = c.sample_rows(n_random=24, seed=71)
    o_ref, l_ref = c.oracle_rows(rows)
    compare(out64[rows], lse64[:, rows], o_ref, l_ref, label=f"long segment ({len(rows)} rows)")


def test_two_thousand_short_segments_full(gpu):
    # 2,000 segments of 0..64 tokens (grid y = 2,000; most tiles ragged, some segments empty).
    rng = np.random.default_rng(72)
    lengths = rng.integers(0, 65, size=2000)
    segs = [[wl.visual(1, 1, int(n))] if n else [] for n in lengths]
    c = Case(segs, 2, seed=72)
    say(f"2000 segments: N={c.N} H=2, empty={int((lengths == 0).sum())}")
    out, lse = c.run()
    o_ref, l_ref = c.oracle_full()
    compare(device_to_f64(out), device_to_f64(lse), o_ref, l_ref, label="2000 segments")


def test_many_heads_full(gpu):
    # 128 heads on a 512-token sequence (grid z = 128; per-token stride 128 x 128 x 2 bytes).
    c = Case([[wl.visual(2, 16, 16)]], 128, seed=73)
    say(f"128 heads: N={c.N} H=128")
    out, lse = c.run()
    o_ref, l_ref = c.oracle_full()
    compare(device_to_f64(out), device_to_f64(lse), o_ref, l_ref, label="128 heads")


@pytest.mark.parametrize("seed_offset", [0, wl.ROBUSTNESS_SEED_OFFSET])
def test_refiner_full(gpu, seed_offset):
    # the token refiner's short path: eight co-batched prompts (77..645 rows), 56 heads, every
    # position 0; every row of every head against the oracle
    cfg = wl.config("refiner")
    seed = cfg["seed"] + seed_offset
    c = Case(cfg["segments"], cfg["heads"], seed)
    say(f"varlen refiner seed {seed}: N={c.N} H={c.heads} lens={c.lens.tolist()}")
    out, lse = c.run()
    o_ref, l_ref = c.oracle_full()
    compare(device_to_f64(out), device_to_f64(lse), o_ref, l_ref, label=f"refiner/{seed}")


def test_running_maximum_moves_every_tile(gpu):
    # Every tile holds larger logits than the one before (the lazy rescale runs on every tile),
    # up to ~50 at the end of the long segment.  There the score operands' 11 significant bits
    # move lse beyond the N(0, 1) bar: rounding this very case's rotated operands to 11 bits
    # (float64 otherwise) moves lse by up to 2.7e-3 and out by up to 1.9e-3.  lse bar at about
    # four times that; out keeps the default bar.
    from test_gpu_fp8 import _rising_case
    c = _rising_case(1200, 2, 192)
    say(f"varlen rising logits: lens={c.lens.tolist()}")
    out, lse = c.run()
    o_ref, l_ref = c.oracle_full()
    compare(device_to_f64(out), device_to_f64(lse), o_ref, l_ref, lse_max=1e-2, label="rising", out_rel=None)


def test_very_large_logits(gpu):
    # q x 64: logits up to ~320.  The score operands carry 11 significant bits, so a logit moves
    # by up to ~|z| 2^-11 times the spread of its products; rounding the rotated operands of this
    # very case to 11 bits (float64 otherwise) moves out by up to 0.048 (mean 4.4e-4) and lse by
    # up to 0.066.  Bars at about four times that.
    c = Case(ragged_segments(), 2, 193, qscale=64.0)
    say(f"varlen very large logits: lens={c.lens.tolist()}")
    out, lse = c.run()
    o_ref, l_ref = c.oracle_full()
    compare(device_to_f64(out), device_to_f64(lse), o_ref, l_ref, out_max=0.2, out_mean=5e-3, lse_max=0.2,
            label="large logits", out_rel=None)


@pytest.mark.parametrize("fp8", [False, True])
def test_short_max_seqlen_truncates_longer_segments(gpu, fp8):
    # max_seqlen below some segments' lengths: each segment is computed as its first max_seqlen
    # tokens alone, both stages agree on that, and later rows of out and lse are left unwritten.
    # Reference: the truncated segments packed as their own batch, bit for bit (segments are
    # computed independently), and the float64 oracle on the truncated batch.
    import torch
    segs = [[wl.visual(1, 10, 30)], [wl.visual(1, 4, 25)], [wl.visual(1, 3, 43)], [wl.visual(1, 1, 7)]]
    c = Case(segs, 2, 74)
    ms = 128
    run = H.h3attn_varlen_fwd_fp8 if fp8 else H.h3attn_varlen_fwd
    out = torch.full_like(c.q, 7.0)
    lse = torch.full((2, c.N), -3.5, dtype=torch.float32, device="cuda")
    run(c.q, c.k, c.v, c.cu_d, c.pos_d, ms, out=out, lse=lse)
    torch.cuda.synchronize()
    keep = np.concatenate([np.arange(int(c.cu[s]), int(c.cu[s]) + min(int(c.lens[s]), ms)) for s in range(len(segs))])
    rest = np.setdiff1d(np.arange(c.N), keep)
    say(f"short max_seqlen {ms}: lens={c.lens.tolist()}, {len(keep)} rows computed, {len(rest)} left")
    assert len(rest) > 0
    ob = bf16_bits(out)
    assert np.all(ob[rest] == bf16_bits(torch.full((1,), 7.0, dtype=torch.bfloat16))[0])
    assert np.all(lse[:, rest].cpu().numpy() == -3.5)
    cu_t = np.concatenate([[0], np.cumsum([min(int(n), ms) for n in c.lens])]).astype(np.int32)
    kt = torch.from_numpy(keep).cuda()
    q_t, k_t, v_t = (x[kt].contiguous() for x in (c.q, c.k, c.v))
    o_t, l_t = run(q_t, k_t, v_t, torch.from_numpy(cu_t).cuda(), c.pos_d[kt].contiguous(), ms)
    torch.cuda.synchronize()
    assert np.array_equal(ob[keep], bf16_bits(o_t))
    assert np.array_equal(lse[:, keep].cpu().numpy(), l_t.cpu().numpy())
    if not fp8:
        o_ref, l_ref = oracle.attention(widen(c.qb[keep]), widen(c.kb[keep]), widen(c.vb[keep]), cu_t, c.pos[keep])
        compare(device_to_f64(o_t), device_to_f64(l_t), o_ref, l_ref, label="short max_seqlen")


def test_nonfinite_inputs_stay_in_their_segment(gpu):
    # a NaN query, an infinite key and a NaN value, each in its own segment, change nothing
    # outside their segment; the NaN row makes its wave take the rare path that moves every row's
    # reference to its exact running maximum, so the other rows of that wave round against it
    c = Case(ragged_segments(), 2, 177)
    nonfinite_isolation(c, lambda c: c.run(), same_row_heads=False)
