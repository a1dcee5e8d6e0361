"""Pins for the oracle's block-quantized FP8 attention (the lossy "SAGE" mode).

The e4m3 rounding is checked against torch's float8_e4m3fn conversion (an
independent library routine) and against hand-worked values; the block scale
against its closed form; the attention against the exact oracle on inputs that
quantization leaves unchanged, against a brute-force loop, and against
invariants that the block structure implies.
"""

import math

import numpy as np
import pytest
import torch

import oracle
from oracle import sage

D = 128


def _e4m3_grid():
    """All finite non-negative e4m3 values, from the encoding: codes 0 .. 126."""
    vals = []
    for code in range(127):
        e, m = code >> 3, code & 7
        vals.append(math.ldexp(m / 8.0, -6) if e == 0 else math.ldexp(1.0 + m / 8.0, e - 7))
    return np.array(vals)


def test_e4m3_grid_closed_form():
    g = _e4m3_grid()
    assert g[0] == 0.0 and g[-1] == 448.0 and len(np.unique(g)) == 127
    assert g[1] == 2.0 ** -9 and g[8] == 2.0 ** -6      # smallest subnormal, smallest normal
    assert np.all(sage.round_e4m3(g) == g)              # every grid value is its own rounding
    assert np.all(sage.round_e4m3(-g) == -g)


def test_e4m3_hand_worked_values():
    cases = {
        1.0625: 1.0,          # midpoint of 1.0 (m=0) and 1.125 (m=1): ties to the even mantissa
        1.1875: 1.25,         # midpoint of 1.125 (m=1) and 1.25 (m=2)
        2.0 ** -10: 0.0,      # midpoint of 0 and the smallest subnormal
        3 * 2.0 ** -10: 2.0 ** -8,
        232.0: 224.0,         # midpoint of 224 (m=6) and 240 (m=7)
        460.0: 448.0,
        0.3: 0.3125,          # 0.3 = 1.2 * 2^-2 -> 1.25 * 2^-2
        -5.1: -5.0,
    }
    for x, want in cases.items():
        assert sage.round_e4m3(x) == want, (x, sage.round_e4m3(x), want)
    with pytest.raises(ValueError):
        sage.round_e4m3(464.0)


def test_e4m3_matches_torch_float8():
    g = _e4m3_grid()
    mids = (g[:-1] + g[1:]) / 2
    rng = np.random.default_rng(3)
    near = np.concatenate([np.nextafter(mids.astype(np.float32), np.float32(0)),
                           np.nextafter(mids.astype(np.float32), np.float32(1000))]).astype(np.float64)
    rand = np.ldexp(rng.uniform(0.5, 1.0, 20000), rng.integers(-14, 9, 20000))
    x = np.concatenate([g, mids, near, rand[rand < 464.0]]).astype(np.float32).astype(np.float64)
    x = np.concatenate([x, -x])
    ref = torch.from_numpy(x).to(torch.float32).to(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(sage.round_e4m3(x), ref)


def test_pow2_scale_exponent_closed_form():
    cases = {448.0: 0, 449.0: 1, 224.0: -1, 224.5: 0, 1.0: -8, 3.5: -7, 3.51: -6, 0.0: 0,
             2.0 ** -200: -127, 896.0: 1, 896.5: 2}
    for amax, e in cases.items():
        assert int(sage.pow2_scale_exponent(amax)) == e, (amax, e)
    rng = np.random.default_rng(4)
    a = np.ldexp(rng.uniform(0.5, 1.0, 5000), rng.integers(-60, 60, 5000))
    e = sage.pow2_scale_exponent(a)
    assert np.all(np.ldexp(a, -e) <= 448.0)             # fits
    assert np.all(np.ldexp(a, -(e - 1)) > 448.0)        # and is the smallest that fits
    assert np.all((np.ldexp(a, -e) > 224.0))


def test_quantize_block_properties():
    rng = np.random.default_rng(5)
    x = rng.standard_normal((16, D)) * 3.0
    qx = sage.quantize_block(x)
    assert np.array_equal(sage.quantize_block(qx), qx)                  # idempotent
    for j in (-9, -1, 3, 20):
        assert np.array_equal(sage.quantize_block(np.ldexp(x, j)), np.ldexp(qx, j))  # power-of-two equivariant
    e = int(sage.pow2_scale_exponent(np.abs(x).max()))
    normal = np.abs(x) >= math.ldexp(1.0, e - 6)
    rel = np.abs(qx - x)[normal] / np.abs(x)[normal]
    assert rel.max() <= 2.0 ** -4                                       # half an ulp of a 3-bit mantissa
    assert 224.0 < np.abs(qx).max() * 2.0 ** -e <= 448.0


def test_key_blocks_start_at_row_zero_and_are_independent():
    rng = np.random.default_rng(6)
    x = rng.standard_normal((40, D))
    base = sage.quantize_key_blocks(x, 16)
    y = x.copy()
    y[17, 5] = 1000.0                                   # a large value in the second block (rows 16..31)
    got = sage.quantize_key_blocks(y, 16)
    assert np.array_equal(got[:16], base[:16]) and np.array_equal(got[32:], base[32:])
    assert not np.array_equal(got[16:32], base[16:32])
    assert np.array_equal(got[32:], sage.quantize_block(x[32:]))        # the short last block stands alone


C_DEFAULT = 1.0 / math.sqrt(D) / math.log(2.0)     # the base-2 logit coefficient at the default scale


def _exact_inputs(n, h, seed):
    """Inputs that the block quantization leaves unchanged.

    k and v: e4m3 values whose every block holds 448.  q: e4m3 values / c, so that the scaled
    rows c q that get quantized are e4m3 values again (up to float32 rounding, which rounds back
    to them); each row holds 416, clear of the 448 boundary where such a rounding could move the
    row's scale.
    """
    rng = np.random.default_rng(seed)
    g = _e4m3_grid()
    pick = lambda shape, top: g[rng.integers(0, top, shape)] * rng.choice([-1.0, 1.0], shape)
    q, k, v = pick((n, h, D), 126), pick((n, h, D), 127), pick((n, h, D), 127)   # code 125 is 416
    q[:, :, 0] = 416.0
    for r0 in range(0, n, 16):
        k[r0, :, 0] = 448.0
    for r0 in range(0, n, 64):
        v[r0, :, 0] = 448.0
    return q / 64.0 / C_DEFAULT, k / 64.0, v     # scales 2^-6: still exact


def test_sage_equals_exact_attention_when_quantization_is_exact():
    n, h = 150, 2
    q, k, v = _exact_inputs(n, h, 7)
    pos = np.zeros((n, 3))                  # identity rotation
    cu = np.array([0, n])
    out_s, lse_s = sage.sage_attention(q, k, v, cu, pos, quantize_p=False)
    out_e, lse_e = oracle.attention(q, k, v, cu, pos)
    assert np.max(np.abs(out_s - out_e)) <= 1e-12 * np.max(np.abs(out_e))
    assert np.max(np.abs(lse_s - lse_e)) <= 1e-12 * np.max(np.abs(lse_e))


def test_sage_p_rounding_stays_within_its_bound():
    n, h = 150, 2
    q, k, v = _exact_inputs(n, h, 8)
    q = q / 8.0                              # softer scores: many probabilities well below the maximum
    pos = np.zeros((n, 3))
    cu = np.array([0, n])
    out_p, lse_p = sage.sage_attention(q, k, v, cu, pos, quantize_p=True)
    out_u, lse_u = sage.sage_attention(q, k, v, cu, pos, quantize_p=False)
    assert np.array_equal(lse_p, lse_u)                # the row sums use unrounded probabilities
    z = (q[:, 0] @ k[:, 0].T) / math.sqrt(D)
    p = np.exp(z - z.max(axis=1, keepdims=True))
    # per probability: half an e4m3 ulp relative, or half the subnormal step (2^-10 / 16) absolute
    err_p = np.maximum(p * 2.0 ** -4, 2.0 ** -14)
    bound = (err_p @ np.abs(v[:, 0])) / p.sum(axis=1, keepdims=True)
    assert np.all(np.abs(out_p[:, 0] - out_u[:, 0]) <= bound * (1 + 1e-12))
    assert np.max(np.abs(out_p - out_u)) > 0           # P rounding is really applied
    # the reported spread: the same per-probability bound, squared over 3, summed with v^2
    _, _, es = sage.sage_attention(q, k, v, cu, pos, quantize_p=False, error_scales=True)
    sig = es["sigma"]
    want = np.sqrt((err_p ** 2 @ v[:, 0] ** 2) / 3.0) / p.sum(axis=1, keepdims=True)
    assert np.allclose(sig[:, 0], want, rtol=1e-12, atol=0)
    zabs = np.array([max(sum(abs(q[i, 0, d] * k[j, 0, d]) for d in range(D)) for j in range(n)) for i in range(0, n, 37)])
    assert np.allclose(es["zabs"][0, ::37], zabs / math.sqrt(D), rtol=1e-12, atol=0)
    # and the actual rounding error, across all rows and dims, is of that size
    ratio = np.abs(out_p - out_u) / sig
    assert np.sqrt(np.mean(ratio ** 2)) < 1.0 and ratio.max() < 6.0


def _scaled_query(x, scale):
    """The row that gets quantized: float32(float32(x) * scale * log2 e), element by element."""
    c = scale / math.log(2.0)
    return np.array([float(np.float32(float(np.float32(t)) * c)) for t in x.ravel()]).reshape(x.shape)


def _brute_sage(q, k, v, cu, scale):
    """Loops over segment, head and query row; quantization from the block definition, written out."""
    N, H, _ = q.shape
    out = np.zeros((N, H, D))
    lse = np.zeros((H, N))

    def qblock(x):
        amax = max(abs(t) for t in x.ravel())
        e = 0
        if amax > 0:
            e = -127
            while amax * 2.0 ** -e > 448.0:
                e += 1
        return np.array([float(sage.round_e4m3(t * 2.0 ** -e)) * 2.0 ** e for t in x.ravel()]).reshape(x.shape)

    for s in range(len(cu) - 1):
        a, b = cu[s], cu[s + 1]
        if a == b:
            continue
        for h in range(H):
            kq = np.concatenate([qblock(k[j:min(j + 16, b), h]) for j in range(a, b, 16)])
            vq = np.concatenate([qblock(v[j:min(j + 64, b), h]) for j in range(a, b, 64)])
            for i in range(a, b):
                qq = qblock(_scaled_query(q[i, h], scale))           # base-2 logits come out of q8 k8
                z = [sum(qq[d] * kq[j][d] for d in range(D)) * math.log(2.0) for j in range(b - a)]
                zm = max(z)
                p = [math.exp(t - zm) for t in z]
                tot = sum(p)
                pq = [float(sage.round_e4m3(t * 16.0)) / 16.0 for t in p]
                for d in range(D):
                    out[i, h, d] = sum(pq[j] * vq[j][d] for j in range(b - a)) / tot
                lse[h, i] = zm + math.log(tot)
    return out, lse


def test_sage_matches_brute_force():
    rng = np.random.default_rng(9)
    cu = np.array([0, 5, 5, 75])            # an empty segment and one that spans several blocks
    n, h = 75, 2
    q, k, v = (rng.standard_normal((n, h, D)) for _ in range(3))
    q, k, v = (x.astype(np.float32).astype(np.float64) for x in (q, k, v))
    pos = np.zeros((n, 3))
    out, lse = sage.sage_attention(q, k, v, cu, pos)
    bo, bl = _brute_sage(q, k, v, cu, 1.0 / math.sqrt(D))
    assert np.max(np.abs(out - bo)) <= 1e-12
    assert np.max(np.abs(lse - bl)) <= 1e-12


def test_sage_segment_isolation_and_row_independence():
    rng = np.random.default_rng(10)
    lens = [37, 70, 21]
    cu = np.concatenate([[0], np.cumsum(lens)])
    n, h = int(cu[-1]), 2
    q, k, v = (rng.standard_normal((n, h, D)) for _ in range(3))
    pos = np.stack([rng.integers(0, 5, n), rng.integers(0, 9, n), rng.integers(0, 9, n)], axis=1).astype(float)
    out, lse = sage.sage_attention(q, k, v, cu, pos)
    for s in range(3):
        a, b = cu[s], cu[s + 1]
        o1, l1 = sage.sage_attention(q[a:b], k[a:b], v[a:b], np.array([0, b - a]), pos[a:b])
        assert np.array_equal(o1, out[a:b]) and np.array_equal(l1, lse[:, a:b])
    q2 = q.copy()
    q2[40] *= 1000.0                        # another query row's magnitude: its own block only
    o2, l2 = sage.sage_attention(q2, k, v, cu, pos)
    keep = np.arange(n) != 40
    assert np.array_equal(o2[keep], out[keep]) and np.array_equal(l2[:, keep], lse[:, keep])
    rows = np.array([0, 36, 37, 80, 106, 127])
    orow, lrow = sage.sage_attention_rows(q, k, v, cu, pos, rows)
    assert np.array_equal(orow, out[rows]) and np.array_equal(lrow, lse[:, rows])


def test_sage_value_scaling_is_exact():
    rng = np.random.default_rng(11)
    n, h = 90, 1
    q, k, v = (rng.standard_normal((n, h, D)) for _ in range(3))
    pos = np.zeros((n, 3))
    cu = np.array([0, n])
    out, _ = sage.sage_attention(q, k, v, cu, pos)
    out2, _ = sage.sage_attention(q, k, np.ldexp(v, 7), cu, pos)
    assert np.array_equal(out2, np.ldexp(out, 7))


def test_sage_close_to_exact_on_the_tiny_workload():
    from joint_sequence_attention_amd import workloads as wl
    cfg = wl.config("tiny")
    cu, pos = oracle.layout(cfg["segments"])
    n = int(cu[-1])
    qb, kb, vb = wl.random_qkv(n, cfg["heads"], cfg["seed"])
    q, k, v = (wl.bf16_bits_to_f32(b).astype(np.float64) for b in (qb, kb, vb))
    out_s, lse_s = sage.sage_attention(q, k, v, cu, pos)
    out_e, lse_e = oracle.attention(q, k, v, cu, pos)
    # lossy, but not far: 3-bit mantissas on every operand
    assert np.max(np.abs(lse_s - lse_e)) < 0.05
    assert np.max(np.abs(out_s - out_e)) < 0.1
    assert np.mean(np.abs(out_s - out_e)) < 0.01


def test_rotation_error_bound_covers_float32_rotation():
    # An independent float32 evaluation of the rotation (numpy float32 arithmetic, angles
    # rounded to float32 first) stays within the bound the oracle states for fp32 kernels.
    from oracle.rope import rope_frequencies
    rng = np.random.default_rng(12)
    n, h = 300, 2
    x = rng.standard_normal((n, h, D)).astype(np.float32).astype(np.float64)
    pos = np.stack([rng.integers(0, 300, n), rng.integers(0, 48, n), rng.integers(0, 84, n)], axis=1).astype(float)
    exact = oracle.rope(x, pos)
    y = np.empty_like(exact)
    off = 0
    for axis, width in enumerate((32, 48, 48)):
        om = rope_frequencies(10000.0, width).astype(np.float32)
        phi = pos[:, axis].astype(np.float32)[:, None] * om[None, :]
        c, s = np.cos(phi)[:, None, :], np.sin(phi)[:, None, :]
        x0 = x[:, :, off:off + width:2].astype(np.float32)
        x1 = x[:, :, off + 1:off + width:2].astype(np.float32)
        y[:, :, off:off + width:2] = x0 * c - x1 * s
        y[:, :, off + 1:off + width:2] = x0 * s + x1 * c
        off += width
    bound = sage.rotation_error_bound(x, pos)
    assert np.all(np.abs(y - exact) <= bound)
    # pairs at angle 0 (position 0 on their axis) carry no error: there the bound is 0, and met exactly
    assert (bound == 0).any() and np.all(y[bound == 0] == x[bound == 0])


def test_quantize_block_margin():
    rng = np.random.default_rng(13)
    x = rng.standard_normal((16, D))
    w = np.full_like(x, 1e-3)
    q, change = sage.quantize_block_margin(x, w)
    assert np.array_equal(q, sage.quantize_block(x))
    # a value whose window holds no midpoint rounds the same way anywhere inside it
    for _ in range(20):
        xp = x + rng.uniform(-1, 1, x.shape) * w
        qp = sage.quantize_block(xp)
        if int(sage.pow2_scale_exponent(np.abs(xp).max())) != int(sage.pow2_scale_exponent(np.abs(x).max())):
            continue
        moved = qp != q
        assert np.all(change[moved] > 0)
        assert np.all(np.abs(qp - q)[moved] <= change[moved])
    # an exact midpoint is flagged with one step (1.0625 sits between 1.0 and 1.125 at scale 2^0)
    blk = np.zeros(4)
    blk[0] = 416.0                            # scale 2^0, clear of the boundary at 448
    blk[1] = 1.0625
    q, change = sage.quantize_block_margin(blk, np.full(4, 1e-9))
    assert change[1] == 0.125 and change[0] == 0 and change[2] == 0
    # a block maximum next to a scale boundary flags the whole block
    blk[0] = 448.0 * (1 + 1e-12)
    q, change = sage.quantize_block_margin(blk, np.full(4, 1e-6))
    assert np.all(change > 0)


# ---- Skip-Softmax rule -----------------------------------------------------------------------


def _skip_case(seed, n=200, h=1, qscale=3.0):
    """Local attention: q_i . k_j = a^2 sum_m cos((i - j) w_m) + noise peaks at i = j, so tiles
    far after a block's own keys carry almost no weight."""
    rng = np.random.default_rng(seed)
    w = 0.5 * np.power(10.0, -np.arange(D // 2) / (D // 2))
    ang = np.arange(n)[:, None] * w[None, :]
    f = np.concatenate([np.cos(ang), np.sin(ang)], axis=1) * qscale / 1.5
    q = (f + 0.3 * rng.standard_normal((n, D)))[:, None, :].repeat(h, axis=1)
    k = (f + 0.3 * rng.standard_normal((n, D)))[:, None, :].repeat(h, axis=1)
    v = rng.standard_normal((n, h, D))
    return q, k, v, np.zeros((n, 3)), np.array([0, n])


def test_skip_with_negligible_threshold_is_dense():
    q, k, v, pos, cu = _skip_case(20)
    dense = sage.sage_attention(q, k, v, cu, pos)
    tiny = sage.sage_attention(q, k, v, cu, pos, skip_threshold=1e-300)
    assert np.array_equal(dense[0], tiny[0]) and np.array_equal(dense[1], tiny[1])


def test_skip_drops_a_negligible_tile():
    # Tile 1 (keys 64..127) points away from every query: its logits sit ~40 below tile 0's,
    # so it is skipped and the rows equal attention over tile 0 alone.
    rng = np.random.default_rng(21)
    n = 128
    u = rng.standard_normal(D)
    u /= np.linalg.norm(u)
    q = (8.0 * u + 0.1 * rng.standard_normal((n, D)))[:, None, :]
    k = np.empty((n, 1, D))
    k[:64, 0] = 4.0 * u + 0.5 * rng.standard_normal((64, D))
    k[64:, 0] = -4.0 * u + 0.5 * rng.standard_normal((64, D))
    v = rng.standard_normal((n, 1, D))
    pos = np.zeros((n, 3))
    out, lse, es = sage.sage_attention(q, k, v, np.array([0, n]), pos, skip_threshold=0.05, error_scales=True)
    ref_o, ref_l = sage.sage_attention_rows(q[:, :, :], np.concatenate([k[:64], k[:64]]),
                                            np.concatenate([v[:64], np.zeros_like(v[:64])]),
                                            np.array([0, 64, 128]), pos, np.arange(64))
    # rows 0..63 against a segment holding only tile 0: same quantization of tile 0's blocks
    assert np.allclose(out[:64], ref_o, rtol=0, atol=1e-12) and np.allclose(lse[:, :64], ref_l, rtol=0, atol=1e-12)
    assert np.all(es["skipped"] == 0.5)


def _brute_skip(q8, k8, v8, scale, thr):
    """Loops: per 32-row block, per 64-key tile in order, the rule written out; exact softmax."""
    R, S = q8.shape[0], k8.shape[0]
    z = [[sum(q8[i, d] * k8[j, d] for d in range(D)) * scale for j in range(S)] for i in range(R)]
    keep = [[True] * S for _ in range(R)]
    for b0 in range(0, R, 32):
        rows = range(b0, min(R, b0 + 32))
        running = {i: -math.inf for i in rows}
        for t0 in range(0, S, 64):
            tmax = {i: max(z[i][t0:t0 + 64]) for i in rows}
            if all(tmax[i] < running[i] + math.log(thr) for i in rows):
                for i in rows:
                    for j in range(t0, min(S, t0 + 64)):
                        keep[i][j] = False
            for i in rows:
                running[i] = max(running[i], tmax[i])
    out = np.zeros((R, D))
    lse = np.zeros(R)
    for i in range(R):
        ks = [j for j in range(S) if keep[i][j]]
        zm = max(z[i][j] for j in ks)
        e = {j: math.exp(z[i][j] - zm) for j in ks}
        tot = sum(e.values())
        for d in range(D):
            out[i, d] = sum(e[j] * v8[j, d] for j in ks) / tot
        lse[i] = zm + math.log(tot)
    return out, lse, keep


def test_skip_matches_brute_force():
    q, k, v, pos, cu = _skip_case(22, n=230, qscale=3.0)
    out, lse, es = sage.sage_attention(q, k, v, cu, pos, quantize_p=False, skip_threshold=0.05, error_scales=True)
    # the same quantized operands, through the brute-force rule
    q8 = sage.quantize_rows(_scaled_query(q[:, 0], 1.0 / math.sqrt(D)))
    k8 = sage.quantize_key_blocks(k[:, 0], 16)
    v8 = sage.quantize_key_blocks(v[:, 0], 64)
    bo, bl, keep = _brute_skip(q8, k8, v8, math.log(2.0), 0.05)
    assert np.max(np.abs(out[:, 0] - bo)) <= 1e-12 and np.max(np.abs(lse[0] - bl)) <= 1e-12
    share = 1.0 - np.array([sum(keep[i][::64]) for i in range(len(keep))]) / 4.0
    assert np.allclose(es["skipped"][0], share)
    assert share.max() > 0                  # the case really skips something


def test_skip_is_monotone_in_the_threshold_and_decided_per_block():
    q, k, v, pos, cu = _skip_case(23, n=230, qscale=3.0)
    shares = []
    for thr in (1e-6, 1e-3, 0.05, 0.3):
        _, _, es = sage.sage_attention(q, k, v, cu, pos, skip_threshold=thr, error_scales=True)
        shares.append(es["skipped"][0])
    for lo, hi in zip(shares, shares[1:]):
        assert np.all(hi >= lo)
    # every row of a 32-row block shares the block's decisions
    for b0 in range(0, 230, 32):
        assert np.all(shares[2][b0:b0 + 32] == shares[2][b0])
    # one row that needs tile 1 keeps it for its whole block: give row 5 a key of tile 1 that it
    # matches strongly
    k2 = k.copy()
    k2[70, 0] = q[5, 0] * 3.0
    _, _, es2 = sage.sage_attention(q, k2, v, cu, pos, skip_threshold=0.05, error_scales=True)
    assert es2["skipped"][0][0] <= shares[2][0]
