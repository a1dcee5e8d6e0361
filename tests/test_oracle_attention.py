"""Pins for the oracle's attention: brute force, closed forms, invariants, library routines."""

import math

import numpy as np
import pytest
import torch

import oracle

D = 128


def _rand(n, h, seed, scale=1.0):
    rng = np.random.default_rng(seed)
    return [rng.standard_normal((n, h, D)) * scale for _ in range(3)]


def _pos(n, seed):
    rng = np.random.default_rng(seed)
    p = np.zeros((n, 3))
    p[:, 0] = rng.integers(0, 8, n)
    p[:, 1] = rng.integers(0, 24, n)
    p[:, 2] = rng.integers(0, 42, n)
    return p


def _brute_rope_row(x, p):
    """One token's rotation, pair by pair, straight from the closed form."""
    out = list(x)
    offsets = ((0, 32), (32, 48), (80, 48))
    for axis, (off, width) in enumerate(offsets):
        for j in range(width // 2):
            w = 10000.0 ** (-2.0 * j / width)
            phi = p[axis] * w
            a, b = x[off + 2 * j], x[off + 2 * j + 1]
            out[off + 2 * j] = a * math.cos(phi) - b * math.sin(phi)
            out[off + 2 * j + 1] = a * math.sin(phi) + b * math.cos(phi)
    return out


def _brute_attention(q, k, v, cu, pos):
    """Triple loop over segment, head, query; scores by explicit dot products."""
    N, H, _ = q.shape
    out = np.zeros_like(q)
    lse = np.zeros((H, N))
    for s in range(len(cu) - 1):
        a, b = cu[s], cu[s + 1]
        for h in range(H):
            kr = [_brute_rope_row(k[j, h], pos[j]) for j in range(a, b)]
            for i in range(a, b):
                qr = _brute_rope_row(q[i, h], pos[i])
                z = [sum(qr[d] * kr[j - a][d] for d in range(D)) / math.sqrt(D) for j in range(a, b)]
                zmax = max(z)
                e = [math.exp(t - zmax) for t in z]
                tot = sum(e)
                for d in range(D):
                    out[i, h, d] = sum(e[j] * v[a + j, h, d] for j in range(b - a)) / tot
                lse[h, i] = zmax + math.log(tot)
    return out, lse


def test_brute_force_tiny():
    cu = [0, 3, 3, 8, 9]       # includes an empty and a length-1 segment
    n = cu[-1]
    q, k, v = _rand(n, 2, 10)
    pos = _pos(n, 11)
    o, l = oracle.attention(q, k, v, np.array(cu), pos)
    ob, lb = _brute_attention(q, k, v, cu, pos)
    np.testing.assert_allclose(o, ob, rtol=0, atol=1e-13)
    np.testing.assert_allclose(l, lb, rtol=0, atol=1e-13)


def test_constant_values_give_constant_output():
    n = 40
    q, k, _ = _rand(n, 2, 12)
    c = np.random.default_rng(13).standard_normal((1, 2, D))
    v = np.repeat(c, n, axis=0)
    o, _ = oracle.attention(q, k, v, np.array([0, 17, 40]), _pos(n, 14))
    np.testing.assert_allclose(o, v, rtol=0, atol=1e-13)


def test_zero_query_gives_segment_mean():
    cu = np.array([0, 5, 18, 30])
    n = 30
    _, k, v = _rand(n, 3, 15)
    q = np.zeros((n, 3, D))
    o, l = oracle.attention(q, k, v, cu, _pos(n, 16))
    for s in range(3):
        a, b = cu[s], cu[s + 1]
        np.testing.assert_allclose(o[a:b], np.repeat(v[a:b].mean(axis=0, keepdims=True), b - a, 0), atol=1e-13)
        np.testing.assert_allclose(l[:, a:b], math.log(b - a), atol=1e-13)


def test_length_one_segment():
    q, k, v = _rand(1, 2, 17)
    pos = np.array([[3.0, 4.0, 5.0]])
    o, l = oracle.attention(q, k, v, np.array([0, 1]), pos)
    np.testing.assert_allclose(o, v, atol=1e-15)
    qr = oracle.rope(q, pos)
    kr = oracle.rope(k, pos)
    for h in range(2):
        np.testing.assert_allclose(l[h, 0], float(qr[0, h] @ kr[0, h]) / math.sqrt(D), atol=1e-13)


def test_two_key_closed_form():
    # with two keys the weights are a logistic function of the score gap
    q, k, v = _rand(2, 1, 18)
    pos = np.zeros((2, 3))
    o, l = oracle.attention(q, k, v, np.array([0, 2]), pos)
    for i in range(2):
        z0 = float(q[i, 0] @ k[0, 0]) / math.sqrt(D)
        z1 = float(q[i, 0] @ k[1, 0]) / math.sqrt(D)
        w1 = 1.0 / (1.0 + math.exp(z0 - z1))
        np.testing.assert_allclose(o[i, 0], (1 - w1) * v[0, 0] + w1 * v[1, 0], atol=1e-14)
        np.testing.assert_allclose(l[0, i], math.log(math.exp(z0) + math.exp(z1)), atol=1e-13)


def test_softmax_rows_sum_to_one():
    # weights recovered by putting one-hot value vectors through the oracle
    n = 24
    q, k, _ = _rand(n, 1, 19, scale=2.0)
    pos = _pos(n, 20)
    v = np.zeros((n, 1, D))
    for j in range(n):
        v[j, 0, j] = 1.0
    o, _ = oracle.attention(q, k, v, np.array([0, n]), pos)
    w = o[:, 0, :n]
    assert np.all(w >= 0)
    np.testing.assert_allclose(w.sum(axis=1), 1.0, atol=1e-13)


def test_segment_isolation_bitwise():
    cu = np.array([0, 37, 90, 128])
    n = 128
    q, k, v = _rand(n, 2, 21)
    pos = _pos(n, 22)
    o, l = oracle.attention(q, k, v, cu, pos)
    for s in range(3):
        a, b = cu[s], cu[s + 1]
        os_, ls_ = oracle.attention(q[a:b], k[a:b], v[a:b], np.array([0, b - a]), pos[a:b])
        assert np.array_equal(o[a:b], os_)
        assert np.array_equal(l[:, a:b], ls_)


def test_key_permutation_equivariance():
    n = 50
    q, k, v = _rand(n, 2, 23)
    pos = _pos(n, 24)
    o, l = oracle.attention(q, k, v, np.array([0, n]), pos)
    perm = np.random.default_rng(25).permutation(n)
    # permute every token (q, k, v and positions together): outputs permute the same way
    o2, l2 = oracle.attention(q[perm], k[perm], v[perm], np.array([0, n]), pos[perm])
    np.testing.assert_allclose(o2, o[perm], atol=1e-12)
    np.testing.assert_allclose(l2, l[:, perm], atol=1e-12)


def test_output_shift_invariance():
    n = 64
    q, k, v = _rand(n, 2, 26)
    pos = _pos(n, 27)
    o, l = oracle.attention(q, k, v, np.array([0, 20, n]), pos)
    o2, l2 = oracle.attention(q, k, v, np.array([0, 20, n]), pos + np.array([[5.0, 3.0, -2.0]]))
    np.testing.assert_allclose(o2, o, rtol=0, atol=1e-12)
    np.testing.assert_allclose(l2, l, rtol=0, atol=1e-12)


def test_matches_torch_sdpa_float64():
    # library cross-check of the attention core on rotated inputs
    cu = np.array([0, 100, 160])
    n = 160
    q, k, v = _rand(n, 3, 28, scale=1.5)
    pos = _pos(n, 29)
    o, l = oracle.attention(q, k, v, cu, pos)
    qr = torch.from_numpy(oracle.rope(q, pos))
    kr = torch.from_numpy(oracle.rope(k, pos))
    vt = torch.from_numpy(v)
    for s in range(2):
        a, b = cu[s], cu[s + 1]
        ref = torch.nn.functional.scaled_dot_product_attention(
            qr[a:b].transpose(0, 1), kr[a:b].transpose(0, 1), vt[a:b].transpose(0, 1)).transpose(0, 1)
        np.testing.assert_allclose(o[a:b], ref.numpy(), rtol=0, atol=1e-12)
        z = torch.einsum("ihd,jhd->hij", qr[a:b], kr[a:b]) / math.sqrt(D)
        np.testing.assert_allclose(l[:, a:b], torch.logsumexp(z, dim=-1).numpy(), rtol=0, atol=1e-12)


def test_attention_rows_agrees_with_full():
    cu = np.array([0, 70, 70, 200])
    n = 200
    q, k, v = _rand(n, 3, 30)
    pos = _pos(n, 31)
    o, l = oracle.attention(q, k, v, cu, pos, row_block=16)
    rows = np.array([0, 5, 69, 70, 150, 199])
    heads = [2, 0]
    orow, lrow = oracle.attention_rows(q, k, v, cu, pos, rows, heads)
    np.testing.assert_allclose(orow, o[rows][:, heads], atol=1e-13)
    np.testing.assert_allclose(lrow, l[heads][:, rows], atol=1e-13)


def test_row_blocking_does_not_change_results():
    n = 90
    q, k, v = _rand(n, 1, 32)
    pos = _pos(n, 33)
    o1, l1 = oracle.attention(q, k, v, np.array([0, n]), pos, row_block=7)
    o2, l2 = oracle.attention(q, k, v, np.array([0, n]), pos, row_block=512)
    np.testing.assert_allclose(o1, o2, atol=1e-14)
    np.testing.assert_allclose(l1, l2, atol=1e-14)


def test_explicit_scale():
    n = 12
    q, k, v = _rand(n, 1, 34)
    pos = np.zeros((n, 3))
    o, l = oracle.attention(q, k, v, np.array([0, n]), pos, scale=0.05)
    z = q[:, 0] @ k[:, 0].T * 0.05
    w = np.exp(z - z.max(1, keepdims=True))
    w /= w.sum(1, keepdims=True)
    np.testing.assert_allclose(o[:, 0], w @ v[:, 0], atol=1e-13)


def test_rejects_bad_cu():
    q, k, v = _rand(4, 1, 35)
    with pytest.raises(ValueError):
        oracle.attention(q, k, v, np.array([0, 3]), np.zeros((4, 3)))
    with pytest.raises(ValueError):
        oracle.attention(q, k, v, np.array([0, 3, 2, 4]), np.zeros((4, 3)))
