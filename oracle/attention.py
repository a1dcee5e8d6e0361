"""Oracle: exact per-segment softmax attention in float64.

Test infrastructure only; see the package docstring.

The DiT attends jointly over the whole packed video+audio sequence, with no
causal order ("Day 0 Support for MiniMax-H3 on AMD Instinct GPUs", "The
diffusion transformer (DiT)"), and a packed batch keeps one attention document
per request (vLLM-Omni "MiniMax-H3" recipe, "Step execution and continuous
batching"): a token sees every token of its own segment and nothing else.

For segment s, head h, with Q~ = rope(Q), K~ = rope(K):

    z   = Q~_s K~_s^T * scale          scale = 1 / sqrt(d) unless given
    m   = rowmax(z)
    p   = exp(z - m)
    l   = rowsum(p)
    out = (p V_s) / l
    lse = m + ln l                      natural log, one value per (head, row)

Softmax is exact per row (not online).  Query rows are processed in blocks of
``row_block`` only to bound memory; each block sees all keys of its segment.
"""

from __future__ import annotations

import math

import numpy as np

from .rope import rope


def _check(q, k, v, cu_seqlens, pos):
    if q.shape != k.shape or q.shape != v.shape or q.ndim != 3:
        raise ValueError("q, k, v must share one [N, H, D] shape")
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    if cu[0] != 0 or cu[-1] != q.shape[0] or np.any(np.diff(cu) < 0):
        raise ValueError("cu_seqlens must rise from 0 to N")
    if pos.shape != (q.shape[0], 3):
        raise ValueError("pos must be [N, 3]")
    return cu


def _segment_head(qr_rows, kr_seg, v_seg, scale):
    z = (qr_rows @ kr_seg.T) * scale
    m = z.max(axis=1, keepdims=True)
    p = np.exp(z - m)
    l = p.sum(axis=1, keepdims=True)
    out = (p @ v_seg) / l
    lse = m[:, 0] + np.log(l[:, 0])
    return out, lse


def attention(q, k, v, cu_seqlens, pos, *, theta=10000.0, dims=(32, 48, 48), scale=None, row_block=512):
    """Full oracle: returns (out float64 [N, H, D], lse float64 [H, N])."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    pos = np.asarray(pos, dtype=np.float64)
    cu = _check(q, k, v, cu_seqlens, pos)
    N, H, D = q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    qr = rope(q, pos, theta, dims)
    kr = rope(k, pos, theta, dims)
    out = np.zeros((N, H, D), dtype=np.float64)
    lse = np.zeros((H, N), dtype=np.float64)
    for s in range(len(cu) - 1):
        a, b = int(cu[s]), int(cu[s + 1])
        if a == b:
            continue
        for h in range(H):
            kr_seg = kr[a:b, h, :]
            v_seg = v[a:b, h, :]
            for r0 in range(a, b, row_block):
                r1 = min(b, r0 + row_block)
                o, l = _segment_head(qr[r0:r1, h, :], kr_seg, v_seg, scale)
                out[r0:r1, h, :] = o
                lse[h, r0:r1] = l
    return out, lse


def attention_rows(q, k, v, cu_seqlens, pos, rows, heads=None, *, theta=10000.0, dims=(32, 48, 48),
                   scale=None):
    """Oracle for selected query rows only (each against all keys of its segment).

    Returns (out float64 [len(rows), len(heads), D], lse float64 [len(heads), len(rows)]).
    Used where the full oracle would take too long; every selected row is
    computed exactly as in ``attention``.
    """
    q = np.asarray(q)
    k = np.asarray(k)
    v = np.asarray(v)
    pos = np.asarray(pos, dtype=np.float64)
    cu = _check(q, k, v, cu_seqlens, pos)
    N, H, D = q.shape
    if heads is None:
        heads = list(range(H))
    heads = [int(h) for h in heads]
    rows = np.asarray(rows, dtype=np.int64)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    seg_of = np.searchsorted(cu, rows, side="right") - 1
    out = np.zeros((len(rows), len(heads), D), dtype=np.float64)
    lse = np.zeros((len(heads), len(rows)), dtype=np.float64)
    for s in np.unique(seg_of):
        a, b = int(cu[s]), int(cu[s + 1])
        sel = np.nonzero(seg_of == s)[0]
        kr = rope(np.asarray(k[a:b][:, heads, :], dtype=np.float64), pos[a:b], theta, dims)
        vs = np.asarray(v[a:b][:, heads, :], dtype=np.float64)
        qr = rope(np.asarray(q[rows[sel]][:, heads, :], dtype=np.float64), pos[rows[sel]], theta, dims)
        for j in range(len(heads)):
            o, l = _segment_head(qr[:, j, :], kr[:, j, :], vs[:, j, :], scale)
            out[sel, j, :] = o
            lse[j, sel] = l
    return out, lse
