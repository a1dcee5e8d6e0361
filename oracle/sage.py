"""Oracle: block-quantized FP8 (e4m3) attention, the lossy "SAGE" mode, in float64.

Test infrastructure only; see the package docstring.

The vLLM-Omni "MiniMax-H3" recipe ("Attention Backends", the optional lossy
optimizations of its datacenter-Blackwell backend) offers SAGE attention
quantization for the long main DiT attention: Q and K in FP8 e4m3 with one
scale per query token (query block size 1) and one scale per 16 keys (key
block size 16), and P and V always in FP8.  It is lossy by design; the recipe
asks to compare it against dense output before adopting it.

The steps, in that order, with the readings taken where the page is silent:

1. Rotate Q and K (``rope``), then hold the rotated values in float32, the
   precision device arithmetic uses (the position contract in "MiniMax H3 on
   Moore Threads MUSA", "MUSA validation").  Quantization decisions are taken
   on those float32 values.
2. Block scales are powers of two: a block with largest magnitude a gets
   2**e with e the smallest integer for which a * 2**-e <= 448 (the largest
   finite e4m3 value), limited to [-127, 127]; a block of zeros gets 2**0.
   Reading: the page gives block sizes, not the scale format; power-of-two
   scales keep the scaling exact and match the hardware's 8-bit exponent
   block scales.
3. Q: one block per (token, head) row of 128 dims.  K: per head, blocks of 16
   consecutive keys counted from the first key of each segment (the last block
   of a segment may be shorter).  V: per head, blocks of 64 consecutive keys
   from the segment start, all 128 dims (reading: the page says V is FP8 but
   gives no V block size).  Each element is x8 = e4m3(x * 2**-e), rounded to
   nearest even, and stands for x8 * 2**e.
4. The softmax scale enters through the queries: each rotated query row is
   multiplied by c = scale * log2(e) and held in float32 before it is
   quantized, so q8 k8^T is the row's logits in base 2; z = (q8 k8^T) ln 2.
   Reading: the page does not say where the scale enters; putting it into Q
   before quantization gives a kernel base-2 logits straight from the matrix
   core.  Exact softmax per row: m = max z, p = exp(z - m), l = sum p,
   lse = m + ln l.
5. P in FP8 (``quantize_p``): p8 = e4m3(p * 16) / 16, i.e. probabilities
   relative to the row maximum, scaled by 2**4 so that values down to 2**-10
   stay normal (reading: the page gives no P scale).  out = (p8 v8) / l.
   A kernel that evaluates softmax online rounds its probabilities relative
   to a running maximum instead, so its P rounding differs element by element;
   both are draws of the same rounding noise, which the GPU tests bound.

Skip-Softmax (optional, ``skip_threshold``).  The same recipe section offers
a second lossy option, Skip-Softmax sparse attention with a direct threshold
(0.05 there): tiles of keys whose probabilities are all below the threshold,
relative to the running maximum, are left out.  The page names the knob, not
the rule; the reading taken here, stated so that the result is a function of
the logits alone:

* queries go in blocks of 32 rows and keys in tiles of 64 (the FP8 kernel's
  units), both counted from the segment start, tiles in key order;
* for each row, the running maximum before tile T is the largest logit of
  the tiles before T (minus infinity for the first tile), whether or not
  they were skipped;
* tile T is skipped for a block when every valid row r of the block has
  max_{j in T} z_rj < running_max_r + ln(threshold);
* a skipped tile contributes nothing to that block's softmax: out and lse
  are exact softmax over the keys of the tiles that are kept.

Rounding decisions near a midpoint.  A kernel rotates in its own fp32
arithmetic, within 2^-22 (1 + |phi|)(|x0| + |x1|) of the exact rotation
(angle rounding, sin/cos and the multiply-adds); this oracle's float32 values
are within a quarter of that.  Where a midpoint of the e4m3 grid (or a
power-of-two boundary of a block scale) lies inside that window, both
roundings are correct.  ``error_scales`` reports, per row, how far such
elements can move lse and out (first order, with margin), so that a test can
tell a valid alternative rounding from a wrong one.
"""

from __future__ import annotations

import math

import numpy as np

from .rope import rope

E4M3_MAX = 448.0
E4M3_MIN_NORMAL_EXP = -6          # smallest normal 2**-6
E4M3_MANTISSA_BITS = 3
Q_BLOCK = 1                        # query rows per scale
K_BLOCK = 16                       # keys per scale
V_BLOCK = 64                       # keys per scale (all dims)
P_SCALE_LOG2 = 4                   # P is quantized as p * 2**4
SKIP_QUERY_BLOCK = 32              # Skip-Softmax: query rows that decide together
SKIP_KEY_TILE = 64                 # Skip-Softmax: keys skipped together
LN2 = math.log(2.0)


def round_e4m3(x) -> np.ndarray:
    """Round float64 values to the nearest e4m3 (OCP "fn") value, ties to even.

    e4m3: 1 sign bit, 4 exponent bits (bias 7), 3 mantissa bits; normals from
    2**-6 to 448, subnormals in steps of 2**-9.  Inputs must satisfy
    |x| < 464 (the midpoint above 448); larger values have no finite encoding.
    """
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    if np.any(~np.isfinite(a)) or np.any(a >= 464.0):
        raise ValueError("value outside the finite e4m3 range")
    _, e = np.frexp(a)                               # a = f * 2**e, f in [0.5, 1)
    expo = np.maximum(e - 1, E4M3_MIN_NORMAL_EXP)    # binade of a, subnormals share the lowest one
    ulp = np.ldexp(1.0, expo - E4M3_MANTISSA_BITS)
    r = np.rint(a / ulp) * ulp                       # np.rint rounds half to even
    r = np.minimum(r, E4M3_MAX)                      # 448 < a < 464 rounds down to 448
    return np.copysign(r, x)


def pow2_scale_exponent(amax) -> np.ndarray:
    """Smallest integer e with amax * 2**-e <= 448, limited to [-127, 127]; 0 for amax == 0."""
    amax = np.asarray(amax, dtype=np.float64)
    if np.any(amax < 0) or np.any(~np.isfinite(amax)):
        raise ValueError("amax must be finite and >= 0")
    safe = np.where(amax > 0, amax, 1.0)
    e = np.ceil(np.log2(safe / E4M3_MAX)).astype(np.int64)
    # log2 may land one off next to powers of two: step to the exact smallest e
    e = np.where(np.ldexp(safe, -e) > E4M3_MAX, e + 1, e)
    e = np.where(np.ldexp(safe, -(e - 1)) <= E4M3_MAX, e - 1, e)
    e = np.where(amax > 0, e, 0)
    return np.clip(e, -127, 127)


def quantize_block(x) -> np.ndarray:
    """Quantize one block (any shape) with its power-of-two scale; returns the values it stands for."""
    x = np.asarray(x, dtype=np.float64)
    e = int(pow2_scale_exponent(np.abs(x).max() if x.size else 0.0))
    return np.ldexp(round_e4m3(np.ldexp(x, -e)), e)


def quantize_rows(x) -> np.ndarray:
    """Q-style quantization: one block per row of the last axis (any leading shape)."""
    x = np.asarray(x, dtype=np.float64)
    e = pow2_scale_exponent(np.abs(x).max(axis=-1))[..., None]
    return np.ldexp(round_e4m3(np.ldexp(x, -e)), e)


def quantize_key_blocks(x, block) -> np.ndarray:
    """Quantize x [S, D] in blocks of ``block`` consecutive rows from row 0 (last block may be short)."""
    x = np.asarray(x, dtype=np.float64)
    out = np.empty_like(x)
    for r0 in range(0, x.shape[0], block):
        out[r0:r0 + block] = quantize_block(x[r0:r0 + block])
    return out


ROTATION_ERROR = 2.0 ** -22          # fp32 rotation error coefficient (see the module docstring)


def rotation_error_bound(x, pos, theta=10000.0, dims=(32, 48, 48)) -> np.ndarray:
    """Per element of rope(x): 2^-22 (1 + |phi|)(|x0| + |x1|) over its rotation pair, float64 [N, H, D].

    A pair that turns by phi = 0 gets 0: sin 0 = 0 and cos 0 = 1 are exact in
    float32, so x0 * 1 - x1 * 0 and x0 * 0 + x1 * 1 give the pair back unchanged.
    """
    from .rope import rope_frequencies
    x = np.abs(np.asarray(x, dtype=np.float64))
    pos = np.asarray(pos, dtype=np.float64)
    out = np.empty_like(x)
    offset = 0
    for axis, width in enumerate(dims):
        phi = pos[:, axis][:, None] * rope_frequencies(theta, width)[None, :]      # [N, width/2]
        pair = x[:, :, offset:offset + width:2] + x[:, :, offset + 1:offset + width:2]
        b = np.where((phi == 0.0)[:, None, :], 0.0, ROTATION_ERROR * (1.0 + np.abs(phi))[:, None, :] * pair)
        out[:, :, offset:offset + width:2] = b
        out[:, :, offset + 1:offset + width:2] = b
        offset += width
    return out


def quantize_block_margin(x, w):
    """Quantize one block, and bound how much a rounding within +-w of each value could differ.

    Returns (values the block stands for, change): change is 0 where every
    value within +-w rounds the same way, else the largest move the other
    rounding makes (one e4m3 step; for the whole block when its scale itself
    could differ).
    """
    x = np.asarray(x, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    a = float(np.abs(x).max()) if x.size else 0.0
    wmax = float(w.max()) if w.size else 0.0
    e = int(pow2_scale_exponent(a))
    s = np.ldexp(x, -e)
    r = round_e4m3(s)
    q = np.ldexp(r, e)
    if int(pow2_scale_exponent(max(a - wmax, 0.0))) != int(pow2_scale_exponent(a + wmax)):
        # the block scale may be 2^(e-1) or 2^(e+1): every value may move by a step at the coarser scale
        change = np.abs(x) * 2.0 ** -3 + np.ldexp(1.0, e + 1 - 9)
        return q, change
    ws = np.ldexp(w, -e)
    lo = round_e4m3(s - ws)
    hi = round_e4m3(s + ws)
    change = np.ldexp(np.maximum(np.abs(lo - r), np.abs(hi - r)), e)
    return q, change


def _to_f32(x):
    return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)


def _quantized_segment_kv(kr_seg, kw_seg, v_seg):
    """Per-head K (16-key blocks, with rounding margins) and V (64-key blocks) of one segment, [S, H, D] each."""
    kq = np.empty_like(kr_seg)
    kc = np.empty_like(kr_seg)
    vq = np.empty_like(v_seg)
    for h in range(kr_seg.shape[1]):
        for r0 in range(0, kr_seg.shape[0], K_BLOCK):
            kq[r0:r0 + K_BLOCK, h], kc[r0:r0 + K_BLOCK, h] = quantize_block_margin(kr_seg[r0:r0 + K_BLOCK, h],
                                                                                 kw_seg[r0:r0 + K_BLOCK, h])
        vq[:, h, :] = quantize_key_blocks(v_seg[:, h, :], V_BLOCK)
    return kq, kc, vq


def _segment_head(q8, k8, v8, scale, quantize_p, qc=None, kc=None, keep=None, amb=None, tile=64):
    """One head of one segment for a set of query rows.

    keep: bool [R, S], the keys that count (all when None).  amb: bool [R, n_tiles], tiles whose
    skip decision could go either way for the row's block (their effect is added to the error
    scales).
    """
    z = (q8 @ k8.T) * scale
    zk = z if keep is None else np.where(keep, z, -np.inf)
    m = zk.max(axis=1, keepdims=True)
    p = np.exp(zk - m)
    l = p.sum(axis=1, keepdims=True)
    pw = np.ldexp(round_e4m3(np.ldexp(p, P_SCALE_LOG2)), -P_SCALE_LOG2) if quantize_p else p
    out = (pw @ v8) / l
    lse = m[:, 0] + np.log(l[:, 0])
    # Spread of the P rounding: each probability moves by at most half an e4m3 ulp, 2^-4 of
    # itself, or half the subnormal step, 2^-14 in these units; a rounding error spread evenly
    # over that interval has standard deviation (bound) / sqrt(3).
    e = np.where(p > 0, np.maximum(p * 2.0 ** -4, 2.0 ** -(10 + P_SCALE_LOG2)), 0.0)
    sigma = np.sqrt(((e * e) @ (v8 * v8)) / 3.0) / l
    # Largest sum of absolute products behind one logit of the row: the scale of
    # the rounding error any finite-precision evaluation of the row's scores has.
    zabs = (np.abs(q8) @ np.abs(k8).T).max(axis=1) * abs(scale)
    # Alternative roundings of elements next to a midpoint (qc, kc: how far each may move): the
    # logits move by at most dz, lse by the probability-weighted dz, out by the weighted dz times
    # the distance of v from out, plus the same for the lse shift (first order; 25 % margin).
    if qc is None:
        qc = np.zeros_like(q8)
    if kc is None:
        kc = np.zeros_like(k8)
    dz = (np.abs(q8) @ kc.T + qc @ np.abs(k8).T) * abs(scale)
    pd = p * dz
    lse_flip = pd.sum(axis=1) / l[:, 0]
    av = np.abs(v8)
    ao = np.abs(out)
    out_flip = (pd @ av + pd.sum(axis=1, keepdims=True) * ao + lse_flip[:, None] * (p @ av + l * ao)) / l
    lse_flip = 1.25 * lse_flip
    out_flip = 1.25 * out_flip
    if amb is not None and amb.any():
        # A tile whose decision could go the other way: with weight w = (sum of its probabilities
        # relative to this row's maximum) / l, keeping or dropping it moves lse by at most
        # w / (1 - w) and out by that times (max |v| over the tile + |out|).
        pall = np.exp(z - m)
        S = k8.shape[0]
        for t in np.nonzero(amb.any(axis=0))[0]:
            rows_t = amb[:, t]
            j0, j1 = t * tile, min(S, (t + 1) * tile)
            w = pall[rows_t, j0:j1].sum(axis=1) / l[rows_t, 0]
            wb = w / np.maximum(1.0 - w, 1e-3)
            vmax = np.abs(v8[j0:j1]).max(axis=0)
            lse_flip[rows_t] += wb
            out_flip[rows_t] += wb[:, None] * (vmax[None, :] + ao[rows_t])
    return out, lse, (sigma, zabs, lse_flip, out_flip)


def skip_decisions(z, valid, threshold, tile=64, delta=None):
    """Skip-Softmax decisions for one query block.

    z: float64 [R, S] logits of the block's rows (natural units); valid: bool [R], the rows that
    exist.  Returns (skip bool [n_tiles], ambiguous bool [n_tiles]).  A decision is ambiguous
    when moving each row's logits by up to delta [R] (its evaluation error) could change it.
    """
    R, S = z.shape
    n_tiles = (S + tile - 1) // tile
    skip = np.zeros(n_tiles, dtype=bool)
    amb = np.zeros(n_tiles, dtype=bool)
    if not threshold or threshold <= 0 or not valid.any():
        return skip, amb
    ln_thr = math.log(threshold)
    zv = z[valid]
    d = np.zeros(zv.shape[0]) if delta is None else np.asarray(delta)[valid]
    running = np.full(zv.shape[0], -np.inf)
    for t in range(n_tiles):
        tm = zv[:, t * tile:min(S, (t + 1) * tile)].max(axis=1)
        margin = running + ln_thr - tm           # > 0: this row lets the tile go
        skip[t] = bool(np.all(margin > 0))
        could_skip = bool(np.all(margin > -2 * d))
        could_keep = bool(np.any(margin < 2 * d))
        amb[t] = could_skip and could_keep
        running = np.maximum(running, tm)
    return skip, amb


def sage_attention_rows(q, k, v, cu_seqlens, pos, rows=None, heads=None, *, theta=10000.0, dims=(32, 48, 48),
                        scale=None, quantize_p=True, error_scales=False, skip_threshold=None):
    """Block-quantized FP8 attention for selected query rows (all rows when ``rows`` is None).

    Keys and values of a row's segment are always quantized whole, exactly as
    for the full computation.  Returns (out float64 [R, len(heads), D],
    lse float64 [len(heads), R]), and with ``error_scales`` also a dict with
    "sigma", the standard deviation of ``out`` that rounding P to e4m3 causes,
    float64 [R, len(heads), D]; "zabs", per row the largest
    scale * sum_i |q8_i k8_i| over its keys, float64 [len(heads), R]; and
    "lse_flip" [len(heads), R] and "out_flip" [R, len(heads), D], how far
    alternative roundings next to a midpoint (and skip decisions next to the
    threshold) can move lse and out; "skipped" [len(heads), R], the share of
    the row's key tiles left out, and "skip_ambiguous" [len(heads), R], how
    many of its block's decisions could go either way.

    skip_threshold: apply the Skip-Softmax rule above (None or 0: every tile
    counts).  Each requested row's whole 32-row block is evaluated, since the
    decision belongs to the block.
    """
    q = np.asarray(q)
    k = np.asarray(k)
    v = np.asarray(v)
    pos = np.asarray(pos, dtype=np.float64)
    if q.shape != k.shape or q.shape != v.shape or q.ndim != 3:
        raise ValueError("q, k, v must share one [N, H, D] shape")
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    if cu[0] != 0 or cu[-1] != q.shape[0] or np.any(np.diff(cu) < 0):
        raise ValueError("cu_seqlens must rise from 0 to N")
    N, H, D = q.shape
    heads = list(range(H)) if heads is None else [int(h) for h in heads]
    rows = np.arange(N, dtype=np.int64) if rows is None else np.asarray(rows, dtype=np.int64)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    c = scale / LN2                     # base-2 logit coefficient, folded into the queries
    seg_of = np.searchsorted(cu, rows, side="right") - 1
    out = np.zeros((len(rows), len(heads), D), dtype=np.float64)
    lse = np.zeros((len(heads), len(rows)), dtype=np.float64)
    sig = np.zeros((len(rows), len(heads), D), dtype=np.float64)
    zabs = np.zeros((len(heads), len(rows)), dtype=np.float64)
    lflip = np.zeros((len(heads), len(rows)), dtype=np.float64)
    oflip = np.zeros((len(rows), len(heads), D), dtype=np.float64)
    skipped = np.zeros((len(heads), len(rows)), dtype=np.float64)
    ambiguous = np.zeros((len(heads), len(rows)), dtype=np.int64)
    for s in np.unique(seg_of):
        a, b = int(cu[s]), int(cu[s + 1])
        sel = np.nonzero(seg_of == s)[0]
        k_seg = np.asarray(k[a:b][:, heads, :], dtype=np.float64)
        kr = _to_f32(rope(k_seg, pos[a:b], theta, dims))
        kw = 2.0 * rotation_error_bound(k_seg, pos[a:b], theta, dims)
        vs = np.asarray(v[a:b][:, heads, :], dtype=np.float64)
        kq, kc, vq = _quantized_segment_kv(kr, kw, vs)
        # rows to evaluate: the requested ones, or with skipping their whole 32-row blocks
        want = rows[sel] - a
        if skip_threshold:
            blocks = np.unique(want // SKIP_QUERY_BLOCK)
            ev = np.concatenate([np.arange(bq * SKIP_QUERY_BLOCK, min(b - a, (bq + 1) * SKIP_QUERY_BLOCK))
                                 for bq in blocks])
        else:
            ev = want
        q_rows = np.asarray(q[a + ev][:, heads, :], dtype=np.float64)
        qr = _to_f32(_to_f32(rope(q_rows, pos[a + ev], theta, dims)) * c)
        # the rotation window times c, plus the float32 roundings of c and of the product
        qw = 2.0 * rotation_error_bound(q_rows, pos[a + ev], theta, dims) * abs(c) + np.abs(qr) * 2.0 ** -22
        qq = np.empty_like(qr)
        qc = np.empty_like(qr)
        for i in range(qr.shape[0]):
            for j in range(qr.shape[1]):
                qq[i, j], qc[i, j] = quantize_block_margin(qr[i, j], qw[i, j])
        pos_in_ev = {int(r): i for i, r in enumerate(ev)}
        pick = np.array([pos_in_ev[int(r)] for r in want])
        S_seg = b - a
        n_tiles = (S_seg + SKIP_KEY_TILE - 1) // SKIP_KEY_TILE
        for j in range(len(heads)):
            # 512-row chunks hold whole 32-row blocks: every block but a segment's last is full
            for r0 in range(0, len(ev), 512):
                part = slice(r0, r0 + 512)
                keep = amb = None
                if skip_threshold:
                    qp, qcp = qq[part, j, :], qc[part, j, :]
                    z = (qp @ kq[:, j, :].T) * LN2
                    za = (np.abs(qp) @ np.abs(kq[:, j, :]).T).max(axis=1) * LN2
                    dzmax = ((np.abs(qp) @ kc[:, j, :].T + qcp @ np.abs(kq[:, j, :]).T) * LN2).max(axis=1)
                    delta = 2.0 ** -14 * za + dzmax
                    evp = ev[part]
                    keep = np.ones((len(evp), S_seg), dtype=bool)
                    amb = np.zeros((len(evp), n_tiles), dtype=bool)
                    for bq in np.unique(evp // SKIP_QUERY_BLOCK):
                        in_b = (evp // SKIP_QUERY_BLOCK) == bq
                        sk, am = skip_decisions(z[in_b], np.ones(int(in_b.sum()), dtype=bool), skip_threshold,
                                                SKIP_KEY_TILE, delta[in_b])
                        keys_off = np.repeat(sk, SKIP_KEY_TILE)[:S_seg]
                        keep[np.ix_(in_b, keys_off)] = False
                        amb[in_b] = am
                    del z
                o, l, (sg, za2, lf, of) = _segment_head(
                    qq[part, j, :], kq[:, j, :], vq[:, j, :], LN2, quantize_p, qc[part, j, :], kc[:, j, :], keep,
                    amb, SKIP_KEY_TILE)
                idx = np.arange(len(ev))[part]
                sel_here = np.nonzero(np.isin(pick, idx))[0]
                loc = pick[sel_here] - r0
                out[sel[sel_here], j, :] = o[loc]
                lse[j, sel[sel_here]] = l[loc]
                sig[sel[sel_here], j, :] = sg[loc]
                zabs[j, sel[sel_here]] = za2[loc]
                lflip[j, sel[sel_here]] = lf[loc]
                oflip[sel[sel_here], j, :] = of[loc]
                if keep is not None:
                    kept_tiles = keep[loc][:, ::SKIP_KEY_TILE].sum(axis=1)
                    skipped[j, sel[sel_here]] = 1.0 - kept_tiles / n_tiles
                    ambiguous[j, sel[sel_here]] = amb[loc].sum(axis=1)
    scales = {"sigma": sig, "zabs": zabs, "lse_flip": lflip, "out_flip": oflip, "skipped": skipped,
              "skip_ambiguous": ambiguous}
    return (out, lse, scales) if error_scales else (out, lse)


def sage_attention(q, k, v, cu_seqlens, pos, **kw):
    """Full block-quantized FP8 attention: (out float64 [N, H, D], lse float64 [H, N]) (and the error scales)."""
    return sage_attention_rows(q, k, v, cu_seqlens, pos, None, None, **kw)
