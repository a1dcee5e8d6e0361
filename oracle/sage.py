"""Oracle: block-quantized FP8 (e4m3) attention, the lossy "SAGE" mode, in float64.

Test infrastructure only; see the package docstring.

What the page fixes.  The vLLM-Omni "MiniMax-H3" recipe, section "Attention
Backends", describes two optional lossy optimizations of the long main DiT
attention on its datacenter-Blackwell backend:

* SAGE attention quantization: Q and K in FP8 e4m3 with one scale per query
  token (query block size 1) and one scale per 16 keys (key block size 16);
  P and V are always FP8 in that kernel.
* Skip-Softmax sparse attention with a direct threshold (0.05 in its
  example): a low threshold skips only clearly negligible tiles of keys.

It gives nothing else: no scale format, no V or P block, no tile size, and
no statement of where the softmax scale enters.  Those points are read here as
follows, each for a reason that does not depend on any implementation.

R1  Scale format.  One power-of-two scale 2^e per block, e the smallest
    integer with amax * 2^-e <= 448 (the largest finite e4m3 value), limited
    to [-127, 127]; a block of zeros takes 2^0.  Reason: plainest to check.
    Scaling by a power of two is exact, so every quantized element is one
    round-to-nearest-even of x * 2^-e that a reader can verify bit for bit;
    of the power-of-two scales this is the finest that never saturates.
R2  e4m3 flavour.  The OCP 8-bit floating-point E4M3 format the page names
    ("fp8_e4m3": finite, largest 448, no infinities), round to nearest even
    (the IEEE default).
R3  Q blocks.  One block per (token, head) row of 128 rotated dims: the
    page's query block size 1.
R4  K blocks.  Per head, 16 consecutive keys counted from each segment's
    first key (a segment's last block may be shorter): the page's key block
    size 16.  A segment is one attention document, so no block spans two.
R5  V blocks.  Per head, one scale per value channel (each of the 128 dims)
    over all keys of the segment.  Reason: the page says V is FP8 and gives
    no block.  The P.V product sums over keys, out_d = sum_j p_j v_jd / l, so
    a scale that is constant along the keys of channel d factors out of that
    sum exactly, whereas one that changed along the keys would not; per-channel
    scaling of V is also the published SageAttention2 method's choice (Zhang
    et al., "SageAttention2", FP8 quantization of P and V).
R6  P.  Softmax itself is exact: the row maximum m, the probabilities
    p = exp(z - m) and their sum l are taken in full precision, and P is
    rounded to FP8 only where it enters the product with V.  Its scale comes
    from R1 applied to P's bound known in advance: relative to the row
    maximum every p lies in (0, 1], so e = -8 and p8 = e4m3(256 p) / 256.
    lse = m + ln l and out = (p8 v8) / l.
R7  Quantization precision.  Rotated Q and K are held in float32 (the
    precision of device arithmetic: "MiniMax H3 on Moore Threads MUSA",
    "MUSA validation") before they are scaled and rounded; V enters as given.
R8  Where the softmax scale enters.  The logits are z = scale * (q8 . k8),
    the scale applied to the product of the quantized operands: the page
    quantizes Q and K themselves, and the scale belongs to the softmax, as in
    the exact attention.

Skip-Softmax readings.

S1  Decisions are per query row, and keys go in tiles of 64 counted from the
    segment start, in key order.  Reason: the page speaks of tiles and gives
    no size; 64 keys is four of the page's 16-key K blocks, so a tile never
    splits a quantization block.  A per-row rule makes each row's result a
    function of its own logits alone, which is the plainest to check.
S2  Rule.  For row r, tile T is left out when max_{j in T} z_rj is below
    M_r(T) + ln(threshold), where M_r(T) is the row's largest logit over the
    tiles before T (minus infinity for the first tile, which is always kept).
    A left-out tile's maximum lies below M_r(T), so M_r is also the running
    maximum over the kept tiles.
S3  Effect.  A left-out tile adds nothing to the row: out and lse are R6 over
    the kept keys.
S4  The rule sees the logits of R8, the scores of the quantized operands.

Alternative roundings.  A kernel rotates in its own fp32 arithmetic, within
2^-22 (1 + |phi|)(|x0| + |x1|) of the exact rotation (angle rounding, sin/cos
and the multiply-adds); this oracle's float32 values are within a quarter of
that.  Where a midpoint of the e4m3 grid (or a power-of-two boundary of a
block scale) lies inside that window, both roundings are correct.
``error_scales`` reports, per row, how far such elements can move lse and
out (first order, with margin), and how far a skip decision next to the
threshold can, so that a test can tell a valid alternative from a wrong one.
V is not rotated: its quantization has no alternatives.
"""

from __future__ import annotations

import math

import numpy as np

from .rope import rope

E4M3_MAX = 448.0
E4M3_MIN_NORMAL_EXP = -6          # smallest normal 2**-6
E4M3_MANTISSA_BITS = 3
Q_BLOCK = 1                        # R3: query rows per scale
K_BLOCK = 16                       # R4: keys per scale
P_SCALE_LOG2 = 8                   # R6: P is quantized as 256 p, p in (0, 1]
SKIP_KEY_TILE = 64                 # S1: keys skipped together
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
    """R1: smallest integer e with amax * 2**-e <= 448, limited to [-127, 127]; 0 for amax == 0."""
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
    """R3, Q-style: one block per row of the last axis (any leading shape)."""
    x = np.asarray(x, dtype=np.float64)
    e = pow2_scale_exponent(np.abs(x).max(axis=-1))[..., None]
    return np.ldexp(round_e4m3(np.ldexp(x, -e)), e)


def quantize_key_blocks(x, block=K_BLOCK) -> np.ndarray:
    """R4: quantize x [S, D] in blocks of ``block`` consecutive rows from row 0 (last block may be short)."""
    x = np.asarray(x, dtype=np.float64)
    out = np.empty_like(x)
    for r0 in range(0, x.shape[0], block):
        out[r0:r0 + block] = quantize_block(x[r0:r0 + block])
    return out


def quantize_channels(x) -> np.ndarray:
    """R5: quantize x [S, D] with one scale per column (channel) over all S rows."""
    x = np.asarray(x, dtype=np.float64)
    if x.shape[0] == 0:
        return x.copy()
    e = pow2_scale_exponent(np.abs(x).max(axis=0))[None, :]
    return np.ldexp(round_e4m3(np.ldexp(x, -e)), e)


def quantize_p(p) -> np.ndarray:
    """R6: probabilities relative to the row maximum, p in [0, 1], as e4m3(256 p) / 256."""
    return np.ldexp(round_e4m3(np.ldexp(np.asarray(p, dtype=np.float64), P_SCALE_LOG2)), -P_SCALE_LOG2)


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


def quantize_blocks_margin(xb, wb):
    """Quantize blocks, and bound how much a rounding within +-w of each value could differ.

    xb, wb: float64 [n_blocks, m], one block per row.  Returns (values the
    blocks stand for, change), both [n_blocks, m]: change is 0 where every value
    within +-w rounds the same way, else the largest move another valid
    rounding makes.  Another evaluation may also find the block's largest
    magnitude anywhere within +-wmax of this one's, and so a neighbouring
    power-of-two scale where that crosses a boundary; each possible scale's
    roundings of x - w, x and x + w count.  (A power of two leaves the e4m3
    rounding of normal values alone: a scale change moves only values in or
    near the subnormal range.)
    """
    xb = np.asarray(xb, dtype=np.float64)
    wb = np.asarray(wb, dtype=np.float64)
    a = np.abs(xb).max(axis=1) if xb.shape[1] else np.zeros(xb.shape[0])
    wmax = wb.max(axis=1) if xb.shape[1] else np.zeros(xb.shape[0])
    e = pow2_scale_exponent(a)[:, None]
    q = np.ldexp(round_e4m3(np.ldexp(xb, -e)), e)
    change = np.zeros_like(xb)
    for e_alt in (pow2_scale_exponent(np.maximum(a - wmax, 0.0))[:, None], e,
                  pow2_scale_exponent(a + wmax)[:, None]):
        for sgn in (-1.0, 0.0, 1.0):
            s_alt = np.clip(np.ldexp(xb + sgn * wb, -e_alt), -463.0, 463.0)
            change = np.maximum(change, np.abs(np.ldexp(round_e4m3(s_alt), e_alt) - q))
    return q, change


def quantize_block_margin(x, w):
    """One block (any shape) through quantize_blocks_margin."""
    x = np.asarray(x, dtype=np.float64)
    q, change = quantize_blocks_margin(x.reshape(1, -1), np.asarray(w, dtype=np.float64).reshape(1, -1))
    return q.reshape(x.shape), change.reshape(x.shape)


def _to_f32(x):
    return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)


def _quantized_segment_kv(kr_seg, kw_seg, v_seg):
    """Per head: K in 16-key blocks with rounding margins (R4), V per channel over the segment (R5)."""
    S, H, D = kr_seg.shape
    nb = (S + K_BLOCK - 1) // K_BLOCK
    pad = nb * K_BLOCK - S                 # zero rows: they change no block's largest magnitude
    kq = np.empty_like(kr_seg)
    kc = np.empty_like(kr_seg)
    vq = np.empty_like(v_seg)
    for h in range(H):
        xb = np.concatenate([kr_seg[:, h], np.zeros((pad, D))]).reshape(nb, K_BLOCK * D)
        wb = np.concatenate([kw_seg[:, h], np.zeros((pad, D))]).reshape(nb, K_BLOCK * D)
        q, c = quantize_blocks_margin(xb, wb)
        kq[:, h] = q.reshape(nb * K_BLOCK, D)[:S]
        kc[:, h] = c.reshape(nb * K_BLOCK, D)[:S]
        vq[:, h, :] = quantize_channels(v_seg[:, h, :])
    return kq, kc, vq


def tile_maxima(m, tile=SKIP_KEY_TILE):
    """Per row, the largest entry of each run of ``tile`` columns (the last run may be short): [R, n_tiles]."""
    R, S = m.shape
    full = S // tile
    parts = [m[:, :full * tile].reshape(R, full, tile).max(axis=2)] if full else []
    if S > full * tile:
        parts.append(m[:, full * tile:].max(axis=1, keepdims=True))
    return np.concatenate(parts, axis=1) if parts else np.zeros((R, 0))


def skip_decisions(z, threshold, tile=SKIP_KEY_TILE, delta=None):
    """S1-S2 for a set of rows: z float64 [R, S] (natural-unit logits) -> (skip, ambiguous), bool [R, n_tiles].

    delta: float64 [R, n_tiles], how far evaluation error can move each logit of each tile (None:
    0).  A decision is ambiguous when moving every tile's largest logit within its error could
    change it: the running maximum then lies between the largest of the earlier tiles' maxima
    moved down and the largest moved up.
    """
    R, S = z.shape
    n_tiles = (S + tile - 1) // tile
    skip = np.zeros((R, n_tiles), dtype=bool)
    amb = np.zeros((R, n_tiles), dtype=bool)
    if not threshold or threshold <= 0 or R == 0:
        return skip, amb
    ln_thr = math.log(threshold)
    d = np.zeros((R, n_tiles)) if delta is None else np.asarray(delta, dtype=np.float64)
    tm = tile_maxima(z, tile)

    def before(x):
        """Per tile, the largest of x over the earlier tiles (-inf for the first)."""
        return np.maximum.accumulate(np.concatenate([np.full((R, 1), -np.inf), x[:, :-1]], axis=1), axis=1)

    margin = before(tm) + ln_thr - tm                  # > 0: the row leaves the tile out
    skip = margin > 0
    lo = before(tm - d) + ln_thr - (tm + d)
    hi = before(tm + d) + ln_thr - (tm - d)
    amb = (lo <= 0) & (hi > 0)
    return skip, amb


def tile_logit_errors(q8, qc, k8, kc, scale, tile=SKIP_KEY_TILE):
    """Per (row, key tile), how far a logit of the tile can move, float64 [R, n_tiles].

    Two parts: fp32 evaluation of the 128 products, at most 2^-14 of their summed magnitudes,
    bounded here by |scale| |q8_r|_2 |k8_j|_2 (Cauchy-Schwarz) with the tile's largest key norm;
    and alternative roundings next to an e4m3 midpoint (qc, kc: how far each element may move),
    |scale| sum_d (|q8_rd| kc_jd + qc_rd |k8_jd|), taken over the tile's keys.  Only keys and rows
    that have an alternative enter the second part.
    """
    R, S = q8.shape[0], k8.shape[0]
    sc = abs(scale)
    knorm = np.sqrt((k8 * k8).sum(axis=1))
    kmax = tile_maxima(knorm[None, :], tile)[0]
    err = 2.0 ** -14 * sc * np.sqrt((q8 * q8).sum(axis=1))[:, None] * kmax[None, :]
    jk = np.nonzero(kc.any(axis=1))[0]                 # keys with an alternative, ascending
    if len(jk):
        m = (np.abs(q8) @ kc[jk].T) * sc               # [R, len(jk)]
        t_of = jk // tile
        starts = np.concatenate([[0], np.nonzero(np.diff(t_of))[0] + 1])
        err[:, t_of[starts]] += np.maximum.reduceat(m, starts, axis=1)
    rq = np.nonzero(qc.any(axis=1))[0]
    if len(rq):
        err[rq] += tile_maxima((qc[rq] @ np.abs(k8).T) * sc, tile)
    return err


def skip_counts(q, k, cu_seqlens, pos, threshold, *, theta=10000.0, dims=(32, 48, 48), scale=None,
                row_block=512):
    """S1-S2 over every row: (left out, ambiguous), int64 [H, N]: per (head, row) the key tiles the
    rule leaves out and the decisions among them that an evaluation error could flip.

    The same quantized operands, rule and error bounds as ``sage_attention_rows``, without the
    outputs.
    """
    q = np.asarray(q)
    k = np.asarray(k)
    pos = np.asarray(pos, dtype=np.float64)
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    N, H, D = q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    left = np.zeros((H, N), dtype=np.int64)
    amb_n = np.zeros((H, N), dtype=np.int64)
    for s in range(len(cu) - 1):
        a, b = int(cu[s]), int(cu[s + 1])
        if a == b:
            continue
        k_seg = np.asarray(k[a:b], dtype=np.float64)
        kr = _to_f32(rope(k_seg, pos[a:b], theta, dims))
        kw = 2.0 * rotation_error_bound(k_seg, pos[a:b], theta, dims)
        kq, kc, _ = _quantized_segment_kv(kr, kw, np.zeros_like(kr))
        for r0 in range(a, b, row_block):
            r1 = min(b, r0 + row_block)
            q_rows = np.asarray(q[r0:r1], dtype=np.float64)
            qr = _to_f32(rope(q_rows, pos[r0:r1], theta, dims))
            qw = 2.0 * rotation_error_bound(q_rows, pos[r0:r1], theta, dims)
            qq, qc = quantize_blocks_margin(qr.reshape(-1, D), qw.reshape(-1, D))
            qq, qc = qq.reshape(qr.shape), qc.reshape(qr.shape)
            for h in range(H):
                z = (qq[:, h] @ kq[:, h].T) * scale
                err = tile_logit_errors(qq[:, h], qc[:, h], kq[:, h], kc[:, h], scale)
                sk, am = skip_decisions(z, threshold, SKIP_KEY_TILE, err)
                left[h, r0:r1] = sk.sum(axis=1)
                amb_n[h, r0:r1] = am.sum(axis=1)
    return left, amb_n


def _segment_head(q8, k8, v8, scale, quantize, qc=None, kc=None, keep=None, amb=None, tile=SKIP_KEY_TILE):
    """One head of one segment for a set of query rows (R6, R8).

    keep: bool [R, S], the keys that count (all when None).  amb: bool [R, n_tiles], tiles whose
    skip decision could go either way for the row (their effect is added to the error scales).
    """
    z = (q8 @ k8.T) * scale
    zk = z if keep is None else np.where(keep, z, -np.inf)
    m = zk.max(axis=1, keepdims=True)
    p = np.exp(zk - m)
    l = p.sum(axis=1, keepdims=True)
    pw = quantize_p(p) if quantize else p
    out = (pw @ v8) / l
    lse = m[:, 0] + np.log(l[:, 0])
    # Spread of the P rounding: each probability moves by at most half an e4m3 ulp, 2^-4 of
    # itself, or half the subnormal step, 2^-10 / 256; a rounding error spread evenly over that
    # interval has standard deviation (bound) / sqrt(3).
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
    threshold) can move lse and out; "skipped" [len(heads), R], the row's key
    tiles left out, "tiles" [R], its segment's key tiles, and
    "skip_ambiguous" [len(heads), R], how many of the row's decisions could go
    either way.

    skip_threshold: apply the Skip-Softmax rule S1-S3 (None or 0: every tile counts).
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
    seg_of = np.searchsorted(cu, rows, side="right") - 1
    R = len(rows)
    out = np.zeros((R, len(heads), D), dtype=np.float64)
    lse = np.zeros((len(heads), R), dtype=np.float64)
    sig = np.zeros((R, len(heads), D), dtype=np.float64)
    zabs = np.zeros((len(heads), R), dtype=np.float64)
    lflip = np.zeros((len(heads), R), dtype=np.float64)
    oflip = np.zeros((R, len(heads), D), dtype=np.float64)
    skipped = np.zeros((len(heads), R), dtype=np.int64)
    ambiguous = np.zeros((len(heads), R), dtype=np.int64)
    tiles = np.zeros(R, dtype=np.int64)
    for s in np.unique(seg_of):
        a, b = int(cu[s]), int(cu[s + 1])
        sel = np.nonzero(seg_of == s)[0]
        k_seg = np.asarray(k[a:b][:, heads, :], dtype=np.float64)
        kr = _to_f32(rope(k_seg, pos[a:b], theta, dims))
        kw = 2.0 * rotation_error_bound(k_seg, pos[a:b], theta, dims)
        vs = np.asarray(v[a:b][:, heads, :], dtype=np.float64)
        kq, kc, vq = _quantized_segment_kv(kr, kw, vs)
        r_seg = rows[sel]
        q_rows = np.asarray(q[r_seg][:, heads, :], dtype=np.float64)
        qr = _to_f32(rope(q_rows, pos[r_seg], theta, dims))
        qw = 2.0 * rotation_error_bound(q_rows, pos[r_seg], theta, dims)
        qq, qc = quantize_blocks_margin(qr.reshape(-1, D), qw.reshape(-1, D))   # R3: one block per row
        qq, qc = qq.reshape(qr.shape), qc.reshape(qr.shape)
        S_seg = b - a
        tiles[sel] = (S_seg + SKIP_KEY_TILE - 1) // SKIP_KEY_TILE
        for j in range(len(heads)):
            for r0 in range(0, len(sel), 512):
                part = slice(r0, r0 + 512)
                qp, qcp = qq[part, j, :], qc[part, j, :]
                keep = amb = None
                if skip_threshold:
                    z = (qp @ kq[:, j, :].T) * scale
                    err = tile_logit_errors(qp, qcp, kq[:, j, :], kc[:, j, :], scale)
                    sk, amb = skip_decisions(z, skip_threshold, SKIP_KEY_TILE, err)
                    keep = ~np.repeat(sk, SKIP_KEY_TILE, axis=1)[:, :S_seg]
                    del z
                o, l, (sg, za2, lf, of) = _segment_head(qp, kq[:, j, :], vq[:, j, :], scale, quantize_p, qcp,
                                                        kc[:, j, :], keep, amb, SKIP_KEY_TILE)
                idx = sel[part]
                out[idx, j, :] = o
                lse[j, idx] = l
                sig[idx, j, :] = sg
                zabs[j, idx] = za2
                lflip[j, idx] = lf
                oflip[idx, j, :] = of
                if keep is not None:
                    skipped[j, idx] = sk.sum(axis=1)
                    ambiguous[j, idx] = amb.sum(axis=1)
    scales = {"sigma": sig, "zabs": zabs, "lse_flip": lflip, "out_flip": oflip, "skipped": skipped,
              "tiles": tiles, "skip_ambiguous": ambiguous}
    return (out, lse, scales) if error_scales else (out, lse)


def sage_attention(q, k, v, cu_seqlens, pos, **kw):
    """Full block-quantized FP8 attention: (out float64 [N, H, D], lse float64 [H, N]) (and the error scales)."""
    return sage_attention_rows(q, k, v, cu_seqlens, pos, None, None, **kw)
