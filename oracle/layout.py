"""Oracle: packed-sequence layout and shared-clock positions (float64 -> float32).

Test infrastructure only; see the package docstring.

The steps, in the order the pages imply them:

1. A packed batch is a list of segments, one attention document per request
   (vLLM-Omni "MiniMax-H3" recipe, "Step execution and continuous batching").
   Each segment starts its own clock at 0.
2. Inside a segment the items are read in reference order, references in
   front of the generated rows ("minimax-h3-reference" README, "AoTI-compiled
   blocks"), and each reference advances the shared audio/video rotary clock
   ("minimax-h3-reference" README, "References").
3. A visual grid (T, H, W) flattens with w fastest, then h, then t, the
   way the DiT flattens a latent video into tokens ("Day 0 Support for
   MiniMax-H3 on AMD Instinct GPUs", "The diffusion transformer (DiT)"), and
   its token at (t, h, w) sits at position (clock + t, h, w).  The clock then
   advances by T.
4. An audio run carries a time position only: (clock_start + a(i), 0, 0).
   Attached audio (a video's own soundtrack) starts where that video started
   and does not move the clock again; a standalone audio reference starts at
   the current clock and advances it by its span.  a(i) = i * span / n, or
   that value rounded half to even for the "round" rule.
5. Positions are formed in float64 and cast to float32 for device arithmetic
   ("MiniMax H3 on Moore Threads MUSA", "MUSA validation").
6. cu_seqlens is the int32 prefix sum of segment lengths.
"""

from __future__ import annotations

import math

import numpy as np


def round_half_even(x: float) -> float:
    """Round to the nearest integer, ties to even (IEEE default rounding)."""
    f = math.floor(x)
    d = x - f
    if d > 0.5:
        return float(f + 1)
    if d < 0.5:
        return float(f)
    return float(f if f % 2 == 0 else f + 1)


def _audio_offset(i: int, n: int, span: float, rule: str) -> float:
    a = i * span / n
    if rule == "round":
        return round_half_even(a)
    if rule == "linear":
        return a
    raise ValueError(f"unknown audio position rule {rule!r}")


def layout(segments):
    """Return (cu_seqlens int32 [B+1], pos_thw float32 [N, 3]) for the packed batch."""
    rows = []
    cu = [0]
    for seg in segments:
        clock = 0.0
        last_visual_start = None
        for item in seg:
            kind = item["kind"]
            if kind == "visual":
                T, H, W = item["T"], item["H"], item["W"]
                for t in range(T):
                    for h in range(H):
                        for w in range(W):
                            rows.append((clock + t, float(h), float(w)))
                last_visual_start = clock
                clock += T
            elif kind == "audio":
                n, span = item["n"], float(item["span"])
                if item["attached"]:
                    if last_visual_start is None:
                        raise ValueError("attached audio needs a visual item before it")
                    start = last_visual_start
                else:
                    start = clock
                for i in range(n):
                    rows.append((start + _audio_offset(i, n, span, item["rule"]), 0.0, 0.0))
                if not item["attached"]:
                    clock += span
            else:
                raise ValueError(f"unknown item kind {kind!r}")
        cu.append(len(rows))
    pos64 = np.array(rows, dtype=np.float64).reshape(-1, 3)
    return np.array(cu, dtype=np.int32), pos64.astype(np.float32)
