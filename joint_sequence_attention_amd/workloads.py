"""Seeded synthetic workloads: sequence structure and random bf16 Q/K/V.

This module is the one place both sides of a parity check draw their inputs
from.  It holds the *shape* of each workload (which visual grids and audio
runs make up each packed sequence, in reference order) and a seeded random
number recipe.  It holds none of the method's arithmetic: it does not compute
positions, rotations or attention.  The layout rules named here ("attached",
"rule") are interpreted independently by the library's layout builder and by
the oracle.

Item vocabulary (one dict per item, items listed in reference order):

* ``{"kind": "visual", "T": T, "H": H, "W": W}`` -- a latent video grid
  (an image reference is a grid with T = 1).
* ``{"kind": "audio", "n": n, "span": s, "attached": bool, "rule": r}`` --
  a run of ``n`` audio latent rows covering ``s`` latent frames of the shared
  clock.  ``attached`` audio rides the clock span of the visual item just
  before it (a video's own soundtrack); a standalone audio reference starts at
  the current clock and advances it by ``s``.  ``rule`` is ``"linear"``
  (offset i*s/n) or ``"round"`` (that offset rounded half-to-even).
* ``{"kind": "clock", "span": s}`` -- no rows; moves the clock forward by
  ``s`` (a long video's continuation chunk at its global time).
* ``{"kind": "text", "n": n}`` -- ``n`` rows at position (0, 0, 0), e.g.
  one prompt for the token refiner.

The workloads follow the sequence structure the pages describe: the DiT packs
the video latent and the audio latent into one long token sequence
("Day 0 Support for MiniMax-H3 on AMD Instinct GPUs", section "The diffusion
transformer (DiT)"); references sit in front of the generated rows, in
reference order, on one shared audio/video rotary clock ("minimax-h3-reference"
Space README, sections "References" and "AoTI-compiled blocks"); co-batched
requests are packed with one attention document each (vLLM-Omni "MiniMax-H3"
recipe, section "Step execution and continuous batching").

Random inputs: ``numpy.random.Generator(PCG64(seed))``, then
``standard_normal((N, H, D), float32)`` drawn for q, k, v in that order,
optionally multiplied by a per-tensor factor, then rounded to bfloat16 by
round-to-nearest-even on the float32 bit pattern.  The result is returned as
uint16 bit patterns so that neither side needs a bfloat16 dtype to agree on
the exact input values.

Local-attention inputs (``local_qkv``), for the Skip-Softmax mode: with the
same generator, first one direction per head, ``c_h = g / |g|`` for
``g = standard_normal((H, D), float64)``; then q and k as
``amp * c_h + standard_normal((N, H, D), float32)`` and v as
``standard_normal((N, H, D), float32)``, each rounded to bfloat16 as above.
When q and k share a direction, the rotary score of a pair depends mostly on
the difference of their positions and peaks where it is zero, so attention
is local in (t, h, w).  This stands in for the locality of a trained DiT's
attention maps, which random weights do not have.
"""

from __future__ import annotations

import numpy as np

HEAD_DIM = 128
ROPE_THETA = 10000.0
ROPE_DIMS = (32, 48, 48)  # (t, h, w) widths inside the 128-wide head


def visual(T: int, H: int, W: int) -> dict:
    return {"kind": "visual", "T": int(T), "H": int(H), "W": int(W)}


def audio(n: int, span: float, attached: bool, rule: str = "linear") -> dict:
    assert rule in ("linear", "round")
    return {"kind": "audio", "n": int(n), "span": float(span), "attached": bool(attached), "rule": rule}


def clock(span: float) -> dict:
    return {"kind": "clock", "span": float(span)}


def text(n: int) -> dict:
    return {"kind": "text", "n": int(n)}


def native_frames(seconds: float, fps: int = 24) -> int:
    """Frames of the native 17n+5 video-frame grid that cover ``seconds`` (the smallest n that does)."""
    need = seconds * fps
    n = max(0, -(-int(round(need - 5)) // 17))
    return 17 * n + 5


def latent_frames(frames: int) -> int:
    """Latent frames of a 17n+5-frame video on the 5n+2 latent grid."""
    assert (frames - 5) % 17 == 0
    return 5 * ((frames - 5) // 17) + 2


# Long video by latent continuation: the last chunk of a 300-second request (the continuation
# limit), one image reference in front; the chunk keeps its global temporal positions.
LONG_SECONDS = 300
LONG_CHUNK = 17


def _long_segment():
    total = latent_frames(native_frames(LONG_SECONDS))
    return [[visual(1, 24, 42), clock(total - LONG_CHUNK), visual(LONG_CHUNK, 24, 42),
             audio(32 * LONG_CHUNK, LONG_CHUNK, attached=True)]]


# Token refiner: eight co-batched prompts, each its own document.
REFINER_PROMPTS = (77, 128, 203, 256, 300, 421, 512, 645)


def _packed_segments():
    return [[visual(T, 24, 42), audio(32 * T, T, attached=True)] for T in (5, 9, 13, 17)]


def _ref2va_segment():
    seg = [visual(1, 24, 42) for _ in range(9)]          # 9 image references
    seg += [visual(8, 24, 42), audio(256, 8, attached=True)]  # reference video + its soundtrack
    seg += [audio(256, 8, attached=False)]               # standalone reference audio
    seg += [visual(17, 24, 42), audio(544, 17, attached=True)]  # generated target
    return [seg]


# The five workloads.  "heads" is the head count one GPU computes.
CONFIGS = {
    "tiny": {
        "heads": 4,
        "segments": [[visual(3, 8, 8), audio(24, 3, attached=True, rule="round")]],
        "seed": 1,
    },
    "480p": {
        "heads": 24,
        "segments": [[visual(8, 24, 40), audio(256, 8, attached=True)]],
        "seed": 2,
    },
    "packed": {
        "heads": 16,
        "segments": _packed_segments(),
        "seed": 3,
    },
    "1344x768": {
        "heads": 5,
        "segments": [[visual(32, 48, 84), audio(1024, 32, attached=True)]],
        "seed": 4,
    },
    "ref2va": {
        "heads": 24,
        "segments": _ref2va_segment(),
        "seed": 5,
    },
    "long300": {
        "heads": 24,
        "segments": _long_segment(),
        "seed": 6,
    },
    "refiner": {
        "heads": 56,
        "segments": [[text(n)] for n in REFINER_PROMPTS],
        "seed": 7,
    },
}

CONFIG_ORDER = ["tiny", "480p", "packed", "1344x768", "ref2va", "long300", "refiner"]

# Seed offset for the second (robustness) seed of each workload.
ROBUSTNESS_SEED_OFFSET = 1000


def item_rows(item: dict) -> int:
    if item["kind"] == "visual":
        return item["T"] * item["H"] * item["W"]
    if item["kind"] == "clock":
        return 0
    return item["n"]


def n_tokens(segments) -> int:
    return sum(item_rows(it) for seg in segments for it in seg)


def segment_lengths(segments):
    return [sum(item_rows(it) for it in seg) for seg in segments]


def _round_bf16_bits(x32: np.ndarray) -> np.ndarray:
    """float32 array -> uint16 bfloat16 bit patterns, round to nearest even."""
    u = np.ascontiguousarray(x32, dtype=np.float32).view(np.uint32)
    bias = np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns to float32."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def random_qkv(n: int, heads: int, seed: int, head_dim: int = HEAD_DIM, scale=(1.0, 1.0, 1.0)):
    """Seeded bf16 q, k, v as uint16 bit patterns of shape [n, heads, head_dim]."""
    rng = np.random.Generator(np.random.PCG64(seed))
    out = []
    for s in scale:
        x = rng.standard_normal((n, heads, head_dim), dtype=np.float32)
        if s != 1.0:
            x = x * np.float32(s)
        out.append(_round_bf16_bits(x))
    return tuple(out)


def local_qkv(n: int, heads: int, seed: int, amp: float, head_dim: int = HEAD_DIM):
    """Seeded bf16 q, k, v (uint16 bit patterns, [n, heads, head_dim]) whose attention is local."""
    rng = np.random.Generator(np.random.PCG64(seed))
    g = rng.standard_normal((heads, head_dim))
    c = (g / np.linalg.norm(g, axis=1, keepdims=True)).astype(np.float32)
    out = []
    for shared in (True, True, False):
        x = rng.standard_normal((n, heads, head_dim), dtype=np.float32)
        if shared:
            x = x + np.float32(amp) * c[None, :, :]
        out.append(_round_bf16_bits(x))
    return tuple(out)


def config(name: str) -> dict:
    return CONFIGS[name]
