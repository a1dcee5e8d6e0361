"""Oracle: multi-axis rotary position embedding in float64.

Test infrastructure only; see the package docstring.

The DiT's position encoding is rotary ("Day 0 Support for MiniMax-H3 on AMD
Instinct GPUs", DiT property table).  The pages do not spell out the
multi-axis form; the reading used here:

* the 128-wide head is split into consecutive axis chunks, t then h then w,
  of widths (32, 48, 48);
* inside a chunk of width d_a, dims (2j, 2j+1) form the j-th rotation pair,
  j < d_a / 2, with angular frequency theta ** (-2 j / d_a), theta = 10000;
* the pair (x0, x1) at position p on that axis turns by phi = p * omega:
  (x0 cos phi - x1 sin phi, x0 sin phi + x1 cos phi).

Audio tokens carry (t, 0, 0), so their h and w chunks turn by zero.
"""

from __future__ import annotations

import numpy as np


def rope_frequencies(theta: float, width: int) -> np.ndarray:
    """omega_j = theta ** (-2 j / width) for j = 0 .. width/2 - 1, float64."""
    if width % 2:
        raise ValueError("axis width must be even")
    j = np.arange(width // 2, dtype=np.float64)
    return np.power(np.float64(theta), -2.0 * j / width)


def rope(x: np.ndarray, pos: np.ndarray, theta: float = 10000.0, dims=(32, 48, 48)) -> np.ndarray:
    """Rotate x [N, H, D] (float64) by positions pos [N, 3] (t, h, w)."""
    x = np.asarray(x, dtype=np.float64)
    pos = np.asarray(pos, dtype=np.float64)
    N, H, D = x.shape
    if sum(dims) != D:
        raise ValueError("axis widths must add up to the head dim")
    if pos.shape != (N, len(dims)):
        raise ValueError("pos must be [N, n_axes]")
    out = x.copy()
    offset = 0
    for axis, width in enumerate(dims):
        omega = rope_frequencies(theta, width)              # [width/2]
        phi = pos[:, axis][:, None] * omega[None, :]        # [N, width/2]
        c = np.cos(phi)[:, None, :]                         # [N, 1, width/2]
        s = np.sin(phi)[:, None, :]
        x0 = x[:, :, offset + 0:offset + width:2]           # first of each pair
        x1 = x[:, :, offset + 1:offset + width:2]           # second of each pair
        out[:, :, offset + 0:offset + width:2] = x0 * c - x1 * s
        out[:, :, offset + 1:offset + width:2] = x0 * s + x1 * c
        offset += width
    return out
