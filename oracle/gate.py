"""Skip-Softmax timestep gate and the denoising noise schedule it is read against.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Source: vLLM-Omni "MiniMax-H3" recipe, section "Attention Backends".  The
Skip-Softmax setting there carries a cutoff, ``disabled_until_timestep``, that
keeps the early, high-noise steps dense; the cutoff is compared with the
video sigma of the step; H3's default flow shift is 12; and with 50 steps the
cutoffs 0.99, 0.97 and 0.95 keep the first 6, 14 and 19 of 49 denoiser
forwards dense.

Readings (the page names the quantities but not their formulas):

* The schedule is the flow-matching time shift applied to evenly spaced
  noise levels: sigma' = s * sigma / (1 + (s - 1) * sigma) for shift s.
* 50 steps are 50 evenly spaced levels from 1 down to 0; the last one is
  clean and runs no forward, which leaves the 49 forwards the page counts,
  at sigma_i = 1 - i / 49 for i = 0..48.
* A step runs dense while its sigma is above the cutoff.

These three readings together give exactly the page's counts (6, 14, 19);
the other natural readings do not (a 50-point grid of forwards gives 20 for
the cutoff 0.95), so the worked example pins them.
"""

from __future__ import annotations

import numpy as np


def flow_shift(sigma, shift: float):
    """Flow-matching time shift of noise levels in [0, 1]."""
    sigma = np.asarray(sigma, dtype=np.float64)
    return shift * sigma / (1.0 + (shift - 1.0) * sigma)


def forward_sigmas(steps: int, shift: float) -> np.ndarray:
    """Noise levels of the denoiser forwards of a ``steps``-step run (steps - 1 of them)."""
    levels = np.linspace(1.0, 0.0, steps)
    return flow_shift(levels[:-1], shift)


def skip_threshold_at(threshold: float, disabled_until_timestep: float, sigma: float) -> float:
    """The Skip-Softmax threshold in force at noise level sigma: 0 (every tile kept) above the cutoff."""
    return 0.0 if sigma > disabled_until_timestep else float(threshold)
