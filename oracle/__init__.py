"""Plain float64 CPU oracle for joint audio/video attention.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute anything in this package.  Only the tests, the smoke check of the
package entry point and the ``cpu_baseline`` leg of ``bench.py`` use it.  It
shares no code with the HIP library: it re-derives positions, rotations and
attention from the pages' description, in float64, with no blocking, fusion or
reordering beyond bounding memory by splitting query rows.

What it computes (sources are the pages the method is described on):

* ``layout``  -- per-token (t, h, w) positions on one shared audio/video clock
  and the packed-sequence prefix sums.  The sequence is the video latent
  followed by the audio latent, flattened into one token sequence ("Day 0
  Support for MiniMax-H3 on AMD Instinct GPUs", "The diffusion transformer
  (DiT)"); references are packed in front of the generated rows and each one
  advances the shared rotary clock in reference order ("minimax-h3-reference"
  README, "References" and "AoTI-compiled blocks"); each co-batched request
  is its own attention document (vLLM-Omni "MiniMax-H3" recipe, "Step
  execution and continuous batching"); position metadata is built in float64
  and cast to float32 for device arithmetic ("MiniMax H3 on Moore Threads
  MUSA", "MUSA validation").
* ``rope``    -- multi-axis rotary position embedding (the DiT's position
  encoding is rotary: "Day 0 Support ...", DiT property table).
* ``attention`` -- exact softmax(Q~ K~^T / sqrt(d)) V per segment and head,
  plus the natural-log log-sum-exp of each row.
* ``sage``    -- the lossy FP8 mode of the same attention: Q and K in e4m3
  with one scale per query row and per 16 keys, P and V in e4m3 (vLLM-Omni
  "MiniMax-H3" recipe, "Attention Backends", SAGE quantization), with the
  Skip-Softmax rule.
* ``gate``    -- the Skip-Softmax timestep gate and the noise schedule of the
  denoising steps it is compared with (same recipe section).

Every function is pinned by tests under ``tests/`` against closed forms,
invariants, brute force and library routines (see ``tests/test_oracle_*.py``).
The pages fix no numeric attention output, so agreement with the pages
themselves rests on those pins and on the readings stated in each module.
"""

from .layout import layout, round_half_even
from .rope import rope, rope_frequencies
from .attention import attention, attention_rows
from .sage import round_e4m3, sage_attention, sage_attention_rows
from .gate import flow_shift, forward_sigmas, skip_threshold_at

__all__ = [
    "layout",
    "round_half_even",
    "rope",
    "rope_frequencies",
    "attention",
    "attention_rows",
    "round_e4m3",
    "sage_attention",
    "sage_attention_rows",
]
