"""MI355X-native joint audio/video attention (h3attn): multi-axis RoPE on a
shared audio/video clock, then packed variable-length flash-attention forward.

The compute lives in the HIP library ``libh3attn.so`` (built from ``csrc/``);
this package only marshals arguments to its C ABI.
"""

from . import workloads  # noqa: F401  (seeded synthetic inputs; no method arithmetic)

__all__ = ["workloads"]
