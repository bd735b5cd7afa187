"""Per-head RMS normalisation (QK-norm) in float64 (oracle; test infrastructure only).

The MiniMax-H3 DiT normalises queries and keys before its 3D rotary encoding
(MiniMax-H3 deep-dive page, attention paragraph after the DiT configuration
table). The pages name QK-norm but not its form; this module fixes the plain
RMSNorm reading: over the ``d`` elements of one head of one row,

    x_c -> x_c / sqrt(mean_c(x_c ** 2) + eps) * w_c,

with a learned weight ``w`` shared by all heads (``[d]``) or per head
(``[H][d]``), and the normalisation applied before the rotation.
"""

import numpy as np


def rmsnorm(x, weight, eps):
    """RMS-normalise the last axis of ``x`` (``[..., H, d]``), then scale by ``weight``.

    ``weight``: ``None`` (all ones), ``[d]`` or ``[H][d]``; ``eps >= 0``.
    """
    x = np.asarray(x, dtype=np.float64)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    y = x / np.sqrt(ms + float(eps))
    if weight is not None:
        y = y * np.asarray(weight, dtype=np.float64)
    return y
