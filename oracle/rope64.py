"""3D rotary position encoding in float64 (oracle; test infrastructure only).

The MiniMax-H3 DiT applies a 3D "MM-RoPE" over (time, height, width) to queries
and keys (MiniMax-H3 deep-dive page, components table, H3-Omni-Transformer row,
and the attention paragraph after the DiT configuration table). The pages give
neither the split of the head dimension over the three axes nor the frequency
schedule nor the pair layout, so this module fixes the plainest reading:

* the head dimension ``d`` is cut into three consecutive bands of even widths
  ``(D_t, D_h, D_w)`` with ``D_t + D_h + D_w = d``; band ``a`` starts at
  ``o_a`` (``o_t = 0``, ``o_h = D_t``, ``o_w = D_t + D_h``);
* inside band ``a`` the rotary pairs are adjacent dimensions
  ``(o_a + 2i, o_a + 2i + 1)``, ``0 <= i < D_a / 2``;
* pair ``i`` of band ``a`` turns by ``phi = p_a * theta ** (-2 i / D_a)``
  where ``p_a`` is the token's coordinate on that axis;
* the turn is counter-clockwise:
  ``(x, y) -> (x cos phi - y sin phi, x sin phi + y cos phi)``.

Angles are computed here from the positions with libm-quality float64
``cos``/``sin``; nothing computed by the GPU library is consumed.
"""

import numpy as np


def check_axis_dims(axis_dims, head_dim):
    """Validate a (D_t, D_h, D_w) band split of ``head_dim``."""
    if len(axis_dims) != 3:
        raise ValueError("axis_dims must have three entries (t, h, w)")
    if any(int(a) < 0 or int(a) % 2 for a in axis_dims):
        raise ValueError("each axis band width must be even and >= 0")
    if sum(int(a) for a in axis_dims) != head_dim:
        raise ValueError("axis band widths must sum to the head dimension")


def pair_axis_and_freq(axis_dims, theta):
    """Per rotary pair: which axis it follows and its angular frequency.

    Returns ``(axis, freq)``, two arrays of length ``d / 2``; pair ``p`` covers
    dimensions ``(2p, 2p + 1)``. ``freq = theta ** (-2 i / D_a)`` for the
    ``i``-th pair of band ``a``.
    """
    axis = []
    freq = []
    for a, width in enumerate(axis_dims):
        width = int(width)
        for i in range(width // 2):
            axis.append(a)
            freq.append(float(theta) ** (-2.0 * i / width))
    return np.asarray(axis, dtype=np.int64), np.asarray(freq, dtype=np.float64)


def angles(pos, axis_dims, theta):
    """Rotation angle of every rotary pair of every token.

    ``pos``: ``[n][3]`` (t, h, w) coordinates (any float dtype; upcast to
    float64 exactly). Returns ``phi``: float64 ``[n][d / 2]``.
    """
    pos = np.asarray(pos, dtype=np.float64).reshape(-1, 3)
    axis, freq = pair_axis_and_freq(axis_dims, theta)
    return pos[:, axis] * freq[None, :]


def rotate(x, phi):
    """Rotate adjacent pairs of the last dimension of ``x`` by ``phi``.

    ``x``: ``[n][H][d]`` (or ``[n][d]``); ``phi``: ``[n][d / 2]``. The same
    angles apply to every head. Returns float64 of the shape of ``x``.
    """
    x = np.asarray(x, dtype=np.float64)
    squeeze = x.ndim == 2
    if squeeze:
        x = x[:, None, :]
    n, _, d = x.shape
    phi = np.asarray(phi, dtype=np.float64).reshape(n, d // 2)
    c = np.cos(phi)[:, None, :]
    s = np.sin(phi)[:, None, :]
    xe = x[..., 0::2]
    xo = x[..., 1::2]
    out = np.empty_like(x)
    out[..., 0::2] = xe * c - xo * s
    out[..., 1::2] = xe * s + xo * c
    return out[:, 0, :] if squeeze else out
