"""Spatial pooling of aged history into a coarser tier, float64 (oracle).

TEST INFRASTRUCTURE ONLY (see the package docstring for who may call it).

AlayaRenderer-Flash page, key contributions and technical details: history
that has aged out of the most recent chunk is kept at progressively lower
resolution (three tiers by temporal distance) and still inserted into the
attention context. The pages give neither the pooling operator nor where in
the block it applies; the plain reading taken here:

* a tier is an s x s spatial mean (s = 2 or 4) over each latent frame's token
  grid; the frame (time) axis is not pooled;
* it is taken of the keys as they enter attention before their QK-norm and
  rotation (a mean of keys is the key of the mean of the tokens, the key
  projection being linear), and of the values;
* the pooled key is then normalised and rotated like any other key, at the
  pooled cell's position: the centre of the full-resolution cells it covers.

Rows are ordered frame-major, then grid row, then grid column, for the
full-resolution input and for the pooled output alike.
"""

import numpy as np


def pool_frames(x, grid_h, grid_w, s):
    """Mean of every s x s block of each latent frame.

    ``x``: ``[F * grid_h * grid_w][H][d]``; ``grid_h`` and ``grid_w`` are
    multiples of ``s``. Returns float64 ``[F * (grid_h/s) * (grid_w/s)][H][d]``
    whose row (f, i, j) is the mean of input rows (f, s*i + a, s*j + b) over
    a, b in [0, s).
    """
    x = np.asarray(x, dtype=np.float64)
    if s < 1 or grid_h % s or grid_w % s:
        raise ValueError("grid sides must be multiples of the pooling factor")
    per_frame = grid_h * grid_w
    if x.shape[0] % per_frame:
        raise ValueError("row count is not a whole number of frames")
    frames = x.shape[0] // per_frame
    rest = x.shape[1:]
    blocks = x.reshape((frames, grid_h // s, s, grid_w // s, s) + rest)
    return blocks.mean(axis=(2, 4)).reshape((frames * (grid_h // s) * (grid_w // s),) + rest)
