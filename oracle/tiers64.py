"""Ageing of the hierarchical history from chunk to chunk, float64 (oracle).

TEST INFRASTRUCTURE ONLY (see the package docstring for who may call it).

AlayaRenderer-Flash page, key contributions and technical details: the
renderer generates its video chunk by chunk and keeps the history in three
tiers by temporal distance, the most recent at full resolution and older
history at progressively lower resolution, all of it in the attention context
of the chunk being generated. The pages fix neither the tier boundaries nor
the pooling; the plain reading taken here (and by the pack's pooled segments):

* every chunk spans the same F latent frames;
* while chunk c is generated the history holds chunk c-1 at full
  resolution, chunk c-2 as its 2x2 spatial means and chunk c-3 as its 4x4
  spatial means; chunks older than c-3 have left the context; a tier whose
  chunk does not exist yet (c < 3) is empty;
* a tier is pooled from its chunk's own full-resolution keys and values (keys
  before their normalisation and rotation, see ``pool64``), so each chunk
  ages 1x1 -> 2x2 -> 4x4 -> gone over four steps;
* the positions form one fixed template whatever the chunk: reference frame
  at t = 0, then the 4x4 tier, the 2x2 tier and the full-resolution chunk,
  F frames each, oldest first, then the current chunk (t = 1 .. 4F); a pooled
  token sits at the centre of the cells it covers (``pool64``).

Only the arithmetic of ``pool64`` and ``attn64`` is used: this module states
which chunk feeds which tier.
"""

import numpy as np

from . import attn64, pool64

# (tier name, pooling factor, age in chunks), oldest tier first: the order of
# the segments in the context
TIERS = (("pool4", 4, 3), ("pool2", 2, 2), ("prev", 1, 1))


def tier_chunks(c):
    """``[(name, s, chunk index or None)]`` of the history while chunk ``c`` is
    generated (None: the tier is still empty)."""
    return [(name, s, c - age if c - age >= 0 else None) for name, s, age in TIERS]


def cell_positions(t_values, grid_h, grid_w, s):
    """(t, h, w) of every token of frames ``t_values`` after s x s pooling,
    each at the centre of the full-resolution cells it covers."""
    gh, gw = grid_h // s, grid_w // s
    hh, ww = np.meshgrid(np.arange(gh) * s + (s - 1) / 2.0, np.arange(gw) * s + (s - 1) / 2.0, indexing="ij")
    out = []
    for t in t_values:
        out.append(np.stack([np.full(gh * gw, float(t)), hh.reshape(-1), ww.reshape(-1)], axis=1))
    return np.concatenate(out, axis=0)


def template_t(frames):
    """Frame indices of the template: ``{tier or "current": [t ...]}``."""
    out = {}
    for i, (name, _, _) in enumerate(TIERS):
        out[name] = list(range(1 + i * frames, 1 + (i + 1) * frames))
    out["current"] = list(range(1 + len(TIERS) * frames, 1 + (len(TIERS) + 1) * frames))
    return out


def history_segments(chunk_kv, c, frames, grid_h, grid_w, positions=None):
    """History segments ``[(k, v, pos)]`` of chunk ``c``, oldest tier first.

    ``chunk_kv(j)`` returns chunk j's full-resolution ``(k, v)``, each
    ``[frames * grid_h * grid_w][H][d]``. ``positions(name, s)`` may override
    a tier's positions (default: the template, float64); an empty tier is
    left out (it holds no rows)."""
    tt = template_t(frames)
    segs = []
    for name, s, j in tier_chunks(c):
        if j is None:
            continue
        k, v = chunk_kv(j)
        pos = positions(name, s) if positions else cell_positions(tt[name], grid_h, grid_w, s)
        if s > 1:
            k, v = pool64.pool_frames(k, grid_h, grid_w, s), pool64.pool_frames(v, grid_h, grid_w, s)
        segs.append((np.asarray(k, dtype=np.float64), np.asarray(v, dtype=np.float64), pos))
    return segs


def chunk_attention(q, q_pos, static_segments, chunk_kv, c, frames, grid_h, grid_w, axis_dims, theta, scale,
                    rows=None, positions=None, q_norm=None, k_norm=None):
    """Attention of chunk ``c``'s queries over static segments (prompt,
    reference), the aged history tiers and the current chunk."""
    segs = list(static_segments) + history_segments(chunk_kv, c, frames, grid_h, grid_w, positions)
    k, v = chunk_kv(c)
    tt = template_t(frames)
    cur_pos = positions("current", 1) if positions else cell_positions(tt["current"], grid_h, grid_w, 1)
    segs.append((k, v, cur_pos))
    return attn64.chunk_attention(q, q_pos, segs, axis_dims, theta, scale, rows=rows, q_norm=q_norm, k_norm=k_norm)
