"""Dense softmax attention of one streaming chunk, float64 (oracle).

TEST INFRASTRUCTURE ONLY (see the package docstring for who may call it).

The operation (plain definition; flash-style online softmax is an exact
reformulation of it, so this is what a fast kernel must reproduce up to
rounding):

1. Optionally RMS-normalise queries and keys per head (QK-norm, see
   ``norm64``), then rotate the queries by their own 3D positions and every
   key of a rotary segment by that key's positions; keys of a non-rotary
   segment (the persistent style-prompt key/values) are not rotated.
   (MiniMax-H3 deep-dive page: dense softmax attention with 3D MM-RoPE.
   AlayaRenderer-Flash page, key contributions / method: prompt-derived
   persistent key/values are added to every self-attention layer.)
2. Concatenate the segments, in order, into one key/value set: style prompt,
   session reference frame, clean history (coarser tiers for older history),
   current noisy chunk. (AlayaRenderer-Flash page, key contributions and
   technical details; StreamRender-H3 page, streaming-context section: the
   prefix cache holds conditions, reference and sink.)
3. For every head and query: scores against *all* keys with no mask (the
   window is bidirectional and its moving part attends to the whole window:
   StreamRender-H3 page, streaming-context section), scaled by ``scale``;
   softmax over keys; weighted sum of the values.

``split_attention`` states the same attention restricted to runs of keys:
each run's own softmax attention and the natural log of the sum of
``exp(scores)`` over the run (what a split-key evaluation must produce
before its runs are merged).
"""

import numpy as np

from . import norm64, rope64


def softmax_rows(s):
    """Row softmax of a float64 score block ``s`` ``[rows][keys]``."""
    s = np.asarray(s, dtype=np.float64)
    m = np.max(s, axis=-1, keepdims=True)
    e = np.exp(s - m)
    return e / np.sum(e, axis=-1, keepdims=True)


def attention(q, k, v, scale, block=512):
    """Plain scaled-dot-product attention, float64, no mask.

    ``q``: ``[Nq][H][d]``; ``k``, ``v``: ``[Nk][H][d]``. Returns ``[Nq][H][d]``.
    Queries are processed in blocks of ``block`` rows per head only to bound
    memory; rows are independent, so blocking does not change any value.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    nq, heads, d = q.shape
    out = np.empty((nq, heads, d), dtype=np.float64)
    for h in range(heads):
        kh = np.ascontiguousarray(k[:, h, :])
        vh = np.ascontiguousarray(v[:, h, :])
        for r0 in range(0, nq, block):
            qh = q[r0:r0 + block, h, :]
            p = softmax_rows(scale * (qh @ kh.T))
            out[r0:r0 + block, h, :] = p @ vh
    return out


def prepare(x, pos, norm, axis_dims, theta):
    """One query or key block ``[n][H][d]`` as attention sees it: QK-norm
    (``norm`` = ``(weight, eps)`` or ``None``) first, then the rotation by
    ``pos`` (``[n][3]`` or ``None`` for no rotation)."""
    x = np.asarray(x, dtype=np.float64)
    if x.shape[0] == 0:
        return x
    if norm is not None:
        x = norm64.rmsnorm(x, norm[0], norm[1])
    if pos is not None:
        x = rope64.rotate(x, rope64.angles(pos, axis_dims, theta))
    return x


def rotated_keys(segments, axis_dims, theta, k_norm=None):
    """Concatenate segments into (K', V) with each key normalised (when
    ``k_norm`` is given) and each rotary key rotated.

    ``segments``: sequence of ``(k, v, pos)``; ``k``, ``v`` are ``[n][H][d]``
    and ``pos`` is ``[n][3]`` or ``None`` for a non-rotary segment.
    """
    ks, vs = [], []
    for k, v, pos in segments:
        ks.append(prepare(k, pos, k_norm, axis_dims, theta))
        vs.append(np.asarray(v, dtype=np.float64))
    return np.concatenate(ks, axis=0), np.concatenate(vs, axis=0)


def chunk_attention(q, q_pos, segments, axis_dims, theta, scale, rows=None, block=512, q_norm=None,
                    k_norm=None):
    """Attention of the chunk's queries over the segmented context.

    ``q``: ``[Nq][H][d]``; ``q_pos``: ``[Nq][3]`` or ``None`` (no rotary);
    ``segments`` as in :func:`rotated_keys`. ``rows`` optionally selects query
    rows (rows are independent, so this is exact for the selected rows).
    ``q_norm`` / ``k_norm``: ``(weight, eps)`` QK-norm of queries / of every
    key, or ``None``. Returns float64 ``[len(rows) or Nq][H][d]``.
    """
    q = np.asarray(q, dtype=np.float64)
    head_dim = q.shape[-1]
    rope64.check_axis_dims(axis_dims, head_dim)
    if rows is not None:
        rows = np.asarray(rows, dtype=np.int64)
        q = q[rows]
        if q_pos is not None:
            q_pos = np.asarray(q_pos)[rows]
    q = prepare(q, q_pos, q_norm, axis_dims, theta)
    k, v = rotated_keys(segments, axis_dims, theta, k_norm=k_norm)
    if k.shape[0] == 0:
        raise ValueError("the key/value context is empty")
    return attention(q, k, v, scale, block=block)


def split_attention(q, k, v, scale, key_ranges):
    """Per key run ``[a, b)``: softmax attention over the run's keys alone and
    ``log sum_j exp(scale * <q, k_j>)`` over the run (natural log).

    ``q``: ``[Nq][H][d]``; ``k``, ``v``: ``[Nk][H][d]``. Returns
    ``(partial [runs][Nq][H][d], lse [runs][Nq][H])``, float64.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    nq, heads, d = q.shape
    partial = np.empty((len(key_ranges), nq, heads, d))
    lse = np.empty((len(key_ranges), nq, heads))
    for r, (a, b) in enumerate(key_ranges):
        for h in range(heads):
            s = scale * (q[:, h, :] @ k[a:b, h, :].T)
            m = np.max(s, axis=-1, keepdims=True)
            e = np.exp(s - m)
            z = np.sum(e, axis=-1, keepdims=True)
            partial[r, :, h, :] = (e / z) @ v[a:b, h, :]
            lse[r, :, h] = (m + np.log(z))[:, 0]
    return partial, lse


def chunk_split_attention(q, q_pos, segments, axis_dims, theta, scale, key_ranges, rows=None, q_norm=None,
                          k_norm=None):
    """:func:`split_attention` of the chunk's (prepared) queries over the
    concatenated (prepared) context, key runs given in packed-row order."""
    q = np.asarray(q, dtype=np.float64)
    rope64.check_axis_dims(axis_dims, q.shape[-1])
    if rows is not None:
        rows = np.asarray(rows, dtype=np.int64)
        q = q[rows]
        if q_pos is not None:
            q_pos = np.asarray(q_pos)[rows]
    q = prepare(q, q_pos, q_norm, axis_dims, theta)
    k, v = rotated_keys(segments, axis_dims, theta, k_norm=k_norm)
    return split_attention(q, k, v, scale, key_ranges)
