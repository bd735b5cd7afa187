"""Scalar-loop float64 twin of the oracle (tiny inputs only).

TEST INFRASTRUCTURE ONLY. Pure Python loops and ``math.fsum``; no numpy
arithmetic, so it shares no vectorised code with ``attn64``. It states the same
definition (optional QK-norm, 3D rotary encoding of queries and rotary keys, then softmax
attention over all keys with no mask -- MiniMax-H3 deep-dive page, attention
paragraph after the DiT configuration table; StreamRender-H3 page,
streaming-context section) one number at a time.
"""

import math


def pair_angle(p_thw, pair, axis_dims, theta):
    """Angle of rotary pair ``pair`` (dims 2*pair, 2*pair+1) at position p."""
    start = 0
    for a, width in enumerate(axis_dims):
        npairs = int(width) // 2
        if pair < start + npairs:
            i = pair - start
            return float(p_thw[a]) * float(theta) ** (-2.0 * i / int(width))
        start += npairs
    raise IndexError("pair index beyond the head dimension")


def rotate_vec(x, p_thw, axis_dims, theta):
    """Rotate one head vector ``x`` (list of floats) at position ``p_thw``."""
    out = [0.0] * len(x)
    for pair in range(len(x) // 2):
        phi = pair_angle(p_thw, pair, axis_dims, theta)
        c, s = math.cos(phi), math.sin(phi)
        a, b = float(x[2 * pair]), float(x[2 * pair + 1])
        out[2 * pair] = a * c - b * s
        out[2 * pair + 1] = a * s + b * c
    return out


def rms_vec(x, h, norm):
    """RMS-normalise one head vector ``x`` of head ``h`` (QK-norm before the
    rotation): divide by sqrt(mean of squares + eps), multiply by the weight
    (``norm`` = ``(weight, eps)``; weight ``None``, ``[d]`` or ``[H][d]``)."""
    weight, eps = norm
    d = len(x)
    r = math.sqrt(math.fsum(float(t) * float(t) for t in x) / d + float(eps))
    if weight is None:
        w = [1.0] * d
    elif hasattr(weight[0], "__len__"):
        w = [float(t) for t in weight[h]]
    else:
        w = [float(t) for t in weight]
    return [float(x[c]) / r * w[c] for c in range(d)]


def chunk_attention(q, q_pos, segments, axis_dims, theta, scale, q_norm=None, k_norm=None):
    """Same contract as ``attn64.chunk_attention`` (no row selection).

    ``q``: nested ``[Nq][H][d]``; ``q_pos``: ``[Nq][3]`` or ``None``;
    ``segments``: ``(k, v, pos_or_None)``; ``q_norm`` / ``k_norm``:
    ``(weight, eps)`` or ``None``. Returns nested lists of floats.
    """
    keys, vals = [], []
    for k, v, pos in segments:
        for j in range(len(k)):
            heads_k = []
            for h in range(len(k[j])):
                kv = [float(t) for t in k[j][h]]
                if k_norm is not None:
                    kv = rms_vec(kv, h, k_norm)
                if pos is not None:
                    kv = rotate_vec(kv, pos[j], axis_dims, theta)
                heads_k.append(kv)
            keys.append(heads_k)
            vals.append([[float(t) for t in v[j][h]] for h in range(len(v[j]))])
    out = []
    for n in range(len(q)):
        row = []
        for h in range(len(q[n])):
            qv = [float(t) for t in q[n][h]]
            if q_norm is not None:
                qv = rms_vec(qv, h, q_norm)
            if q_pos is not None:
                qv = rotate_vec(qv, q_pos[n], axis_dims, theta)
            s = [scale * math.fsum(a * b for a, b in zip(qv, keys[j][h])) for j in range(len(keys))]
            m = max(s)
            e = [math.exp(x - m) for x in s]
            z = math.fsum(e)
            d = len(qv)
            row.append([math.fsum(e[j] * vals[j][h][c] for j in range(len(keys))) / z for c in range(d)])
        out.append(row)
    return out
