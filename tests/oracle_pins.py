"""Pins that tie the fp64 oracle to something other than itself.

Each ``pin_*`` function raises ``AssertionError`` when the oracle (the modules
``oracle.rope64``, ``oracle.attn64``) disagrees with a closed form, an
invariant of the mathematics, a library routine or the independent scalar
twin ``oracle.brute``. ``test_oracle_pins.py`` runs them on the real oracle;
``test_oracle_mutations.py`` plants plausible mistakes in the oracle (on the
CPU) and checks that some pin fails for each.

The definition pinned: optional per-head RMS normalisation (QK-norm) before
the rotation; 3D rotary encoding over (t, h, w) bands of the head dimension,
adjacent rotary pairs, angle ``p_a * theta**(-2i/D_a)``, counter-clockwise
turn; dense softmax attention over every key with no mask
(MiniMax-H3 deep-dive page, attention paragraph after the DiT configuration
table; StreamRender-H3 page, streaming-context section).
"""

import math

import numpy as np
import torch

from oracle import attn64, brute, norm64, pool64, rope64, tiers64

AX128 = (32, 48, 48)
THETA = 10000.0


def _rng(tag):
    return np.random.default_rng(np.random.SeedSequence([20261203, tag]))


def _close(a, b, rtol, what):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    err = np.max(np.abs(a - b)) if a.size else 0.0
    ref = max(np.max(np.abs(b)) if b.size else 0.0, 1e-300)
    assert err <= rtol * ref, f"{what}: max abs err {err:.3e} > {rtol:.1e} * {ref:.3e}"


def _tiny_case(tag, d, axis_dims, heads, seg_rows, nq, prompt=0):
    rng = _rng(tag)
    q = rng.standard_normal((nq, heads, d))
    q_pos = rng.random((nq, 3)) * 30.0
    segs = []
    if prompt:
        segs.append((rng.standard_normal((prompt, heads, d)), rng.standard_normal((prompt, heads, d)), None))
    for r in seg_rows:
        segs.append((rng.standard_normal((r, heads, d)), rng.standard_normal((r, heads, d)),
                     rng.random((r, 3)) * 30.0))
    return q, q_pos, segs


def pin_brute_force():
    """Vectorised oracle == scalar-loop twin on tiny inputs, rel <= 1e-12."""
    cases = [
        (1, 2, (2, 0, 0), 1, [3], 2, 0),
        (2, 4, (2, 2, 0), 2, [2, 3], 3, 2),
        (3, 8, (2, 2, 4), 1, [4, 1], 2, 1),
        (4, 64, (16, 24, 24), 2, [5, 4], 3, 3),
        (5, 128, AX128, 1, [3, 2], 2, 2),
    ]
    for tag, d, ax, heads, rows, nq, prompt in cases:
        q, qp, segs = _tiny_case(tag, d, ax, heads, rows, nq, prompt)
        scale = 1.0 / math.sqrt(d)
        got = attn64.chunk_attention(q, qp, segs, ax, THETA, scale)
        ref = brute.chunk_attention(q.tolist(), qp.tolist(),
                                    [(k.tolist(), v.tolist(), None if p is None else p.tolist()) for k, v, p in segs],
                                    ax, THETA, scale)
        _close(got, ref, 1e-12, f"brute force d={d}")


def pin_rotation_closed_form():
    """rotate(e_2p) = cos(phi) e_2p + sin(phi) e_2p+1, phi = p_a theta^(-2i/D_a).

    Checked for every rotary pair of the 32/48/48 split of d = 128; also
    rotate(e_2p+1) = -sin(phi) e_2p + cos(phi) e_2p+1.
    """
    d = 128
    pos = np.array([[3.0, 17.5, 40.25]])
    base = 0
    for a, width in enumerate(AX128):
        for i in range(width // 2):
            p = base // 2 + i
            phi = pos[0, a] * THETA ** (-2.0 * i / width)
            for comp, expect in ((0, {2 * p: math.cos(phi), 2 * p + 1: math.sin(phi)}),
                                 (1, {2 * p: -math.sin(phi), 2 * p + 1: math.cos(phi)})):
                x = np.zeros((1, 1, d))
                x[0, 0, 2 * p + comp] = 1.0
                y = rope64.rotate(x, rope64.angles(pos, AX128, THETA))[0, 0]
                want = np.zeros(d)
                for idx, val in expect.items():
                    want[idx] = val
                _close(y, want, 1e-13, f"rotation closed form band {a} pair {i}")
        base += width


def pin_rotation_group():
    """Rotation is orthogonal, R(0) = I and R(a) R(b) = R(a + b)."""
    rng = _rng(11)
    x = rng.standard_normal((5, 2, 128))
    pa = rng.random((5, 3)) * 50
    pb = rng.random((5, 3)) * 50
    ra = rope64.rotate(x, rope64.angles(pa, AX128, THETA))
    _close(np.linalg.norm(ra, axis=-1), np.linalg.norm(x, axis=-1), 1e-13, "norm preserved")
    _close(rope64.rotate(x, rope64.angles(np.zeros((5, 3)), AX128, THETA)), x, 1e-15, "R(0) = I")
    rab = rope64.rotate(ra, rope64.angles(pb, AX128, THETA))
    _close(rab, rope64.rotate(x, rope64.angles(pa + pb, AX128, THETA)), 1e-11, "R(a)R(b) = R(a+b)")


def pin_single_pair_scores():
    """Score of one-hot q, k in pair i of band a = scale cos((pq_a - pk_a) f_i).

    Read back through the full attention with two keys (k1 one-hot, k2 = 0,
    v1 = e_0, v2 = 0): o_0 = sigmoid(s1), so s1 = logit(o_0).
    """
    d, heads = 128, 1
    scale = 0.7
    pq = np.array([[5.0, 11.0, 2.0]])
    pk = np.array([[2.0, 4.5, 9.0], [0.0, 0.0, 0.0]])
    base = 0
    for a, width in enumerate(AX128):
        for i in (0, 1, width // 4, width // 2 - 1):
            p = base // 2 + i
            q = np.zeros((1, heads, d))
            q[0, 0, 2 * p] = 1.0
            k = np.zeros((2, heads, d))
            k[0, 0, 2 * p] = 1.0
            v = np.zeros((2, heads, d))
            v[0, 0, 0] = 1.0
            o = attn64.chunk_attention(q, pq, [(k, v, pk)], AX128, THETA, scale)[0, 0, 0]
            s1 = math.log(o / (1.0 - o))
            want = scale * math.cos((pq[0, a] - pk[0, a]) * THETA ** (-2.0 * i / width))
            assert abs(s1 - want) <= 1e-10, f"band {a} pair {i}: score {s1} != {want}"
        base += width


def pin_softmax_rows():
    """Softmax rows are non-negative and sum to 1 (|sum - 1| <= 1e-12)."""
    rng = _rng(21)
    s = rng.standard_normal((7, 300)) * 6.0
    p = attn64.softmax_rows(s)
    assert np.all(p >= 0.0)
    _close(p.sum(axis=-1), np.ones(7), 1e-12, "softmax row sums")
    # order-preserving and shift-invariant
    _close(attn64.softmax_rows(s + 3.5), p, 1e-12, "softmax shift invariance")
    assert np.all(np.argsort(p[0]) == np.argsort(s[0]))


def pin_constant_v():
    """All value rows equal c  =>  every output row equals c."""
    q, qp, segs = _tiny_case(31, 128, AX128, 2, [40, 25], 9, prompt=6)
    c = _rng(32).standard_normal((2, 128))
    segs = [(k, np.broadcast_to(c, v.shape).copy(), p) for k, v, p in segs]
    o = attn64.chunk_attention(q, qp, segs, AX128, THETA, 1 / math.sqrt(128))
    _close(o, np.broadcast_to(c, o.shape), 1e-12, "constant V")


def pin_joint_permutation():
    """Permuting key/value rows with their positions leaves the output unchanged.

    Also moves rows between segments (segment boundaries carry no meaning).
    """
    q, qp, segs = _tiny_case(41, 128, AX128, 2, [30, 20], 6, prompt=5)
    scale = 1 / math.sqrt(128)
    o = attn64.chunk_attention(q, qp, segs, AX128, THETA, scale)
    (kp, vp, _), (k1, v1, p1), (k2, v2, p2) = segs
    k = np.concatenate([k1, k2])
    v = np.concatenate([v1, v2])
    p = np.concatenate([p1, p2])
    perm = _rng(42).permutation(k.shape[0])
    cut = 17
    segs2 = [(k[perm[:cut]], v[perm[:cut]], p[perm[:cut]]),
             (kp[::-1], vp[::-1], None),
             (k[perm[cut:]], v[perm[cut:]], p[perm[cut:]])]
    o2 = attn64.chunk_attention(q, qp, segs2, AX128, THETA, scale)
    _close(o2, o, 1e-12, "joint permutation")


def pin_zero_angle_is_sdpa():
    """All positions 0 (and no rotary at all) == torch SDPA in float64 on CPU."""
    rng = _rng(51)
    nq, nk, heads, d = 13, 37, 3, 128
    q = rng.standard_normal((nq, heads, d))
    k = rng.standard_normal((nk, heads, d))
    v = rng.standard_normal((nk, heads, d))
    scale = 0.37
    tq, tk, tv = (torch.from_numpy(x).permute(1, 0, 2).contiguous() for x in (q, k, v))
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, scale=scale)
    ref = ref.permute(1, 0, 2).numpy()
    zero = attn64.chunk_attention(q, np.zeros((nq, 3)), [(k[:20], v[:20], np.zeros((20, 3))),
                                                         (k[20:], v[20:], np.zeros((nk - 20, 3)))],
                                  AX128, THETA, scale)
    _close(zero, ref, 1e-12, "zero angle vs SDPA")
    none = attn64.chunk_attention(q, None, [(k, v, None)], AX128, THETA, scale)
    _close(none, ref, 1e-12, "no rotary vs SDPA")


def pin_two_keys():
    """o = sigmoid(s1 - s2) v1 + sigmoid(s2 - s1) v2 with s = scale <q, k>."""
    rng = _rng(61)
    d = 128
    q = rng.standard_normal((1, 1, d))
    k = rng.standard_normal((2, 1, d))
    v = rng.standard_normal((2, 1, d))
    scale = 0.21
    o = attn64.chunk_attention(q, None, [(k[:1], v[:1], None), (k[1:], v[1:], None)], AX128, THETA, scale)
    s1 = scale * math.fsum(q[0, 0] * k[0, 0])
    s2 = scale * math.fsum(q[0, 0] * k[1, 0])
    w1 = 1.0 / (1.0 + math.exp(s2 - s1))
    w2 = 1.0 / (1.0 + math.exp(s1 - s2))
    _close(o[0, 0], w1 * v[0, 0] + w2 * v[1, 0], 1e-13, "two keys")


def pin_degenerate():
    """scale = 0 gives the mean of the values; a single key returns its value."""
    q, qp, segs = _tiny_case(71, 128, AX128, 2, [11, 6], 4, prompt=3)
    o = attn64.chunk_attention(q, qp, segs, AX128, THETA, 0.0)
    vall = np.concatenate([v for _, v, _ in segs])
    _close(o, np.broadcast_to(vall.mean(axis=0), o.shape), 1e-13, "scale 0 -> mean")
    k1, v1, p1 = segs[1]
    o1 = attn64.chunk_attention(q, qp, [(k1[:1], v1[:1], p1[:1])], AX128, THETA, 0.3)
    _close(o1, np.broadcast_to(v1[0], o1.shape), 1e-15, "single key")


def pin_translation():
    """Shifting every Q and K position on one axis leaves the output unchanged
    when every segment is rotary, and changes it when a non-rotary prompt
    segment is present (relative-position property of rotary encoding)."""
    q, qp, segs = _tiny_case(81, 128, AX128, 2, [24, 19], 7)
    scale = 1 / math.sqrt(128)
    o = attn64.chunk_attention(q, qp, segs, AX128, THETA, scale)
    for axis, delta in ((0, 100.0), (1, 7.25), (2, -31.0)):
        sh = np.zeros(3)
        sh[axis] = delta
        o2 = attn64.chunk_attention(q, qp + sh, [(k, v, p + sh) for k, v, p in segs], AX128, THETA, scale)
        _close(o2, o, 1e-10, f"translation invariance axis {axis}")
    q, qp, segs = _tiny_case(82, 128, AX128, 2, [24, 19], 7, prompt=8)
    o = attn64.chunk_attention(q, qp, segs, AX128, THETA, scale)
    sh = np.array([100.0, 0.0, 0.0])
    o2 = attn64.chunk_attention(q, qp + sh, [(k, v, None if p is None else p + sh) for k, v, p in segs],
                                AX128, THETA, scale)
    assert np.max(np.abs(o2 - o)) > 1e-4, "a prompt segment must break translation invariance"


def pin_row_selection():
    """Selecting query rows gives exactly those rows of the full output."""
    q, qp, segs = _tiny_case(91, 128, AX128, 2, [33, 8], 20, prompt=4)
    scale = 1 / math.sqrt(128)
    full = attn64.chunk_attention(q, qp, segs, AX128, THETA, scale, block=7)
    rows = np.array([19, 0, 7, 13])
    part = attn64.chunk_attention(q, qp, segs, AX128, THETA, scale, rows=rows)
    _close(part, full[rows], 1e-14, "row selection")


def pin_rmsnorm_closed_form():
    """A constant row c*(1..1) normalises to c / sqrt(c^2 + eps) * w, exactly."""
    rng = _rng(101)
    for d, c, eps in [(4, 3.0, 0.0), (8, -0.25, 1e-2), (128, 7.5, 1e-6), (64, 1e-3, 1e-6)]:
        w = rng.standard_normal(d)
        x = np.full((1, 1, d), c)
        got = norm64.rmsnorm(x, w, eps)[0, 0]
        _close(got, c / math.sqrt(c * c + eps) * w, 1e-14, f"rmsnorm closed form d={d}")


def pin_rmsnorm_invariants():
    """eps = 0: scale-invariant, odd, unit mean square; the weight multiplies element-wise."""
    rng = _rng(102)
    x = rng.standard_normal((5, 3, 128))
    w = rng.standard_normal((3, 128))
    y = norm64.rmsnorm(x, None, 0.0)
    _close(norm64.rmsnorm(37.5 * x, None, 0.0), y, 1e-13, "rmsnorm scale invariance")
    _close(norm64.rmsnorm(-x, None, 0.0), -y, 1e-15, "rmsnorm odd")
    _close(np.mean(y * y, axis=-1), np.ones((5, 3)), 1e-13, "rmsnorm unit mean square")
    _close(norm64.rmsnorm(x, w, 0.0), y * w, 1e-15, "rmsnorm per-head weight")
    _close(norm64.rmsnorm(x, w[1], 1e-3), norm64.rmsnorm(x, None, 1e-3) * w[1], 1e-15, "rmsnorm shared weight")


def pin_brute_force_qknorm():
    """With QK-norm (shared and per-head weights), vectorised oracle == scalar twin."""
    cases = [(111, 8, (2, 2, 4), 2, [4, 2], 3, 2, False), (112, 128, AX128, 2, [3, 2], 2, 1, True),
             (113, 64, (16, 24, 24), 1, [5], 2, 0, False)]
    for tag, d, ax, heads, rows, nq, prompt, per_head in cases:
        q, qp, segs = _tiny_case(tag, d, ax, heads, rows, nq, prompt)
        rng = _rng(tag + 1000)
        shape = (heads, d) if per_head else (d,)
        qn = (1.0 + 0.3 * rng.standard_normal(shape), 1e-3)
        kn = (1.0 + 0.3 * rng.standard_normal(shape), 1e-5)
        scale = 1.0 / math.sqrt(d)
        got = attn64.chunk_attention(3.0 * q, qp, segs, ax, THETA, scale, q_norm=qn, k_norm=kn)
        ref = brute.chunk_attention((3.0 * q).tolist(), qp.tolist(),
                                    [(k.tolist(), v.tolist(), None if p is None else p.tolist()) for k, v, p in segs],
                                    ax, THETA, scale, q_norm=(qn[0].tolist(), qn[1]), k_norm=(kn[0].tolist(), kn[1]))
        _close(got, ref, 1e-12, f"brute force with QK-norm d={d}")


def pin_qknorm_then_rotation():
    """One rotary pair (d = 2), two keys: the score of each key has a closed
    form when the row is normalised first and rotated after; with a
    non-uniform weight the other order gives a different result."""
    w = np.array([1.5, 0.5])
    eps = 0.0
    q = np.array([[[0.8, -1.1]]])
    k = np.array([[[1.3, 0.2]], [[-0.4, 0.9]]])
    v = np.array([[[1.0, 0.0]], [[0.0, 1.0]]])
    pq, pk = np.array([[2.0, 0.0, 0.0]]), np.array([[0.5, 0.0, 0.0], [-1.25, 0.0, 0.0]])

    def nrm(x):
        r = math.sqrt((x[0] ** 2 + x[1] ** 2) / 2 + eps)
        return (x[0] / r * w[0], x[1] / r * w[1])

    qa, qb = nrm(q[0, 0])
    s = []
    for j in range(2):
        ka, kb_ = nrm(k[j, 0])
        delta = pk[j, 0] - pq[0, 0]   # angle of the key minus the angle of the query (theta^0 = 1)
        s.append(qa * (ka * math.cos(delta) - kb_ * math.sin(delta)) + qb * (ka * math.sin(delta) + kb_ * math.cos(delta)))
    p1 = 1.0 / (1.0 + math.exp(s[1] - s[0]))
    ref = np.array([[[p1, 1.0 - p1]]])
    got = attn64.chunk_attention(q, pq, [(k, v, pk)], (2, 0, 0), THETA, 1.0, q_norm=(w, eps), k_norm=(w, eps))
    _close(got, ref, 1e-13, "norm then rotation, one pair")


def pin_split_lse_closed_forms():
    """One key: lse = the scaled score and the partial = v; two keys: log(e^a + e^b);
    many keys: scipy's logsumexp of the fp64 scores."""
    from scipy.special import logsumexp
    rng = _rng(121)
    q = rng.standard_normal((3, 2, 8))
    k = rng.standard_normal((5, 2, 8))
    v = rng.standard_normal((5, 2, 8))
    part, lse = attn64.split_attention(q, k, v, 0.7, [(2, 3), (3, 5), (0, 5)])
    s = 0.7 * np.einsum("nhd,jhd->nhj", q, k)
    _close(lse[0], s[:, :, 2], 1e-14, "lse of one key")
    _close(part[0], np.broadcast_to(v[2], part[0].shape), 1e-14, "one key returns its value")
    _close(lse[1], np.log(np.exp(s[:, :, 3]) + np.exp(s[:, :, 4])), 1e-13, "lse of two keys")
    _close(lse[2], logsumexp(s, axis=-1), 1e-13, "lse vs scipy logsumexp")


def pin_split_merge_identity():
    """Merging disjoint runs, each weighted by exp(its lse), gives the full
    softmax attention (the identity split-key evaluation rests on)."""
    q, qp, segs = _tiny_case(122, 64, (16, 24, 24), 2, [40, 23], 6, prompt=3)
    scale = 0.125
    full = attn64.chunk_attention(q, qp, segs, (16, 24, 24), THETA, scale)
    ranges = [(0, 10), (10, 11), (11, 40), (40, 66)]
    part, lse = attn64.chunk_split_attention(q, qp, segs, (16, 24, 24), THETA, scale, ranges)
    w = np.exp(lse - lse.max(axis=0, keepdims=True))
    merged = np.einsum("snh,snhd->nhd", w, part) / w.sum(axis=0)[:, :, None]
    _close(merged, full, 1e-13, "split merge identity")


def _pool_loops(x, grid_h, grid_w, s):
    """Scalar twin of the pooling: every output element as an fsum over its
    s*s source rows, addressed by flat row index."""
    x = np.asarray(x, dtype=np.float64)
    n, heads, d = x.shape
    per = grid_h * grid_w
    ph, pw = grid_h // s, grid_w // s
    out = np.zeros((n // per * ph * pw, heads, d))
    for f in range(n // per):
        for i in range(ph):
            for j in range(pw):
                src = [f * per + (s * i + a) * grid_w + (s * j + b) for a in range(s) for b in range(s)]
                for h in range(heads):
                    for c in range(d):
                        out[(f * ph + i) * pw + j, h, c] = math.fsum(x[r, h, c] for r in src) / (s * s)
    return out


def pin_pool_brute_force():
    """Pooling == scalar loops over a non-square grid (2 frames, 4 x 8 cells), s = 2 and 4."""
    rng = _rng(130)
    x = rng.standard_normal((2 * 4 * 8, 2, 3))
    for s in (2, 4):
        _close(pool64.pool_frames(x, 4, 8, s), _pool_loops(x, 4, 8, s), 1e-14, f"pool s={s}")


def pin_pool_closed_forms():
    """A frame whose value is a*h + b*w + c (h = grid row, w = column) pools to
    a*hc + b*wc + c at the cell centre hc = s*i + (s-1)/2, wc = s*j + (s-1)/2;
    s = 1 is the identity; frames stay separate (no pooling over time)."""
    gh, gw = 4, 8
    h, w = np.meshgrid(np.arange(gh), np.arange(gw), indexing="ij")
    frames = [3.0 * h - 0.5 * w + 1.0, -2.0 * h + 7.0 * w - 4.0]
    x = np.stack([f.reshape(-1) for f in frames]).reshape(-1)[:, None, None]
    rng = _rng(131)
    y = rng.standard_normal((2 * gh * gw, 1, 4))
    _close(pool64.pool_frames(y, gh, gw, 1), y, 0.0, "s = 1 is the identity")
    for s in (2, 4):
        hc, wc = np.meshgrid(np.arange(gh // s) * s + (s - 1) / 2, np.arange(gw // s) * s + (s - 1) / 2,
                             indexing="ij")
        want = np.concatenate([(3.0 * hc - 0.5 * wc + 1.0).reshape(-1), (-2.0 * hc + 7.0 * wc - 4.0).reshape(-1)])
        _close(pool64.pool_frames(x, gh, gw, s)[:, 0, 0], want, 1e-15, f"affine frame, s={s}")


def pin_pool_invariants():
    """Pooling keeps each frame's mean, is linear, and 2x2 of 2x2 equals 4x4."""
    rng = _rng(132)
    gh, gw = 8, 12
    x = rng.standard_normal((3 * gh * gw, 2, 5))
    y = rng.standard_normal(x.shape)
    p4 = pool64.pool_frames(x, gh, gw, 4)
    _close(p4.reshape(3, -1, 2, 5).mean(axis=1), x.reshape(3, -1, 2, 5).mean(axis=1), 1e-14, "frame mean")
    _close(pool64.pool_frames(2.0 * x - 3.0 * y, gh, gw, 2),
           2.0 * pool64.pool_frames(x, gh, gw, 2) - 3.0 * pool64.pool_frames(y, gh, gw, 2), 1e-14, "linear")
    _close(pool64.pool_frames(pool64.pool_frames(x, gh, gw, 2), gh // 2, gw // 2, 2), p4, 1e-14, "2x2 of 2x2")


def pin_pooled_tier_attention():
    """Attention over a pooled tier == brute force over the hand-pooled keys and
    values at the cell-centre positions (pool first, then rotate)."""
    rng = _rng(133)
    d, ax, gh, gw, s = 8, (2, 2, 4), 4, 4, 2
    k = rng.standard_normal((2 * gh * gw, 1, d))
    v = rng.standard_normal((2 * gh * gw, 1, d))
    pos = np.array([[t, (s * i + (s - 1) / 2), (s * j + (s - 1) / 2)]
                    for t in (1, 2) for i in range(gh // s) for j in range(gw // s)], dtype=np.float64)
    q = rng.standard_normal((3, 1, d))
    qp = rng.random((3, 3)) * 5.0
    got = attn64.chunk_attention(q, qp, [(pool64.pool_frames(k, gh, gw, s), pool64.pool_frames(v, gh, gw, s), pos)],
                                 ax, THETA, 0.4)
    kp, vp = _pool_loops(k, gh, gw, s), _pool_loops(v, gh, gw, s)
    ref = brute.chunk_attention(q, qp, [(kp, vp, pos)], ax, THETA, 0.4)
    _close(got, ref, 1e-12, "pooled tier attention")


def pin_tier_schedule():
    """The reading of the three history tiers (AlayaRenderer-Flash page, key
    contributions): while chunk c is generated the context holds chunk c-1 at
    full resolution, c-2 at 2x2 and c-3 at 4x4, nothing older, and tiers stay
    empty until their chunk exists."""
    want = {0: (None, None, None), 1: (None, None, 0), 2: (None, 0, 1), 3: (0, 1, 2), 4: (1, 2, 3), 9: (6, 7, 8)}
    for c, ages in want.items():
        got = {n: j for n, _, j in tiers64.tier_chunks(c)}
        assert (got["pool4"], got["pool2"], got["prev"]) == ages, (c, got)
    assert [(n, s) for n, s, _ in tiers64.TIERS] == [("pool4", 4), ("pool2", 2), ("prev", 1)]
    assert tiers64.template_t(3) == {"pool4": [1, 2, 3], "pool2": [4, 5, 6], "prev": [7, 8, 9],
                                     "current": [10, 11, 12]}


def pin_tier_ageing():
    """One chunk's data moves down the tiers from one step to the next: the
    4x4 tier at chunk c is the 2x2 pooling of the 2x2 tier at chunk c-1, and
    the 2x2 tier at chunk c the 2x2 pooling of the full-resolution tier at
    chunk c-1; the template positions do not move."""
    rng = _rng(141)
    frames, gh, gw = 2, 8, 4
    data = {j: (rng.standard_normal((frames * gh * gw, 2, 4)), rng.standard_normal((frames * gh * gw, 2, 4)))
            for j in range(6)}
    seg = {c: tiers64.history_segments(lambda j: data[j], c, frames, gh, gw) for c in range(6)}
    assert [len(seg[c]) for c in range(6)] == [0, 1, 2, 3, 3, 3]
    for c in (4, 5):
        (k4, v4, p4), (k2, v2, p2), (k1, v1, p1) = seg[c]
        (_, _, q4), (pk2, pv2, q2), (pk1, pv1, q1) = seg[c - 1]
        _close(k4, pool64.pool_frames(pk2, gh // 2, gw // 2, 2), 1e-14, "4x4 tier = 2x2 of last 2x2 tier (k)")
        _close(v4, pool64.pool_frames(pv2, gh // 2, gw // 2, 2), 1e-14, "4x4 tier = 2x2 of last 2x2 tier (v)")
        _close(k2, pool64.pool_frames(pk1, gh, gw, 2), 1e-14, "2x2 tier = 2x2 of last full tier (k)")
        _close(v1, data[c - 1][1], 0.0, "full tier = previous chunk")
        for a, b in ((p4, q4), (p2, q2), (p1, q1)):
            _close(a, b, 0.0, "template positions")
    assert seg[5][0][0].shape[0] == frames * (gh // 4) * (gw // 4)


def pin_tier_attention_brute():
    """Chunk 3's attention over prompt, reference, the three tiers and itself
    == brute force over hand-pooled tiers at hand-written positions."""
    rng = _rng(142)
    d, ax, frames, gh, gw = 8, (2, 2, 4), 1, 4, 4
    data = {j: (rng.standard_normal((gh * gw, 1, d)), rng.standard_normal((gh * gw, 1, d))) for j in range(4)}
    prompt = (rng.standard_normal((3, 1, d)), rng.standard_normal((3, 1, d)), None)
    ref_pos = np.array([[0.0, i, j] for i in range(gh) for j in range(gw)])
    ref = (rng.standard_normal((gh * gw, 1, d)), rng.standard_normal((gh * gw, 1, d)), ref_pos)
    q = rng.standard_normal((5, 1, d))
    qp = np.array([[4.0, i, j] for i in range(gh) for j in range(gw)])[[0, 3, 6, 9, 15]]
    got = tiers64.chunk_attention(q, qp, [prompt, ref], lambda j: data[j], 3, frames, gh, gw, ax, THETA, 0.4)

    def cells(t, s):
        return np.array([[t, s * i + (s - 1) / 2.0, s * j + (s - 1) / 2.0]
                         for i in range(gh // s) for j in range(gw // s)])

    hand = [prompt, ref,
            (_pool_loops(data[0][0], gh, gw, 4), _pool_loops(data[0][1], gh, gw, 4), cells(1, 4)),
            (_pool_loops(data[1][0], gh, gw, 2), _pool_loops(data[1][1], gh, gw, 2), cells(2, 2)),
            (data[2][0], data[2][1], cells(3, 1)),
            (data[3][0], data[3][1], cells(4, 1))]
    want = brute.chunk_attention(q, qp, hand, ax, THETA, 0.4)
    _close(got, want, 1e-12, "tiered chunk attention")


ALL_PINS = [pin_brute_force, pin_rotation_closed_form, pin_rotation_group, pin_single_pair_scores,
            pin_softmax_rows, pin_constant_v, pin_joint_permutation, pin_zero_angle_is_sdpa,
            pin_two_keys, pin_degenerate, pin_translation, pin_row_selection, pin_rmsnorm_closed_form,
            pin_rmsnorm_invariants, pin_brute_force_qknorm, pin_qknorm_then_rotation, pin_split_lse_closed_forms,
            pin_split_merge_identity, pin_pool_brute_force, pin_pool_closed_forms, pin_pool_invariants,
            pin_pooled_tier_attention, pin_tier_schedule, pin_tier_ageing, pin_tier_attention_brute]
