"""The stream-K tail's index arithmetic, restated on the host.

The forward's tail launch cuts the flattened (tail unit, key tile) range of
units * T tiles at b_i = floor(i * total / G) among G workgroups; a unit cut by
a boundary leaves one piece per workgroup in slot 2i (the unit is the first of
that workgroup's range) or 2i + 1 (its last). The merge finds a unit's pieces
by inverting the cut: the workgroup holding tile x is floor(((x + 1) G - 1) /
total). This test checks on random sizes that the merge's view of every unit
is exactly the kernel's partition, that every tile is covered once, that a
unit is stored whole exactly when the merge skips it, and that slots are
unique and below 2G (the workspace holds 2G slots).
"""

import random


def kernel_pieces(units, T, G):
    total = units * T
    pieces = {}
    for i in range(G):
        p, b1 = i * total // G, (i + 1) * total // G
        first = p // T
        while p < b1:
            ul = p // T
            t0 = p - ul * T
            t1 = min(T, t0 + (b1 - p))
            slot = None if (t0 == 0 and t1 == T) else 2 * i + (0 if ul == first else 1)
            pieces.setdefault(ul, []).append((i, t0, t1, slot))
            p += t1 - t0
    return pieces


def merge_view(units, T, G, ul):
    total = units * T
    x0, x1 = ul * T, ul * T + T - 1
    i0, i1 = ((x0 + 1) * G - 1) // total, ((x1 + 1) * G - 1) // total
    if i0 == i1:
        return None
    return [(i, 2 * i if (i * total // G) // T == ul else 2 * i + 1)
            for i in range(i0, i1 + 1) if (i + 1) * total // G > i * total // G]


def test_partition_and_merge_agree():
    rng = random.Random(7)
    cases = [(160, 445, 256), (144, 508, 256), (216, 445, 256), (1, 4, 256), (300, 1, 256)]
    cases += [(rng.randint(1, 300), rng.randint(1, 600), rng.choice([8, 64, 256, 304])) for _ in range(2000)]
    for units, T, G in cases:
        pieces = kernel_pieces(units, T, G)
        used = set()
        for ul in range(units):
            ps = pieces[ul]
            assert ps[0][1] == 0 and ps[-1][2] == T
            assert all(a[2] == b[1] for a, b in zip(ps, ps[1:]))   # contiguous, no overlap
            view = merge_view(units, T, G, ul)
            if len(ps) == 1:
                assert ps[0][3] is None and view is None
            else:
                assert view == [(i, s) for i, _, _, s in ps]
                for _, _, _, s in ps:
                    assert 0 <= s < 2 * G and s not in used
                    used.add(s)
