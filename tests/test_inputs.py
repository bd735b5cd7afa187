"""Seeded workload generator: shapes, positions, rounding and determinism."""

import json
import os

import numpy as np
import torch

from streaming_video_diffusion_amd import inputs as I

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "workload_shapes.json")


def test_shapes_match_fixture():
    fx = json.load(open(GOLDEN))
    assert set(I.CONFIGS) == {k for k in fx if not k.startswith("_")}
    for name, make in I.CONFIGS.items():
        w, want = make(), fx[name]
        assert (w.heads, w.head_dim, w.nq, w.nk) == (want["heads"], want["head_dim"], want["nq"], want["nk"])
        assert [[s.name, s.rows] for s in w.segments] == want["segments"]
        assert w.calls == want.get("calls", 1)
        assert sum(a for a in w.axis_dims) == w.head_dim
        for s in w.segments:
            assert (s.pos is None) == (s.name == "prompt")
            if s.pos is not None:
                assert s.pos.shape == (s.rows, 3) and s.pos.dtype == np.float32


def test_positions_layout():
    w = I.full_1344x768()
    ref = w.segments[1].pos
    assert ref[0].tolist() == [0, 0, 0] and ref[1].tolist() == [0, 0, 1]
    assert ref[84].tolist() == [0, 1, 0] and ref[-1].tolist() == [0, 47, 83]
    cur = w.segments[-1].pos
    assert np.array_equal(cur, w.q_pos)
    assert cur[0, 0] == 4 and cur[-1, 0] == 6
    h = I.hier_1344x768()
    pool4, pool2 = h.segments[2].pos, h.segments[3].pos
    assert pool4[0].tolist() == [1, 1.5, 1.5] and pool4[-1].tolist() == [3, 45.5, 81.5]
    assert pool2[0].tolist() == [4, 0.5, 0.5] and pool2[-1].tolist() == [6, 46.5, 82.5]
    va = I.video_audio_1344x768()
    aud = va.q_pos[-40:]
    assert np.all(aud[:, 1:] == 0)
    np.testing.assert_array_equal(aud[:, 0], np.float32(7 + 0.15 * np.arange(40)))
    assert va.q_pos[24191].tolist() == [12, 47, 83]


def test_round_bf16_matches_torch():
    x = np.random.default_rng(5).standard_normal(100000).astype(np.float32) * 3
    x[:4] = [1.00390625, 1.01171875, -2.00781250, 0.0]   # exact ties either way
    ours = I.round_bf16(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy()
    np.testing.assert_array_equal(ours, ref)


def test_draws_are_seeded_and_distinct():
    w = I.lowres_bf16()
    a, b = w.q(), w.q()
    np.testing.assert_array_equal(a, b)
    k0, v0 = w.kv(0)
    assert not np.array_equal(k0, v0)
    assert np.array_equal(I.round_bf16(a), a)
    va = I.video_audio_1344x768()
    assert va.calls == 2
    ss = [np.random.SeedSequence([I.ENTROPY, 5, c, 0]).generate_state(2).tolist() for c in (0, 1)]
    assert ss[0] != ss[1]
    assert abs(float(a.std()) - 1.0) < 0.02


def test_query_variants():
    """Recomputed history + current as queries, the 7-frame first window, the prefix pass."""
    hq = I.history_query_1344x768()
    assert (hq.nq, hq.nk) == (24192, 28480)
    np.testing.assert_array_equal(hq.q_pos[:12096], hq.segments[2].pos)
    np.testing.assert_array_equal(hq.q_pos[12096:], hq.segments[3].pos)
    fw = I.first_window_1344x768()
    assert (fw.nq, fw.nk) == (7 * 4032, 256 + 4032 + 7 * 4032)
    assert fw.q_pos[0, 0] == 1 and fw.q_pos[-1].tolist() == [7, 47, 83]
    assert np.array_equal(fw.segments[-1].pos, fw.q_pos) and fw.segments[-1].dynamic
    ps = I.prefix_self_1344x768()
    assert (ps.nq, ps.nk) == (3 * 4032, 256 + 3 * 4032)
    assert not any(s.dynamic for s in ps.segments)
    np.testing.assert_array_equal(ps.q_pos, np.concatenate([ps.segments[1].pos, ps.segments[2].pos]))
    ids = {w().cfg_id for w in list(I.CONFIGS.values()) + list(I.VARIANTS.values())}
    assert len(ids) == len(I.CONFIGS) + len(I.VARIANTS)


def test_pooled_positions_are_cell_means():
    """A pooled tier's positions are the mean of the full-resolution positions
    each cell covers (the cell centre), as the oracle pools them."""
    from oracle import pool64
    for s in (2, 4):
        full = I.frame_positions([1, 2], 48, 84)
        pooled = I.frame_positions([1, 2], 48, 84, pool=s)
        np.testing.assert_array_equal(pooled, pool64.pool_frames(full[:, None, :], 48, 84, s)[:, 0, :])


def test_tier_stream_draws_and_template():
    from oracle import tiers64
    st = I.tier_stream_small()
    (pk, pv, ppos), (rk, rv, rpos) = st.static_kv()
    assert pk.shape == (40, 3, 128) and ppos is None
    assert rk.shape == (12 * 16, 3, 128) and np.all(rpos[:, 0] == 0)
    assert np.array_equal(st.chunk_q(2), st.chunk_q(2))
    draws = [st.chunk_q(0), *st.chunk_kv(0), *st.chunk_kv(1), pk, pv, rk[:40], rv[:40]]
    for i in range(len(draws)):
        for j in range(i + 1, len(draws)):
            n = min(len(draws[i]), len(draws[j]))
            assert not np.array_equal(draws[i][:n], draws[j][:n])
    assert np.all(st.chunk_q(0) == I.round_bf16(st.chunk_q(0)))
    tt = tiers64.template_t(st.frames)
    for slot, name in enumerate(["pool4", "pool2", "prev", "current"]):
        assert st.slot_t(slot) == tt[name]
    for slot, (name, s, _) in enumerate(tiers64.TIERS):
        want = tiers64.cell_positions(tt[name], st.grid_h, st.grid_w, s)
        np.testing.assert_array_equal(st.slot_positions(slot, s), want.astype(np.float32))
