"""History tiers ageing across a stream of chunks, against the oracle.

Every chunk of a six-chunk stream (the tiers fill over the first four) is
compared in full with ``oracle.tiers64`` on the same seeded values; the
static prompt / reference rows of the packed context stay bitwise unchanged
while the dynamic region is rewritten in place every step. A 1344x768 stream
is checked on sampled rows (rows are independent, so those rows are exact).
"""

import numpy as np
import pytest
import torch

from gpu_util import assert_parity, note, sample_rows
from oracle import tiers64
from streaming_video_diffusion_amd import inputs as I
from streaming_video_diffusion_amd.stream import TierStreamAttention

pytestmark = pytest.mark.gpu


def _run(stream, chunks, rows_of=None):
    ts = TierStreamAttention(stream)
    ts.pack_static()
    torch.cuda.synchronize()
    n_static = ts.static_rows
    k0 = ts.ctx.k_data().view(stream.heads, ts.ctx.capacity_rows, stream.head_dim)[:, :n_static].clone()
    v0 = ts.ctx.v_data().clone()
    static = stream.static_kv()
    tt = tiers64.template_t(stream.frames)
    template = {"pool4": tt["pool4"], "pool2": tt["pool2"], "prev": tt["prev"], "current": tt["current"]}
    # the stream's template is the oracle's
    for slot, name in enumerate(["pool4", "pool2", "prev", "current"]):
        assert stream.slot_t(slot) == template[name]
    for c in range(chunks):
        q = stream.chunk_q(c)
        k, v = stream.chunk_kv(c)
        dt = ts.dtype
        note(f"[gpu] {stream.name} chunk {c}")
        out = ts.step(torch.from_numpy(q).cuda().to(dt), torch.from_numpy(k).cuda().to(dt),
                      torch.from_numpy(v).cuda().to(dt))
        torch.cuda.synchronize()
        got = out.float().cpu().numpy().astype(np.float64)
        rows = None if rows_of is None else rows_of(c)
        weights = stream.norm_weights()
        qn, kn = (None, None) if weights is None else ((weights[0], stream.norm_eps), (weights[1], stream.norm_eps))
        want = tiers64.chunk_attention(q, stream.slot_positions(len(ts.TIERS)), static, stream.chunk_kv, c,
                                       stream.frames, stream.grid_h, stream.grid_w, stream.axis_dims, stream.theta,
                                       stream.scale, rows=rows, q_norm=qn, k_norm=kn)
        rel, mx = assert_parity(got if rows is None else got[rows], want, stream.dtype, f"{stream.name} chunk {c}")
        note(f"  chunk {c}: nk {ts.ctx.rows} rel-L2 {rel:.3e} max-abs {mx:.3e}")
        expect_nk = n_static + sum(stream.chunk_rows // (s * s) for s, age in ts.TIERS if c - age >= 0) + stream.chunk_rows
        assert ts.ctx.rows == expect_nk
        # the static rows of K are never rewritten
        kn = ts.ctx.k_data().view(stream.heads, ts.ctx.capacity_rows, stream.head_dim)[:, :n_static]
        assert torch.equal(kn, k0)
        if stream.dtype == "bf16":   # V^T [H][d][C]: the static columns of every d-row stay as packed
            vt = ts.ctx.v_data().view(stream.heads, stream.head_dim, ts.ctx.capacity_rows)
            vt0 = v0.view(stream.heads, stream.head_dim, ts.ctx.capacity_rows)
            assert torch.equal(vt[:, :, :n_static // 16 * 16], vt0[:, :, :n_static // 16 * 16])
        else:                        # V [H][C][d]
            vr = ts.ctx.v_data().view(stream.heads, ts.ctx.capacity_rows, stream.head_dim)
            vr0 = v0.view(stream.heads, ts.ctx.capacity_rows, stream.head_dim)
            assert torch.equal(vr[:, :n_static], vr0[:, :n_static])
    return ts


@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("bf16", 64), ("f32", 64)])
def test_tier_stream_small_every_chunk(dtype, d):
    _run(I.tier_stream_small(dtype, d), 6)


@pytest.mark.parametrize("kind", ["shared", "per_head"])
def test_tier_stream_small_qknorm(kind):
    import dataclasses
    _run(dataclasses.replace(I.tier_stream_small("bf16", 128), name=f"tier_stream_small_qkn_{kind}", qk_norm=kind), 5)


def test_tier_stream_1344x768_sampled():
    st = I.tier_stream_1344x768()
    _run(st, 5, rows_of=lambda c: sample_rows(st.chunk_rows, extra=16, seed=c))
