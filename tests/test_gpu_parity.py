"""HIP path vs the fp64 oracle, element by element, through the C ABI.

Small workloads are compared in full; the full-size 1344x768 workloads are
compared on sampled query rows (rows are independent, so the oracle's value
of a sampled row is exact), in the same launch configuration the benchmark
times.
"""

import numpy as np
import pytest
import torch

from gpu_util import assert_parity, note, oracle, run, sample_rows
from streaming_video_diffusion_amd import inputs as I

pytestmark = pytest.mark.gpu


def test_tiny_f32_full():
    w = I.tiny_f32()
    ca, out = run(w)
    ref = oracle(ca)
    rel, _ = assert_parity(out, ref, "f32", w.name)
    note(f"  rel-L2 {rel:.3e}")


@pytest.mark.parametrize("out_dtype", [None, torch.float32], ids=["out_bf16", "out_f32"])
def test_lowres_bf16_full(out_dtype):
    w = I.lowres_bf16()
    ca, out = run(w, out_dtype=out_dtype)
    ref = oracle(ca)
    rel, mx = assert_parity(out, ref, "bf16", w.name)
    note(f"  rel-L2 {rel:.3e} max-abs {mx:.3e}")


RAGGED = [
    # name, dtype, heads, head_dim, seg_rows, nq, prompt
    ("ragged_bf16_d128", "bf16", 3, 128, [17, 100, 333], 300, 5),
    ("ragged_bf16_d64", "bf16", 2, 64, [70, 1, 190], 257, 0),
    ("single_key", "bf16", 2, 128, [1], 33, 0),
    ("single_query", "bf16", 2, 128, [65, 64], 1, 3),
    ("empty_segment", "bf16", 2, 128, [40, 0, 88], 130, 7),
    ("tile_exact", "bf16", 1, 128, [128], 512, 0),
    ("ragged_f32_d128", "f32", 2, 128, [33, 70], 130, 4),
    ("ragged_f32_d64", "f32", 3, 64, [1, 45], 65, 0),
]


@pytest.mark.parametrize("case", RAGGED, ids=[c[0] for c in RAGGED])
def test_ragged_shapes(case):
    name, dtype, heads, d, rows, nq, prompt = case
    w = I.custom(name, 100 + RAGGED.index(case), dtype, heads, d, rows, nq, prompt_rows=prompt)
    ca, out = run(w)
    assert_parity(out, oracle(ca), dtype, name)


def test_unrotated_equals_oracle_sdpa():
    w = I.custom("no_rotary", 150, "bf16", 2, 128, [50, 77], 90, rotary=False)
    ca, out = run(w)
    assert ca.q_table is None and all(s["table"] is None for s in ca.segs)
    assert_parity(out, oracle(ca), "bf16", "no rotary")


def test_strided_q_and_out():
    """Q as a view of a fused [N][3][H][d] tensor, output into a wider buffer."""
    w = I.lowres_bf16()
    ca, _ = run(w)
    fused = torch.zeros((w.nq, 3, w.heads, w.head_dim), dtype=torch.bfloat16, device="cuda")
    fused[:, 1] = ca.q
    wide = torch.full((w.nq, w.heads + 2, w.head_dim + 64), float("nan"), dtype=torch.float32, device="cuda")
    out_view = wide[:, 1:1 + w.heads, 32:32 + w.head_dim]
    from streaming_video_diffusion_amd import binding as B
    B.sa_forward(ca.ctx, fused[:, 1], ca.q_table, w.scale, out=out_view)
    torch.cuda.synchronize()
    got = out_view.cpu().numpy().astype(np.float64)
    assert_parity(got, oracle(ca), "bf16", "strided")
    assert torch.isnan(wide[:, 0]).all() and torch.isnan(wide[:, 1:1 + w.heads, :32]).all()
    assert torch.isnan(wide[:, 1:1 + w.heads, 32 + w.head_dim:]).all()


FULL = [I.full_1344x768, I.hier_1344x768, I.video_audio_1344x768]


@pytest.mark.parametrize("make", FULL, ids=[f.__name__ for f in FULL])
def test_full_size_sampled_rows(make):
    w = make()
    for call in range(w.calls):
        ca, out = run(w, call=call)
        rows = sample_rows(w.nq, seed=call)
        ref = oracle(ca, rows=rows)
        rel, mx = assert_parity(out[rows], ref, "bf16", f"{w.name} call {call}")
        note(f"  {w.name} call {call}: {len(rows)} rows, rel-L2 {rel:.3e} max-abs {mx:.3e}")
        assert np.isfinite(out).all()
        del ca
        torch.cuda.empty_cache()


# The kernel's fast path keeps the running max at 0 and is exact while every
# tile's max (log2 units) stays within +-8 of it; these cases leave that band
# and run the rescaling path. Unrotated bf16 inputs and a softmax scale of
# 2^k * ln 2 keep the scores exact on the GPU (the query pre-scale is then
# exactly 2^k), so the comparison stays within the bf16 bounds.
@pytest.mark.parametrize("c_log2", [0.5, 4.0], ids=["scale_x0.5", "scale_x4"])
def test_rescaling_path_large_scores(c_log2):
    import math
    w = I.custom(f"peaked{c_log2}", 400 + int(c_log2 * 10), "bf16", 3, 128, [150, 333], 300, rotary=False,
                 prompt_rows=40, scale=float(np.float32(c_log2 * math.log(2.0))))
    ca, out = run(w)
    rel, mx = assert_parity(out, oracle(ca), "bf16", w.name)
    note(f"  {w.name}: rel-L2 {rel:.3e} max-abs {mx:.3e}")


def test_rescaling_path_negative_first_tile():
    """The first key tile scores far below 0 for every query; later tiles do not."""
    import math
    from oracle import attn64
    from streaming_video_diffusion_amd.stream import ChunkAttention
    w = I.custom("negfirst", 410, "bf16", 2, 128, [64, 200], 150, rotary=False,
                 scale=float(np.float32(0.5 * math.log(2.0))))
    q = w.q()
    segs = [w.kv(i) for i in range(len(w.segments))]
    qdir = q[:1]
    q = I.round_bf16(qdir + 0.05 * q)                       # every query close to qdir
    k0 = I.round_bf16(np.broadcast_to(-3.0 * qdir, segs[0][0].shape))  # first tile: scores ~ -3 |q|^2
    segs = [(k0, segs[0][1], None), (segs[1][0], segs[1][1], None)]
    ca = ChunkAttention(w)
    ca.q.copy_(torch.from_numpy(q).to(torch.bfloat16))
    ca.segs[0]["k"].copy_(torch.from_numpy(np.ascontiguousarray(k0)).to(torch.bfloat16))
    note("[gpu] negative first tile")
    ca.pack_static()
    out = ca.step().float().cpu().numpy().astype(np.float64)
    torch.cuda.synchronize()
    ref = attn64.chunk_attention(q, None, segs, w.axis_dims, w.theta, w.scale)
    assert_parity(out, ref, "bf16", "negative first tile")


# Rows the main pass cannot hold at a fixed anchor go through the second pass:
# a row whose every score lies far below the float range of 2^s (its row sum
# underflows), and rows whose largest scores overflow 2^s, mixed with ordinary
# rows in the same workgroups.
def test_second_pass_underflowing_rows():
    """Every key is close to a direction u; queries -16 u (exact in bf16) score about -260 (log2 units)."""
    from oracle import attn64
    from streaming_video_diffusion_amd.stream import ChunkAttention
    w = I.custom("underflow", 411, "bf16", 2, 128, [64, 333], 300, rotary=False, prompt_rows=7)
    rng = np.random.default_rng(5)
    u = I.round_bf16(rng.standard_normal((1, w.heads, w.head_dim)).astype(np.float32))
    q = w.q()
    q[:40] = -16.0 * u  # rows 0..39: every score far below 2^-126
    segs = []
    for i in range(len(w.segments)):
        k, v = w.kv(i)
        k = I.round_bf16(u + 0.05 * k)
        segs.append((k, v, None))
    ca = ChunkAttention(w)
    ca.q.copy_(torch.from_numpy(q).to(torch.bfloat16))
    for s, (k, v, _) in zip(ca.segs, segs):
        s["k"].copy_(torch.from_numpy(np.ascontiguousarray(k)).to(torch.bfloat16))
    note("[gpu] second pass: underflowing rows")
    ca.pack_static()
    out = ca.step().float().cpu().numpy().astype(np.float64)
    torch.cuda.synchronize()
    assert np.isfinite(out).all()
    ref = attn64.chunk_attention(q, None, segs, w.axis_dims, w.theta, w.scale)
    rel, mx = assert_parity(out, ref, "bf16", "underflowing rows")
    note(f"  rel-L2 {rel:.3e} max-abs {mx:.3e}")


def test_second_pass_mixed_rows_keep_neighbours_bitwise():
    """A few query rows scaled by 32 overflow; every row matches the oracle and
    the other rows are bit-identical to a run without the scaled rows.

    Unrotated inputs and a softmax scale of ln2 / 8 make the query pre-scale
    exactly 2^-3, so even the scaled rows' scores (up to about 2^7 in log2
    units) are exact on the GPU and the comparison stays within the bf16
    bounds; ordinary rows peak near 4.5 and stay in the main pass."""
    import math
    w = I.custom("mixed", 412, "bf16", 3, 128, [100, 400, 530], 700, rotary=False, prompt_rows=11,
                 scale=float(np.float32(math.log(2.0) / 8.0)))
    ca, base = run(w)
    a = ca.forward().clone()
    rows = [3, 257, 258, 511, 699]
    q = w.q()
    q[rows] *= 32.0
    ca.q.copy_(torch.from_numpy(q).to(torch.bfloat16))
    note("[gpu] second pass: mixed rows")
    b = ca.forward()
    torch.cuda.synchronize()
    keep = torch.ones(w.nq, dtype=torch.bool, device="cuda")
    keep[rows] = False
    assert torch.equal(a[keep], b[keep])
    from oracle import attn64
    segs = [(*w.kv(i), s.pos) for i, s in enumerate(w.segments)]
    ref = attn64.chunk_attention(q, None, segs, w.axis_dims, w.theta, w.scale, rows=np.array(rows))
    got = b[rows].float().cpu().numpy().astype(np.float64)
    rel, mx = assert_parity(got, ref, "bf16", "scaled rows")
    note(f"  scaled rows rel-L2 {rel:.3e} max-abs {mx:.3e}")
