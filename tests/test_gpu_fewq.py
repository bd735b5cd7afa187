"""The few-query path of the bf16 forward (sa_forward_ws / sa_forward_noalloc
with 1 <= nq <= SA_FEW_QUERY_ROWS): every wave of a key-split kernel streams
its own run of a head's key tiles for all the query rows, the runs merged by
their log-sum-exps. Checked against the fp64 oracle on every output element,
and against the paths it stands beside."""

import dataclasses
import math

import numpy as np
import pytest
import torch

from gpu_util import assert_parity, note, oracle, run
from streaming_video_diffusion_amd import binding as B
from streaming_video_diffusion_amd import inputs as I

pytestmark = pytest.mark.gpu


def fewq_bytes(nq, heads, head_dim, nk):
    """Workspace of the few-query plan as the header states it (0: not used)."""
    if not 1 <= nq <= B.SA_FEW_QUERY_ROWS:
        return 0
    n_cu = torch.cuda.get_device_properties(0).multi_processor_count
    runs = max(1, min(4 * n_cu // heads, math.ceil(nk / 64)))
    n = runs * nq * heads * (head_dim + 1) * 4
    return n if n <= B.SA_NOALLOC_SCRATCH_BYTES else 0


def test_workspace_bytes_of_the_few_query_plan():
    for nq, heads, d, nk in [(1, 150, 128, 3000), (40, 40, 128, 52752), (64, 6, 64, 1000), (17, 2, 128, 100),
                             (40, 5, 128, 28480)]:
        ctx = B.PackedContext(heads, d, torch.bfloat16, (nk + 63) // 64 * 64)
        ctx.rows = nk
        want = fewq_bytes(nq, heads, d, nk)
        assert want > 0
        assert B.sa_forward_workspace_bytes(ctx, nq) == want, (nq, heads, d, nk)
    # One row more than the path takes: the plain forward or the stream-K tail.
    ctx = B.PackedContext(6, 128, torch.bfloat16, 1024)
    ctx.rows = 1000
    assert B.sa_forward_workspace_bytes(ctx, B.SA_FEW_QUERY_ROWS + 1) != fewq_bytes(64, 6, 128, 1000)
    # A plan larger than the library's scratch (4096 heads x 64 rows: one run each,
    # 64 x 4096 x 129 x 4 B = 135.3 MB) is not used: such a call sizes its
    # workspace for the other paths.
    assert 64 * 4096 * 129 * 4 > B.SA_NOALLOC_SCRATCH_BYTES
    ctx = B.PackedContext(4096, 128, torch.bfloat16, 64)
    ctx.rows = 64
    assert fewq_bytes(64, 4096, 128, 64) == 0
    assert B.sa_forward_workspace_bytes(ctx, 64) <= B.SA_NOALLOC_SCRATCH_BYTES


def test_plan_larger_than_the_scratch_takes_the_other_paths():
    """4096 heads of 64 rows over 64 keys: no few-query plan; sa_forward_ws and
    sa_forward_noalloc still agree with the oracle."""
    w = I.custom("fewq_too_big", 725, "bf16", 4096, 128, [24], 64, prompt_rows=40)
    assert w.nk == 64
    ca, out = run(w)
    rows = np.array([0, 31, 32, 63])
    heads = np.array([0, 1, 2047, 4095])
    ref = oracle(ca, rows=rows)
    rel, mx = assert_parity(out[rows][:, heads], ref[:, heads], "bf16", w.name)
    note(f"  {w.name}: rel-L2 {rel:.3e} max-abs {mx:.3e}")
    got = B.sa_forward_noalloc(ca.ctx, ca.q, torch.empty_like(ca.out), ca.q_table, w.scale)
    torch.cuda.synchronize()
    assert torch.equal(got, ca.out)


# (nq, head_dim, heads, out dtype, qk-norm): one and two 32-row query blocks,
# both head dims, rows on and around the block edges.
CASES = [
    (1, 128, 6, None, None),
    (17, 64, 6, None, "per_head"),
    (32, 128, 3, torch.float32, None),
    (33, 128, 6, None, "shared"),
    (40, 128, 5, None, "per_head"),
    (64, 64, 7, torch.float32, None),
    (64, 128, 4, None, None),
]


@pytest.mark.parametrize("nq,d,heads,out_dtype,qkn", CASES,
                         ids=[f"nq{c[0]}_d{c[1]}_h{c[2]}_{'f32' if c[3] else 'bf16'}_{c[4] or 'noqkn'}" for c in CASES])
def test_few_query_rows_against_the_oracle(nq, d, heads, out_dtype, qkn):
    """Ragged context (prompt + two rotary segments, not a multiple of 64 keys),
    so that runs end inside the context and the last run holds its padded tile."""
    w = dataclasses.replace(I.custom(f"fewq_{nq}_{d}", 700 + nq + d, "bf16", heads, d, [611, 358], nq,
                                     prompt_rows=23), qk_norm=qkn)
    assert w.nk % 64 != 0
    ca, out = run(w, out_dtype=out_dtype)
    assert ca.workspace is not None and ca.workspace.numel() == fewq_bytes(nq, heads, d, w.nk)
    rel, mx = assert_parity(out, oracle(ca), "bf16", w.name)
    note(f"  {w.name}: rel-L2 {rel:.3e} max-abs {mx:.3e}")
    plain = B.sa_forward(ca.ctx, ca.q, ca.q_table, w.scale, out_dtype=ca.out_dtype, q_norm=ca.q_norm)
    torch.cuda.synchronize()
    d_rel = float(torch.linalg.norm((plain.float() - ca.out.float()).flatten()) / torch.linalg.norm(plain.float()))
    assert d_rel < 5e-3, d_rel


def test_two_key_tiles():
    """100 keys are two tiles: as many runs as tiles (one each), the second
    one holding the padded tile."""
    w = I.custom("fewq_empty_runs", 720, "bf16", 3, 128, [77], 40, prompt_rows=23)
    assert w.nk == 100
    ca, out = run(w)
    assert ca.workspace is not None
    rel, mx = assert_parity(out, oracle(ca), "bf16", w.name)
    note(f"  {w.name}: rel-L2 {rel:.3e} max-abs {mx:.3e}")


def test_second_pass_overflowing_rows():
    """Rows scaled by 32 overflow the anchor-0 pass (scores up to about 2^7 in
    log2 units): their waves run again anchored at the exact row max. Unrotated
    inputs and a softmax scale of ln2 / 8 keep the scores exact on the GPU."""
    w = I.custom("fewq_mixed", 721, "bf16", 3, 128, [400, 530], 40, rotary=False, prompt_rows=11,
                 scale=float(np.float32(math.log(2.0) / 8.0)))
    ca, _ = run(w)
    q = w.q()
    q[[0, 5, 31, 32, 39]] *= 32.0
    ca.q.copy_(torch.from_numpy(q).to(torch.bfloat16))
    note("[gpu] few-query second pass: overflowing rows")
    out = ca.forward().float().cpu().numpy().astype(np.float64)
    torch.cuda.synchronize()
    assert np.isfinite(out).all()
    from oracle import attn64
    segs = [(*w.kv(i), s.pos) for i, s in enumerate(w.segments)]
    ref = attn64.chunk_attention(q, None, segs, w.axis_dims, w.theta, w.scale)
    rel, mx = assert_parity(out, ref, "bf16", "overflowing rows")
    note(f"  rel-L2 {rel:.3e} max-abs {mx:.3e}")


def test_second_pass_underflowing_rows():
    """Every key is close to a direction u; queries -16 u score about -260
    (log2 units), far below the float range of 2^s."""
    from oracle import attn64
    from streaming_video_diffusion_amd.stream import ChunkAttention
    w = I.custom("fewq_underflow", 722, "bf16", 2, 128, [64, 333], 40, rotary=False, prompt_rows=7)
    rng = np.random.default_rng(7)
    u = I.round_bf16(rng.standard_normal((1, w.heads, w.head_dim)).astype(np.float32))
    q = w.q()
    q[:20] = -16.0 * u
    segs = []
    for i in range(len(w.segments)):
        k, v = w.kv(i)
        segs.append((I.round_bf16(u + 0.05 * k), v, None))
    ca = ChunkAttention(w)
    ca.q.copy_(torch.from_numpy(q).to(torch.bfloat16))
    for s, (k, v, _) in zip(ca.segs, segs):
        s["k"].copy_(torch.from_numpy(np.ascontiguousarray(k)).to(torch.bfloat16))
    note("[gpu] few-query second pass: underflowing rows")
    ca.pack_static()
    out = ca.step().float().cpu().numpy().astype(np.float64)
    torch.cuda.synchronize()
    assert ca.workspace is not None
    assert np.isfinite(out).all()
    ref = attn64.chunk_attention(q, None, segs, w.axis_dims, w.theta, w.scale)
    rel, mx = assert_parity(out, ref, "bf16", "underflowing rows")
    note(f"  rel-L2 {rel:.3e} max-abs {mx:.3e}")


def test_strided_output_view_and_no_workspace():
    """The merge writes through the caller's strides and nothing outside the
    view changes; without a workspace the call is exactly sa_forward."""
    w = I.custom("fewq_strided", 723, "bf16", 5, 128, [700, 300], 40, prompt_rows=9)
    ca, _ = run(w)
    want = ca.out.clone()
    big = torch.full((w.nq, w.heads + 3, w.head_dim + 64), 7.0, dtype=torch.bfloat16, device="cuda")
    view = big[:, 1:1 + w.heads, 32:32 + w.head_dim]
    B.sa_forward_ws(ca.ctx, ca.q, ca.q_table, w.scale, out=view, workspace=ca.workspace)
    a = B.sa_forward_ws(ca.ctx, ca.q, ca.q_table, w.scale, workspace=None)
    b = B.sa_forward(ca.ctx, ca.q, ca.q_table, w.scale)
    torch.cuda.synchronize()
    assert torch.equal(view, want)
    outside = torch.ones_like(big, dtype=torch.bool)
    outside[:, 1:1 + w.heads, 32:32 + w.head_dim] = False
    assert bool((big[outside] == 7.0).all())
    assert torch.equal(a, b)


def test_noalloc_is_the_workspace_forward_bitwise():
    """Same launches as sa_forward_ws; two calls in a row, the second smaller."""
    w = I.custom("fewq_noalloc", 724, "bf16", 6, 128, [900, 500], 64, prompt_rows=20)
    ca, _ = run(w)
    for n in (64, 9):
        q, qt = ca.q[:n], ca.q_table[:n]
        ws = torch.empty(B.sa_forward_workspace_bytes(ca.ctx, n), dtype=torch.uint8, device="cuda")
        want = B.sa_forward_ws(ca.ctx, q, qt, w.scale, workspace=ws)
        got = B.sa_forward_noalloc(ca.ctx, q, torch.empty_like(want), qt, w.scale)
        torch.cuda.synchronize()
        assert torch.equal(got, want), n


def test_audio_only_queries_full_size():
    """The 40 audio queries of the 1 s video+audio chunk over its 52752 keys and
    40 heads: every output element against the oracle."""
    w = I.video_audio_1344x768()
    from test_gpu_split import packed
    ca = packed(w)
    q, qt = ca.q[w.nq - 40:], ca.q_table[w.nq - 40:]
    need = B.sa_forward_workspace_bytes(ca.ctx, 40)
    assert need == fewq_bytes(40, w.heads, w.head_dim, w.nk)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    got = B.sa_forward_ws(ca.ctx, q, qt, w.scale, workspace=ws, out_dtype=torch.float32)
    torch.cuda.synchronize()
    rows = np.arange(w.nq - 40, w.nq)
    rel, mx = assert_parity(got.cpu().numpy().astype(np.float64), oracle(ca, rows=rows), "bf16", "audio rows")
    note(f"  audio rows: rel-L2 {rel:.3e} max-abs {mx:.3e}")


@pytest.mark.parametrize("entry", ["noalloc", "ws"])
def test_captured_and_replayed(entry):
    """The few-query path captured into a HIP graph (after one eager call) and
    replayed; each replay bitwise equal to the eager result, with an eager
    few-query call of other size on the same scratch or workspace between."""
    w = I.custom("fewq_graph", 726, "bf16", 40, 128, [2000, 1500], 40, prompt_rows=32)
    ca, _ = run(w)
    ws = torch.empty(B.sa_forward_workspace_bytes(ca.ctx, w.nq), dtype=torch.uint8, device="cuda")

    def call(q, qt, out, stream=None):
        if entry == "noalloc":
            return B.sa_forward_noalloc(ca.ctx, q, out, qt, w.scale, stream=stream)
        return B.sa_forward_ws(ca.ctx, q, qt, w.scale, out=out, stream=stream, workspace=ws)

    eager = torch.empty_like(ca.out)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call(ca.q, ca.q_table, eager, stream=side)
    torch.cuda.synchronize()
    out = torch.empty_like(ca.out)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=side):
        call(ca.q, ca.q_table, out, stream=side)
    torch.cuda.synchronize()
    for i in range(3):
        out.fill_(float("nan"))
        call(ca.q[:17], ca.q_table[:17], torch.empty_like(ca.out[:17]))  # eager work on the same scratch
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), f"replay {i}"
