"""sa_forward_noalloc: the stream-K tail forward with the library's own
per-device scratch, against sa_forward_ws with a caller workspace (the same kernels and
launches, so the two must agree bit for bit) and against the fp64 oracle on
sampled rows. Two calls in a row, the second on a smaller input, so the
second meets the scratch as the first left it."""

import pytest
import torch

from gpu_util import assert_parity, note, oracle, rows_per_workgroup, run, sample_rows
from streaming_video_diffusion_amd import binding as B
from streaming_video_diffusion_amd import inputs as I

pytestmark = pytest.mark.gpu


def case(name, cfg, tiles, short):
    """48 heads x ``tiles`` query tiles (the last one ``short`` rows short)
    over a ragged 2820-key context (45 key tiles)."""
    bm = rows_per_workgroup()
    return I.custom(name, cfg, "bf16", 48, 128, [1500, 1300], tiles * bm - short, prompt_rows=20)


def noalloc_vs_ws(w, out_dtype):
    ca, _ = run(w, out_dtype=out_dtype)
    need = B.sa_forward_workspace_bytes(ca.ctx, w.nq)
    note(f"  {w.name}: nq {w.nq}, tail scratch {need} bytes")
    assert 0 < need <= B.SA_NOALLOC_SCRATCH_BYTES
    got = torch.full_like(ca.out, float("nan"))
    B.sa_forward_noalloc(ca.ctx, ca.q, got, ca.q_table, w.scale)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    want = B.sa_forward_ws(ca.ctx, ca.q, ca.q_table, w.scale, out_dtype=out_dtype or ca.dtype, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(got, want), f"{w.name}: sa_forward_noalloc differs from sa_forward_ws"
    rows = sample_rows(w.nq, extra=24, seed=w.nq)
    rel, mx = assert_parity(got.float().cpu().numpy()[rows], oracle(ca, rows=rows), "bf16", w.name)
    note(f"  {w.name}: equal to sa_forward_ws; sampled rows rel-L2 {rel:.3e} max-abs {mx:.3e}")


@pytest.mark.parametrize("out_dtype", [None, torch.float32], ids=["out_bf16", "out_f32"])
def test_noalloc_two_calls_second_smaller(out_dtype):
    noalloc_vs_ws(case("noalloc_big", 610, 7, 60), out_dtype)     # 336 units: the last round holds 80
    noalloc_vs_ws(case("noalloc_small", 611, 6, 20), out_dtype)   # 288 units: the last round holds 32


def test_noalloc_without_a_tail_is_the_plain_forward():
    w = I.custom("noalloc_one_round", 612, "bf16", 8, 128, [300, 257], 700, prompt_rows=20)
    ca, _ = run(w)
    assert B.sa_forward_workspace_bytes(ca.ctx, w.nq) == 0
    got = B.sa_forward_noalloc(ca.ctx, ca.q, torch.empty_like(ca.out), ca.q_table, w.scale)
    want = B.sa_forward(ca.ctx, ca.q, ca.q_table, w.scale)
    torch.cuda.synchronize()
    assert torch.equal(got, want)


def test_noalloc_forward_captured_and_replayed():
    """The callers it is for: a forward captured into a HIP graph (after one
    eager call, which looks up the scratch's device address) and replayed,
    each replay bitwise equal to the eager result, with eager work between."""
    w = case("noalloc_graph", 613, 7, 60)
    ca, _ = run(w)
    eager = torch.empty_like(ca.out)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        B.sa_forward_noalloc(ca.ctx, ca.q, eager, ca.q_table, w.scale, stream=side)
    torch.cuda.synchronize()
    out = torch.empty_like(ca.out)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=side):
        B.sa_forward_noalloc(ca.ctx, ca.q, out, ca.q_table, w.scale, stream=side)
    torch.cuda.synchronize()
    for i in range(3):
        out.fill_(float("nan"))
        other = B.sa_forward_noalloc(ca.ctx, ca.q[: ca.q.shape[0] // 2], torch.empty_like(ca.out[: ca.q.shape[0] // 2]),
                                     ca.q_table[: ca.q.shape[0] // 2], w.scale)   # eager work on the same scratch
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), f"replay {i}"
        del other
