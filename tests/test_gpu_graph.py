"""The per-chunk sequence captured once into a HIP graph and replayed.

The library's calls allocate nothing, never synchronise and take the stream
from the caller, so a chunk (rotary tables of the template, in-place pack of
the dynamic rows, forward with the stream-K tail where it applies) can be captured and
replayed, as the pages do for their fixed shapes (StreamRender-H3 page,
inference-acceleration section). Every replay, with eager work and
synchronisation between replays, must give the eager result bit for bit.
"""

import pytest
import torch

from gpu_util import note
from streaming_video_diffusion_amd import inputs as I
from streaming_video_diffusion_amd.stream import ChunkAttention

pytestmark = pytest.mark.gpu


def _shard():
    """One GPU's 5-head share of the 1344x768 chunk: its forward runs the stream-K tail."""
    import dataclasses
    return dataclasses.replace(I.full_1344x768(), name="full_1344x768_h5", heads=5)


@pytest.mark.parametrize("name", ["lowres_bf16", "full_1344x768", "full_1344x768_h5"])
def test_captured_chunk_replays_match_eager(name):
    note(f"[gpu] graph capture {name}")
    w = _shard() if name == "full_1344x768_h5" else I.CONFIGS[name]()
    ca = ChunkAttention(w)
    if name == "full_1344x768_h5":
        assert ca.workspace is not None, "the shard's forward should take the stream-K tail"
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        ca.pack_static(side)
        ca.step(side)  # eager run on the capture stream
    torch.cuda.synchronize()
    ref = ca.out.clone()
    k_ref, v_ref = ca.ctx.k_data().clone(), ca.ctx.v_data().clone()

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=side):
        ca.step(side)
    torch.cuda.synchronize()
    for i in range(3):
        # eager work between replays: clobber the outputs and the dynamic rows
        ca.out.fill_(float("nan"))
        n_static = sum(s.rows for s in w.segments if not s.dynamic)
        kv = ca.ctx.k_data().view(w.heads, ca.ctx.capacity_rows, w.head_dim)
        kv[:, n_static:w.nk].zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(ca.out, ref), f"replay {i}: output differs from the eager run"
        assert torch.equal(ca.ctx.k_data(), k_ref) and torch.equal(ca.ctx.v_data(), v_ref), f"replay {i}: packed K/V"
