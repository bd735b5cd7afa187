"""QK-norm fused into the pack (keys) and the forward query load, against the
fp64 oracle (per-head RMS normalisation before the rotation)."""

import dataclasses

import numpy as np
import pytest
import torch

from gpu_util import assert_parity, note, oracle, run, sample_rows
from streaming_video_diffusion_amd import binding as B
from streaming_video_diffusion_amd import inputs as I

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("out_dtype", [None, torch.float32], ids=["out_bf16", "out_f32"])
def test_lowres_shared_norm_full(out_dtype):
    w = dataclasses.replace(I.lowres_bf16(), name="lowres_qknorm", qk_norm="shared")
    ca, out = run(w, out_dtype=out_dtype)
    rel, mx = assert_parity(out, oracle(ca), "bf16", w.name)
    note(f"  rel-L2 {rel:.3e} max-abs {mx:.3e}")


CASES = [
    # name, dtype, heads, head_dim, seg_rows, nq, prompt, norm
    ("qkn_bf16_d128_perhead", "bf16", 3, 128, [17, 100, 333], 300, 5, "per_head"),
    ("qkn_bf16_d64_shared", "bf16", 2, 64, [70, 1, 190], 257, 0, "shared"),
    ("qkn_f32_d128_perhead", "f32", 2, 128, [33, 70], 130, 4, "per_head"),
    ("qkn_f32_d64_shared", "f32", 3, 64, [1, 45], 65, 3, "shared"),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_qknorm_shapes(case):
    name, dtype, heads, d, rows, nq, prompt, norm = case
    w = I.custom(name, 500 + CASES.index(case), dtype, heads, d, rows, nq, prompt_rows=prompt, qk_norm=norm)
    ca, out = run(w)
    rel, mx = assert_parity(out, oracle(ca), dtype, name)
    note(f"  rel-L2 {rel:.3e} max-abs {mx:.3e}")


def test_unweighted_norm():
    """weight NULL means all ones."""
    from oracle import attn64
    from streaming_video_diffusion_amd.stream import ChunkAttention
    w = I.custom("qkn_noweight", 510, "bf16", 2, 128, [64, 200], 150, prompt_rows=6)
    ca = ChunkAttention(w)
    ca.q_norm = B.Norm(None, 1e-5)
    ca.k_norm = B.Norm(None, 1e-5)
    note("[gpu] unweighted QK-norm")
    ca.pack_static()
    out = ca.step().float().cpu().numpy().astype(np.float64)
    torch.cuda.synchronize()
    q, q_pos, segs = ca.host_inputs()
    ref = attn64.chunk_attention(q, q_pos, segs, w.axis_dims, w.theta, w.scale, q_norm=(None, 1e-5),
                                 k_norm=(None, 1e-5))
    assert_parity(out, ref, "bf16", "unweighted QK-norm")


def test_norm_makes_input_scale_irrelevant():
    """eps = 0: scaling Q and K by 64 (exact in bf16) leaves the output bit for bit unchanged."""
    from streaming_video_diffusion_amd.stream import ChunkAttention
    w = dataclasses.replace(I.custom("qkn_scale", 511, "bf16", 2, 128, [64, 200], 150, prompt_rows=6,
                                     qk_norm="shared"), norm_eps=0.0)
    ca = ChunkAttention(w)
    note("[gpu] QK-norm scale invariance")
    ca.pack_static()
    a = ca.step().clone()
    ca.q.mul_(64.0)
    for s in ca.segs:
        s["k"].mul_(64.0)
    ca.pack_static()
    b = ca.step()
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_full_size_qknorm_sampled_rows():
    w = dataclasses.replace(I.full_1344x768(), name="full_1344x768_qknorm", qk_norm="shared")
    ca, out = run(w)
    rows = sample_rows(w.nq, seed=3)
    rel, mx = assert_parity(out[rows], oracle(ca, rows=rows), "bf16", w.name)
    note(f"  {w.name}: {len(rows)} rows, rel-L2 {rel:.3e} max-abs {mx:.3e}")
    assert np.isfinite(out).all()
