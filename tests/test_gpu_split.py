"""Split-KV (sa_forward_split + sa_combine_splits) against the fp64 oracle:
per-run partial outputs and log-sum-exps, and the merged result."""

import dataclasses
import math

import numpy as np
import pytest
import torch

from gpu_util import assert_parity, note, oracle
from oracle import attn64
from streaming_video_diffusion_amd import binding as B
from streaming_video_diffusion_amd import inputs as I
from streaming_video_diffusion_amd.stream import ChunkAttention

pytestmark = pytest.mark.gpu

LSE_MAX_ABS = 2e-2  # same bound as the outputs: scores carry the bf16 rounding of Q' and K'


def key_ranges(nk, n_splits):
    tiles = (nk + 63) // 64
    return [(s * tiles // n_splits * 64, min((s + 1) * tiles // n_splits * 64, nk)) for s in range(n_splits)]


def packed(w, call=0):
    ca = ChunkAttention(w, call=call)
    note(f"[gpu] split-KV {w.name} nq={w.nq} nk={w.nk} H={w.heads} d={w.head_dim} {w.dtype}")
    ca.pack_static()
    ca._tables(True, None)
    ca._pack(True, None)
    return ca


def split_oracle(ca, ranges, rows=None):
    q, q_pos, segs = ca.host_inputs()
    qn, kn = ca.host_norms()
    w = ca.w
    return attn64.chunk_split_attention(q, q_pos, segs, w.axis_dims, w.theta, w.scale, ranges, rows=rows,
                                        q_norm=qn, k_norm=kn)


def check(ca, n_splits, dtype, rows=None, q=None, q_table=None):
    w = ca.w
    q = ca.q if q is None else q
    q_table = ca.q_table if q_table is None else q_table
    partial, lse = B.sa_forward_split(ca.ctx, q, n_splits, q_table, w.scale, q_norm=ca.q_norm)
    out = B.sa_combine_splits(partial, lse, out_dtype=torch.float32)
    torch.cuda.synchronize()
    ranges = key_ranges(w.nk, n_splits)
    p_ref, l_ref = split_oracle(ca, ranges, rows=rows)
    got_p = partial.cpu().numpy().astype(np.float64)
    got_l = lse.cpu().numpy().astype(np.float64)
    assert_parity(got_p, p_ref, dtype, f"{w.name} partial x{n_splits}")
    lerr = float(np.max(np.abs(got_l - l_ref)))
    assert lerr <= (LSE_MAX_ABS if dtype == "bf16" else 1e-4), f"lse max abs err {lerr:.3e}"
    ref = oracle(ca, rows=rows)
    rel, mx = assert_parity(out.cpu().numpy().astype(np.float64), ref, dtype, f"{w.name} merged x{n_splits}")
    note(f"  x{n_splits}: merged rel-L2 {rel:.3e} max-abs {mx:.3e}, lse max abs err {lerr:.2e}")
    return partial, lse, out


@pytest.mark.parametrize("n_splits", [1, 5, 29])
def test_split_lowres(n_splits):
    w = I.lowres_bf16()           # 1828 keys = 29 tiles (ragged last)
    check(packed(w), n_splits, "bf16")


def test_one_split_is_the_forward_bitwise():
    w = I.lowres_bf16()
    ca = packed(w)
    partial, lse = B.sa_forward_split(ca.ctx, ca.q, 1, ca.q_table, w.scale)
    out = B.sa_forward(ca.ctx, ca.q, ca.q_table, w.scale, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(partial[0], out)


def test_split_f32():
    w = I.tiny_f32()               # 304 keys = 5 tiles
    check(packed(w), 3, "f32")


def test_split_second_pass():
    """Peaked scores (exact on the GPU: unrotated, power-of-two pre-scale) leave the main pass."""
    w = I.custom("split_peaked", 420, "bf16", 3, 128, [150, 333], 300, rotary=False, prompt_rows=40,
                 scale=float(np.float32(4.0 * math.log(2.0))))
    check(packed(w), 4, "bf16")


def test_split_with_qknorm():
    w = dataclasses.replace(I.custom("split_qkn", 421, "bf16", 2, 128, [200, 500], 260, prompt_rows=9),
                            qk_norm="per_head")
    check(packed(w), 6, "bf16")


@pytest.mark.parametrize("n_splits", [1, 5, 29])
def test_split_few_rows(n_splits):
    """40 query rows (bf16) of 128 heads: 5 and 29 runs per head (at least
    twice as many runs as a 256-CU part has CUs) take one wave of the few-query
    kernel each, 1 run the forward kernel; 1828 keys = 29 tiles, ragged last,
    so 29 runs hold one tile each."""
    w = I.custom("split_few", 422, "bf16", 128, 128, [1200, 605], 40, prompt_rows=23)
    assert w.nk == 1828 and w.nq <= B.SA_FEW_QUERY_ROWS
    check(packed(w), n_splits, "bf16")


def test_split_few_rows_d64_qknorm_and_second_pass():
    w = dataclasses.replace(I.custom("split_few_d64", 423, "bf16", 96, 64, [700, 333], 17, prompt_rows=9),
                            qk_norm="per_head")
    check(packed(w), 6, "bf16")
    w = I.custom("split_few_peaked", 424, "bf16", 128, 128, [150, 333], 40, rotary=False, prompt_rows=40,
                 scale=float(np.float32(4.0 * math.log(2.0))))
    check(packed(w), 4, "bf16")


def test_audio_only_queries_full_size():
    """The 40 audio queries of the 1 s video+audio chunk (24232 q x 52752 kv), 32 key runs."""
    w = I.video_audio_1344x768()
    ca = packed(w)
    rows = np.arange(w.nq - 40, w.nq)
    q = ca.q[w.nq - 40:]
    qt = ca.q_table[w.nq - 40:]
    check(ca, 32, "bf16", rows=rows, q=q, q_table=qt)
