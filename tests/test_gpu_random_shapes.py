"""Seeded random shapes against the fp64 oracle: heads, head dim, dtype,
segment sizes (empty, single rows, tile edges), prompt rows, query counts
around the 32/64/96/384-row block, tile, wave and workgroup edges, QK-norm and output dtype drawn per case;
each case through the chunk sequence and through split-KV plus the merge."""

import numpy as np
import pytest
import torch

from gpu_util import assert_parity, note, oracle, run
from streaming_video_diffusion_amd import binding as B
from streaming_video_diffusion_amd import inputs as I

pytestmark = pytest.mark.gpu

N_CASES = 16
ROWS = [0, 1, 17, 63, 64, 65, 100, 129, 200, 333]
NQ = [1, 31, 32, 63, 65, 95, 97, 255, 257, 383, 385, 400]


def draw(i):
    rng = np.random.default_rng(np.random.SeedSequence([0x5EED, 77, i]))
    dtype = "f32" if rng.random() < 0.25 else "bf16"
    heads = int(rng.choice([1, 2, 3, 5]))
    d = int(rng.choice([64, 128]))
    seg_rows = [int(x) for x in rng.choice(ROWS, size=int(rng.integers(1, 5)))]
    prompt = int(rng.choice([0, 5, 16]))
    if prompt + sum(seg_rows) == 0:
        seg_rows[0] = 17
    nq = int(rng.choice(NQ))
    qk = [None, "shared", "per_head"][int(rng.integers(0, 3))]
    out = None if rng.random() < 0.7 else (torch.float32 if dtype == "bf16" else None)
    n_splits = int(rng.integers(2, 6))
    w = I.custom(f"rand{i}", 700 + i, dtype, heads, d, seg_rows, nq, prompt_rows=prompt, qk_norm=qk)
    return w, out, n_splits


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_shape_matches_oracle(i):
    w, out_dtype, n_splits = draw(i)
    note(f"[gpu] random case {i}: {w.dtype} H={w.heads} d={w.head_dim} nq={w.nq} nk={w.nk} "
         f"segs={[s.rows for s in w.segments]} qk_norm={w.qk_norm} out={out_dtype} splits={n_splits}")
    ca, out = run(w, out_dtype=out_dtype)
    ref = oracle(ca)
    # a bf16 run with a float32 output is held to the bf16 bound (its inputs are bf16)
    assert_parity(out, ref, w.dtype, f"case {i}")
    ntiles = (w.nk + 63) // 64
    n = min(n_splits, ntiles)
    partial, lse = B.sa_forward_split(ca.ctx, ca.q, n, ca.q_table, w.scale, q_norm=ca.q_norm)
    merged = B.sa_combine_splits(partial, lse, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert_parity(merged.cpu().numpy().astype(np.float64), ref, w.dtype, f"case {i}, {n} key runs")
