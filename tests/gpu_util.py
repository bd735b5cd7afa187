"""Helpers for the GPU tests: run a workload through libstreamattn and compare
with the fp64 oracle on the same seeded host values."""

import sys

import numpy as np
import torch

from oracle import attn64, pool64
from streaming_video_diffusion_amd.stream import ChunkAttention

# Parity bounds against the fp64 oracle.
BF16_REL_L2 = 5e-3
BF16_MAX_ABS = 2e-2
F32_REL_L2 = 1e-5


def note(msg):
    """Print and flush what names the case before a GPU step."""
    print(msg, file=sys.stderr, flush=True)


def errors(got, ref):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    rel = float(np.linalg.norm(got - ref) / np.linalg.norm(ref))
    mx = float(np.max(np.abs(got - ref)))
    return rel, mx


def assert_parity(got, ref, dtype, what=""):
    rel, mx = errors(got, ref)
    if dtype == "bf16":
        assert rel <= BF16_REL_L2 and mx <= BF16_MAX_ABS, f"{what}: rel-L2 {rel:.3e}, max-abs {mx:.3e}"
    else:
        assert rel <= F32_REL_L2, f"{what}: rel-L2 {rel:.3e}"
    return rel, mx


def sample_rows(nq, extra=48, seed=0):
    """Rows that cross the 32-row query blocks, 64-row key tiles, 96-row wave
    and 384-row workgroup edges, the ragged tail, plus random ones."""
    edges = []
    for b in (32, 64, 96, 384):
        for k in range(1, nq // b + 1):
            for r in (k * b - 1, k * b):
                if 0 <= r < nq:
                    edges.append(r)
    edges = sorted(set(edges))
    rng = np.random.default_rng(seed)
    pick = set([0, nq - 1] + list(rng.choice(edges, size=min(len(edges), 32), replace=False)))
    pick |= set(rng.integers(0, nq, size=extra).tolist())
    pick |= set(range(max(0, nq - 5), nq))
    return np.array(sorted(pick), dtype=np.int64)


def run(workload, call=0, out_dtype=None):
    """Pack static + one step on the GPU. Returns (ChunkAttention, out as float64 numpy)."""
    note(f"[gpu] {workload.name} call {call} nq={workload.nq} nk={workload.nk} H={workload.heads} "
         f"d={workload.head_dim} dtype={workload.dtype} out={out_dtype}")
    ca = ChunkAttention(workload, call=call, out_dtype=out_dtype)
    ca.pack_static()
    out = ca.step()
    torch.cuda.synchronize()
    return ca, out.float().cpu().numpy().astype(np.float64)


def attention_segments(segs):
    """Segments as attention sees them: a pooled segment's full-resolution
    frames pooled by the oracle."""
    out = []
    for seg in segs:
        if len(seg) == 4:
            k, v, pos, (gh, gw, s) = seg
            seg = (pool64.pool_frames(k, gh, gw, s), pool64.pool_frames(v, gh, gw, s), pos)
        out.append(seg)
    return out


def oracle(ca, rows=None):
    q, q_pos, segs = ca.host_inputs()
    qn, kn = ca.host_norms()
    w = ca.w
    return attn64.chunk_attention(q, q_pos, attention_segments(segs), w.axis_dims, w.theta, w.scale, rows=rows,
                                  q_norm=qn, k_norm=kn)


def rows_per_workgroup():
    """Query rows per (head, query tile) unit of the bf16 forward, read off the
    workspace the library asks for: n_cu / 2 heads of SA_FEW_QUERY_ROWS + 1
    query rows (one more than the few-query path takes) over 16 key tiles make
    one part-empty round of n_cu / 2 units, which the stream-K tail spreads over
    every CU, with 2 * n_cu slots of rows * (head_dim + 1) floats."""
    import torch
    from streaming_video_diffusion_amd import binding as B
    n_cu = torch.cuda.get_device_properties(0).multi_processor_count
    ctx = B.PackedContext(n_cu // 2, 128, torch.bfloat16, 1024, device="cuda")
    ctx.rows = 1024
    return B.sa_forward_workspace_bytes(ctx, B.SA_FEW_QUERY_ROWS + 1) // (2 * n_cu * 129 * 4)