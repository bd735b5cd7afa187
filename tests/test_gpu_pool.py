"""Pooled history tiers produced by the pack (s x s spatial means of
full-resolution frames, then QK-norm and rotation) against the fp64 oracle:
the packed rows themselves, and attention over contexts that hold them."""

import numpy as np
import pytest
import torch

from gpu_util import assert_parity, note, oracle, run, sample_rows
from oracle import norm64, pool64, rope64
from streaming_video_diffusion_amd import binding as B
from streaming_video_diffusion_amd import inputs as I
from test_gpu_kernels import unpack_v_bf16

pytestmark = pytest.mark.gpu

AX = {64: (16, 24, 24), 128: (32, 48, 48)}


def _pack_pooled(dtype, d, heads, gh, gw, s, frames, dst, norm=None, src_view=False):
    """Pack one pooled segment at packed row ``dst`` (rows before it stay NaN
    bar the padding). Returns host (k_full, v_full, pos, weight) and the packed
    K, V rows [rows][H][d] as float64."""
    note(f"[gpu] pooled pack {dtype} d={d} H={heads} grid={gh}x{gw} s={s} frames={frames} dst={dst} norm={norm}")
    rng = np.random.default_rng(np.random.SeedSequence([I.ENTROPY, 700, s, d, gh]))
    src = frames * gh * gw
    k = rng.standard_normal((src, heads, d), dtype=np.float32)
    v = rng.standard_normal((src, heads, d), dtype=np.float32)
    if dtype == "bf16":
        k, v = I.round_bf16(k), I.round_bf16(v)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    if src_view:   # K/V as head-slices of wider fused tensors
        kb = torch.zeros((src, heads + 2, d), dtype=tdt, device="cuda")
        vb = torch.zeros((src, 2, heads, d), dtype=tdt, device="cuda")
        kb[:, 1:1 + heads] = torch.from_numpy(k).to(tdt).cuda()
        vb[:, 1] = torch.from_numpy(v).to(tdt).cuda()
        kd, vd = kb[:, 1:1 + heads], vb[:, 1]
    else:
        kd, vd = torch.from_numpy(k).to(tdt).cuda(), torch.from_numpy(v).to(tdt).cuda()
    pos = I.frame_positions(list(range(1, frames + 1)), gh, gw, pool=s)
    rows = pos.shape[0]
    table = B.sa_make_rope_tables(torch.from_numpy(pos).cuda(), d, AX[d], I.ROPE_THETA)
    weight = None
    nrm = None
    if norm is not None:
        weight = (1.0 + 0.2 * rng.standard_normal((heads, d) if norm == "per_head" else (d,))).astype(np.float32)
        nrm = B.Norm(torch.from_numpy(weight).cuda(), 1e-6)
    nk = dst + rows
    ctx = B.PackedContext(heads, d, tdt, nk, device="cuda")
    ctx.rows = nk
    ctx.k_packed.fill_(float("nan"))
    ctx.v_packed.fill_(float("nan"))
    B.sa_pack_context(ctx, [(kd, vd, dst, table, nrm, (s, gh, gw))])
    torch.cuda.synchronize()
    cap = ctx.capacity_rows
    if dtype == "bf16":
        kp = ctx.k_data().view(heads, cap, d)[:, :nk].permute(1, 0, 2).float()
        vp = unpack_v_bf16(ctx.v_data(), heads, d, cap, nk).float()
    else:
        kp = ctx.k_data().view(heads, cap, d)[:, :nk].permute(1, 0, 2)
        vp = ctx.v_data().view(heads, cap, d)[:, :nk].permute(1, 0, 2)
    kp = kp.cpu().numpy().astype(np.float64)
    vp = vp.cpu().numpy().astype(np.float64)
    assert np.isnan(kp[:dst]).all() and np.isnan(vp[:dst]).all(), "rows before the segment were written"
    return (k, v, pos, weight), kp[dst:], vp[dst:]


def _expected(k, v, pos, weight, gh, gw, s, d, rotate=True):
    kp = pool64.pool_frames(k, gh, gw, s)
    if weight is not None:
        kp = norm64.rmsnorm(kp, weight, 1e-6)
    if rotate:
        kp = rope64.rotate(kp, rope64.angles(pos, AX[d], I.ROPE_THETA))
    return kp, pool64.pool_frames(v, gh, gw, s)


POOLED = [
    # dtype, d, heads, grid_h, grid_w, s, frames, dst, norm, strided source
    ("bf16", 128, 3, 16, 24, 2, 2, 5, None, False),
    ("bf16", 128, 2, 16, 24, 4, 3, 64, "shared", False),
    ("bf16", 64, 2, 16, 24, 8, 2, 1, "per_head", True),
    ("bf16", 128, 1, 48, 84, 4, 1, 100, None, True),
    ("f32", 64, 2, 8, 12, 2, 2, 3, "per_head", False),
    ("f32", 128, 2, 8, 12, 4, 3, 0, None, True),
]


@pytest.mark.parametrize("case", POOLED, ids=[f"{c[0]}_d{c[1]}_s{c[5]}_{c[3]}x{c[4]}" for c in POOLED])
def test_pooled_pack_rows(case):
    dtype, d, heads, gh, gw, s, frames, dst, norm, view = case
    (k, v, pos, weight), kp, vp = _pack_pooled(dtype, d, heads, gh, gw, s, frames, dst, norm, view)
    # a rotate-in-forward build keeps bf16 keys unrotated in the pack
    kref, vref = _expected(k, v, pos, weight, gh, gw, s, d, rotate=not (dtype == "bf16" and B.rotates_k_in_forward()))
    if dtype == "bf16":
        # float32 mean (exact sum, power-of-two scale), float32 norm and rotation, one rounding to bf16
        assert np.all(np.abs(kp - kref) <= 2.0 ** -8 * np.abs(kref) + 2e-6)
        assert np.all(np.abs(vp - vref) <= 2.0 ** -8 * np.abs(vref) + 1e-7)
    else:
        assert np.max(np.abs(kp - kref)) <= 4e-6
        assert np.max(np.abs(vp - vref)) <= 1e-6


SMALL = [
    ("bf16", 3, 128, 16, 24, 13, None),
    ("bf16", 2, 128, 16, 24, 40, "per_head"),
    ("bf16", 2, 64, 8, 12, 0, "shared"),
    ("f32", 2, 64, 8, 12, 5, None),
]


@pytest.mark.parametrize("case", SMALL, ids=[f"{c[0]}_d{c[2]}_{c[3]}x{c[4]}_{c[6]}" for c in SMALL])
def test_attention_over_produced_tiers(case):
    dtype, heads, d, gh, gw, prompt, qkn = case
    w = I.hier_pooled(f"hier_small_{dtype}_{d}", 510 + SMALL.index(case), dtype, heads, d, gh, gw, prompt,
                      qk_norm=qkn)
    ca, out = run(w)
    rel, mx = assert_parity(out, oracle(ca), dtype, w.name)
    note(f"  {w.name}: rel-L2 {rel:.3e} max-abs {mx:.3e}")


def test_hier_pooled_full_size_sampled_rows():
    w = I.hier_pooled_1344x768()
    ca, out = run(w)
    rows = sample_rows(w.nq, seed=3)
    rel, mx = assert_parity(out[rows], oracle(ca, rows=rows), "bf16", w.name)
    note(f"  {w.name}: {len(rows)} rows, rel-L2 {rel:.3e} max-abs {mx:.3e}")
    assert np.isfinite(out).all()
