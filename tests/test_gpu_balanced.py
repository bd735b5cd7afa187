"""The stream-K tail of the forward (sa_forward_ws): the units of a last round
that would leave at least a quarter of the CUs idle are spread over all CUs
as equal contiguous ranges of their key tiles, the units a range boundary
cuts merged by their log-sum-exps. Checked against the fp64 oracle and
against the plain forward, which every unit computed whole must match bit
for bit."""

import math

import numpy as np
import pytest
import torch

from gpu_util import assert_parity, note, oracle, rows_per_workgroup, run, sample_rows
from streaming_video_diffusion_amd import binding as B
from streaming_video_diffusion_amd import inputs as I

pytestmark = pytest.mark.gpu


def plan(nq, heads, nk):
    """(units in the tail, first tail unit, key tiles per unit) as the library
    plans them on this GPU."""
    n_cu = torch.cuda.get_device_properties(0).multi_processor_count
    units = math.ceil(nq / rows_per_workgroup()) * heads
    rounds = math.ceil(units / n_cu)
    r = units - (rounds - 1) * n_cu
    ntiles = math.ceil(nk / 64)
    if 4 * r > 3 * n_cu or r * ntiles < 4 * n_cu:
        return 0, units, ntiles
    return r, units - r, ntiles


def whole_units(units, first_unit, ntiles):
    """Tail units (counted from first_unit) that one workgroup's range holds
    whole: computed exactly as by the plain forward."""
    n_cu = torch.cuda.get_device_properties(0).multi_processor_count
    total = units * ntiles
    wg = lambda x: ((x + 1) * n_cu - 1) // total  # noqa: E731
    return [first_unit + u for u in range(units) if wg(u * ntiles) == wg((u + 1) * ntiles - 1)]


def unit_mask(nq, heads, units):
    """[nq][heads] True where the (row, head) belongs to one of ``units``."""
    BM = rows_per_workgroup()
    n_qt = math.ceil(nq / BM)
    m = np.zeros((nq, heads), dtype=bool)
    for u in units:
        h, qt = divmod(u, n_qt)
        m[qt * BM:min((qt + 1) * BM, nq), h] = True
    return m


def balanced_case():
    n_cu = torch.cuda.get_device_properties(0).multi_processor_count
    heads = n_cu // 8            # 9 query tiles x n_cu/8 heads = n_cu + n_cu/8 units: a tail of n_cu/8
    return I.custom("balanced", 600, "bf16", heads, 128, [1500, 1300], 9 * rows_per_workgroup() - 100,
                    prompt_rows=20)


def shard_case():
    """One GPU's share of an 8-way head split of the 1344x768 chunk: 5 heads, 160 units on 256 CUs."""
    import dataclasses
    return dataclasses.replace(I.full_1344x768(), name="full_1344x768_h5", heads=5)


def test_workspace_bytes_follow_the_rounds():
    n_cu = torch.cuda.get_device_properties(0).multi_processor_count
    for w in (I.full_1344x768(), I.lowres_bf16(), balanced_case(), shard_case(), I.first_window_1344x768()):
        ctx = B.PackedContext(w.heads, w.head_dim, torch.bfloat16, w.nk)
        ctx.rows = w.nk
        r, _, _ = plan(w.nq, w.heads, w.nk)
        want = 2 * n_cu * rows_per_workgroup() * (w.head_dim + 1) * 4 if r else 0
        assert B.sa_forward_workspace_bytes(ctx, w.nq) == want, w.name
    assert plan(shard_case().nq, 5, shard_case().nk)[0] == 160
    assert plan(I.full_1344x768().nq, 40, I.full_1344x768().nk)[0] == 0   # 1280 units: five full rounds


@pytest.mark.parametrize("out_dtype", [None, torch.float32], ids=["out_bf16", "out_f32"])
def test_tail_small_full(out_dtype):
    w = balanced_case()
    r, first, ntiles = plan(w.nq, w.heads, w.nk)
    assert r > 0
    ca, out = run(w, out_dtype=out_dtype)
    assert ca.workspace is not None
    rel, mx = assert_parity(out, oracle(ca), "bf16", w.name)
    note(f"  {w.name}: tail of {r} units x {ntiles} tiles, rel-L2 {rel:.3e} max-abs {mx:.3e}")
    plain = B.sa_forward(ca.ctx, ca.q, ca.q_table, w.scale, out_dtype=ca.out_dtype)
    torch.cuda.synchronize()
    same = list(range(first)) + whole_units(r, first, ntiles)
    keep = torch.from_numpy(unit_mask(w.nq, w.heads, same)).cuda()
    assert torch.equal(plain[keep], ca.out[keep]), "units computed whole must match the plain forward"


def test_tail_d64_qknorm():
    """The tail at head_dim 64 with per-head QK-norm: 3 query tiles x 96 heads = 288 units (a last round of 32)."""
    import dataclasses
    w = dataclasses.replace(I.custom("tail_d64_qkn", 601, "bf16", 96, 64, [1700, 1400], 3 * rows_per_workgroup() - 7,
                                     prompt_rows=33), qk_norm="per_head")
    r, first, ntiles = plan(w.nq, w.heads, w.nk)
    assert r > 0
    ca, out = run(w)
    assert ca.workspace is not None
    rows = sample_rows(w.nq, extra=24, seed=3)
    rel, mx = assert_parity(out[rows], oracle(ca, rows=rows), "bf16", w.name)
    note(f"  {w.name}: tail of {r} units x {ntiles} tiles, rel-L2 {rel:.3e} max-abs {mx:.3e}")
    plain = B.sa_forward(ca.ctx, ca.q, ca.q_table, w.scale, q_norm=ca.q_norm).float().cpu().numpy()
    torch.cuda.synchronize()
    m = unit_mask(w.nq, w.heads, list(range(first)) + whole_units(r, first, ntiles))
    assert np.array_equal(plain[m], out[m])


def test_tail_strided_output_view():
    """The tail's merge writes through the caller's row and head strides: a
    view into a wider buffer gets exactly the contiguous result, and nothing
    outside the view changes."""
    w = balanced_case()
    ca, _ = run(w)
    want = ca.out.clone()
    big = torch.full((w.nq, w.heads + 3, w.head_dim + 64), 7.0, dtype=torch.bfloat16, device="cuda")
    view = big[:, 1:1 + w.heads, 32:32 + w.head_dim]
    B.sa_forward_ws(ca.ctx, ca.q, ca.q_table, w.scale, out=view, workspace=ca.workspace)
    torch.cuda.synchronize()
    assert torch.equal(view, want)
    outside = torch.ones_like(big, dtype=torch.bool)
    outside[:, 1:1 + w.heads, 32:32 + w.head_dim] = False
    assert bool((big[outside] == 7.0).all())


def test_tail_few_query_rows():
    """150 heads of SA_FEW_QUERY_ROWS + 1 query rows (one more than the
    few-query path takes): every unit holds 65 valid rows (the rest of its 384
    are padding the merge must skip), all in the tail."""
    w = I.custom("tail_few_rows", 602, "bf16", 150, 128, [1700, 1300], B.SA_FEW_QUERY_ROWS + 1, prompt_rows=11)
    r, first, ntiles = plan(w.nq, w.heads, w.nk)
    assert (r, first) == (150, 0)
    ca, out = run(w)
    assert ca.workspace is not None
    rel, mx = assert_parity(out, oracle(ca), "bf16", w.name)
    note(f"  {w.name}: rel-L2 {rel:.3e} max-abs {mx:.3e}")
    plain = B.sa_forward(ca.ctx, ca.q, ca.q_table, w.scale).float().cpu().numpy()
    torch.cuda.synchronize()
    m = unit_mask(w.nq, w.heads, whole_units(r, first, ntiles))
    assert np.array_equal(plain[m], out[m])


def test_no_workspace_is_the_plain_forward():
    w = balanced_case()
    ca, _ = run(w)
    a = B.sa_forward_ws(ca.ctx, ca.q, ca.q_table, w.scale, workspace=None)
    b = B.sa_forward(ca.ctx, ca.q, ca.q_table, w.scale)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_small_workspace_is_rejected():
    w = balanced_case()
    ca, _ = run(w)
    need = B.sa_forward_workspace_bytes(ca.ctx, w.nq)
    small = torch.empty(need - 16, dtype=torch.uint8, device="cuda")
    with pytest.raises(B.SaError) as e:
        B.sa_forward_ws(ca.ctx, ca.q, ca.q_table, w.scale, workspace=small)
    assert e.value.status == -5


def test_tail_head_shard_full_size():
    """5 heads of the 1344x768 chunk: all 160 units go through the tail (no whole rounds)."""
    w = shard_case()
    r, first, ntiles = plan(w.nq, w.heads, w.nk)
    assert (r, first) == (160, 0)
    ca, out = run(w)
    rows = sample_rows(w.nq, extra=24, seed=12)
    rel, mx = assert_parity(out[rows], oracle(ca, rows=rows), "bf16", w.name)
    note(f"  {w.name}: rel-L2 {rel:.3e} max-abs {mx:.3e}")
    plain = B.sa_forward(ca.ctx, ca.q, ca.q_table, w.scale).float().cpu().numpy()
    torch.cuda.synchronize()
    whole = whole_units(r, first, ntiles)
    note(f"  {len(whole)} of {r} units whole")
    m = unit_mask(w.nq, w.heads, whole)
    assert np.array_equal(plain[m], out[m])
    cut = ~m
    rel2 = np.linalg.norm(plain[cut] - out[cut]) / np.linalg.norm(plain[cut])
    assert rel2 < 5e-3, rel2


def test_tail_first_window_sampled_rows():
    """The 7-frame first window: 2960 units, a last round of 144 spread over every CU."""
    w = I.first_window_1344x768()
    r, first, ntiles = plan(w.nq, w.heads, w.nk)
    ca, out = run(w)
    note(f"  tail of {r} units from unit {first}")
    rows = sample_rows(w.nq, seed=11)
    rel, mx = assert_parity(out[rows], oracle(ca, rows=rows), "bf16", w.name)
    note(f"  rel-L2 {rel:.3e} max-abs {mx:.3e}")
    if r:
        plain = B.sa_forward(ca.ctx, ca.q, ca.q_table, w.scale).float().cpu().numpy()
        torch.cuda.synchronize()
        m = unit_mask(w.nq, w.heads, list(range(first)) + whole_units(r, first, ntiles))
        assert np.array_equal(plain[m], out[m])
