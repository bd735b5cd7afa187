"""The largest packed context the ABI accepts, against a closed form.

One head's packed K (or V) must stay below 2^31 bytes: 8388544 rows at head
dim 128 in bf16 is the largest capacity, one 64-row tile below the limit.
With two heads every in-head offset uses 31 bits and the second head starts
past 2^31 bytes. The fp64 oracle cannot hold such a context, so the keys are
built so the result has a closed form: a small random segment, then
millions of keys that are exactly zero (score 0, weight exactly 1 in the
softmax) each with its own random value, so for every query row

    out = (sum_small e^{s_j} v_j + sum_big v_j) / (sum_small e^{s_j} + N_big),

computed here in float64 from the same seeded values."""

import numpy as np
import pytest
import torch

from gpu_util import assert_parity, note
from streaming_video_diffusion_amd import binding as B

pytestmark = pytest.mark.gpu

CAP = (1 << 31) // 256 - 64   # rows: one head's bf16 K at d 128 just below 2^31 bytes


def test_max_capacity_context():
    heads, d, nq, small = 2, 128, 40, 96
    big = CAP - small
    note(f"[gpu] max capacity: {heads} heads x {CAP} rows (one head's K {CAP * d * 2} bytes)")
    gen = torch.Generator(device="cuda").manual_seed(20261203)
    ctx = B.PackedContext(heads, d, torch.bfloat16, CAP)
    ctx.rows = CAP
    q = torch.randn((nq, heads, d), generator=gen, device="cuda").to(torch.bfloat16)
    ks = torch.randn((small, heads, d), generator=gen, device="cuda").to(torch.bfloat16)
    vs = torch.randn((small, heads, d), generator=gen, device="cuda").to(torch.bfloat16)
    kb = torch.zeros((big, heads, d), dtype=torch.bfloat16, device="cuda")
    vb = torch.randn((big, heads, d), generator=gen, device="cuda").to(torch.bfloat16)
    B.sa_pack_context(ctx, [(ks, vs, 0, None), (kb, vb, small, None)])
    scale = d ** -0.5
    out = B.sa_forward(ctx, q, None, scale, out_dtype=torch.float32)
    torch.cuda.synchronize()
    # closed form in float64
    big_sum = torch.zeros((heads, d), dtype=torch.float64)
    for a in range(0, big, 1 << 20):
        big_sum += vb[a:a + (1 << 20)].double().sum(dim=0).cpu()
    qh, kh, vh = (x.double().cpu() for x in (q, ks, vs))
    s = scale * torch.einsum("nhd,jhd->nhj", qh, kh)          # [nq][heads][small]
    m = s.amax(dim=-1, keepdim=True).clamp(min=0.0)            # the big keys score 0
    e = torch.exp(s - m)
    num = torch.einsum("nhj,jhd->nhd", e, vh) + torch.exp(-m) * big_sum[None]
    den = e.sum(dim=-1, keepdim=True) + big * torch.exp(-m)
    ref = (num / den).numpy()
    rel, mx = assert_parity(out.cpu().numpy().astype(np.float64), ref, "bf16", "max capacity")
    note(f"  rel-L2 {rel:.3e} max-abs {mx:.3e}")
    del ctx, kb, vb
    torch.cuda.empty_cache()
