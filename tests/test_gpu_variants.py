"""Query-side variants of the same forward kernel against the fp64 oracle on
sampled rows: recomputed history + current chunk as queries, the seven-frame
first window, and the prefix's self-attention pass (1344x768 shapes)."""

import numpy as np
import pytest
import torch

from gpu_util import assert_parity, note, oracle, run, sample_rows
from streaming_video_diffusion_amd import inputs as I

pytestmark = pytest.mark.gpu

VARIANTS = list(I.VARIANTS.values())


@pytest.mark.parametrize("make", VARIANTS, ids=[f.__name__ for f in VARIANTS])
def test_variant_sampled_rows(make):
    w = make()
    ca, out = run(w)
    rows = sample_rows(w.nq, seed=7)
    ref = oracle(ca, rows=rows)
    rel, mx = assert_parity(out[rows], ref, "bf16", w.name)
    note(f"  {w.name}: {len(rows)} rows, rel-L2 {rel:.3e} max-abs {mx:.3e}")
    assert np.isfinite(out).all()
    del ca
    torch.cuda.empty_cache()
