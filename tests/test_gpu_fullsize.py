"""The whole output at 1344x768 against the fp64 oracle.

The other full-size tests compare sampled rows (each exact, since rows are
independent); these compare every one of the Nq x 40 x 128 outputs of the
1344x768 chunk and of the hierarchical-history chunk, in the launch
configuration the benchmark times (sa_forward_ws). The oracle runs in
float64 on the host cores, about a minute per workload.
"""

import time

import numpy as np
import pytest
import torch

from gpu_util import assert_parity, note, oracle, run
from streaming_video_diffusion_amd import inputs as I

pytestmark = [pytest.mark.gpu, pytest.mark.slow]


@pytest.mark.parametrize("make", [I.full_1344x768, I.hier_1344x768], ids=["full_1344x768", "hier_1344x768"])
def test_whole_output(make):
    w = make()
    ca, out = run(w)
    t0 = time.time()
    ref = oracle(ca)
    note(f"  oracle over all {w.nq} rows x {w.heads} heads in {time.time() - t0:.1f} s")
    assert np.isfinite(out).all()
    rel, mx = assert_parity(out, ref, "bf16", w.name)
    note(f"  {w.name}: every output, rel-L2 {rel:.3e} max-abs {mx:.3e}")
    del ca
    torch.cuda.empty_cache()
