"""The rotate-in-forward build (keys stored unrotated with per-row tables,
rotated in the forward's key-tile load) against the fp64 oracle, loaded next
to the default library in the same process."""

import os

import pytest

from gpu_util import assert_parity, note, oracle, run, sample_rows
from streaming_video_diffusion_amd import binding as B
from streaming_video_diffusion_amd import build
from streaming_video_diffusion_amd import inputs as I

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def variant():
    if not os.path.exists(build.ROTK_LIB):
        pytest.skip("the rotate-in-forward library is not built (__graft_entry__.build() builds it)")
    saved = B.lib()
    B._lib = B.load(build.ROTK_LIB)
    try:
        assert B.rotates_k_in_forward()
        yield
    finally:
        B._lib = saved


CASES = [
    I.lowres_bf16,
    lambda: I.custom("rotk_ragged_d64", 801, "bf16", 3, 64, [17, 100, 333], 300, prompt_rows=5),
    lambda: I.custom("rotk_ragged_qknorm", 802, "bf16", 2, 128, [1, 64, 65, 129], 257, prompt_rows=16,
                     qk_norm="per_head"),
]


@pytest.mark.parametrize("make", CASES, ids=["lowres", "ragged_d64", "ragged_qknorm"])
def test_variant_matches_oracle(variant, make):
    w = make()
    note(f"[gpu] rotate-in-forward build: {w.name}")
    ca, out = run(w)
    assert_parity(out, oracle(ca), w.dtype, w.name)


def test_variant_full_size_sampled_rows(variant):
    w = I.full_1344x768()
    note("[gpu] rotate-in-forward build: full_1344x768 sampled rows")
    ca, out = run(w)
    rows = sample_rows(w.nq)
    assert_parity(out[rows], oracle(ca, rows=rows), "bf16", "full_1344x768 (rotate-in-forward)")


# The default build's tests of the rarer paths, run again with the variant
# loaded: peaked scores and underflowing rows take the second pass (which
# reloads every tile and rotates it again), and split-KV stores per-run
# partial outputs and log-sum-exps.
import test_gpu_parity as P  # noqa: E402
import test_gpu_split as S  # noqa: E402


@pytest.mark.parametrize("c_log2", [0.5, 4.0], ids=["scale_x0.5", "scale_x4"])
def test_variant_peaked_scores(variant, c_log2):
    note(f"[gpu] rotate-in-forward build: peaked scores x{c_log2}")
    P.test_rescaling_path_large_scores(c_log2)


def test_variant_underflowing_rows(variant):
    note("[gpu] rotate-in-forward build: underflowing rows")
    P.test_second_pass_underflowing_rows()


def test_variant_mixed_rows_keep_neighbours_bitwise(variant):
    note("[gpu] rotate-in-forward build: mixed rows")
    P.test_second_pass_mixed_rows_keep_neighbours_bitwise()


@pytest.mark.parametrize("n_splits", [1, 5, 29])
def test_variant_split_kv(variant, n_splits):
    note(f"[gpu] rotate-in-forward build: split-KV x{n_splits}")
    S.test_split_lowres(n_splits)


def test_variant_split_second_pass(variant):
    note("[gpu] rotate-in-forward build: split-KV with peaked scores")
    S.test_split_second_pass()
