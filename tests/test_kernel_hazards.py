"""The forward kernel's gfx950 assembly holds no matrix-core hazard.

Its products are inline assembly, which the compiler's hazard recognizer does
not see, so a compiler-made copy or select placed right after a product (at a
join of two paths, a loop exit, a ragged-tile mask) would read a result that
is not written yet: wrong values that change from run to run. The test builds
the kernel's device assembly exactly as the library is built and scans every
instantiation along every control-flow path (``mfma_hazards``). Planted cases
check that the scan sees the straight-line, back-edge and join forms.
"""

import os
import subprocess

import pytest

from mfma_hazards import kernels, scan
from streaming_video_diffusion_amd import build as BLD

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "streaming_video_diffusion_amd", "csrc", "fwd_bf16.hip")


BUILDS = {"default": ((), 8),                          # head_dim 64/128 x bf16/f32 output x plain/stream-K tail
          "rotate_k_in_forward": (BLD.ROTK_FLAGS, 4)}  # head_dim 64/128 x bf16/f32 output


@pytest.mark.parametrize("build", sorted(BUILDS))
def test_every_forward_instantiation_is_clean(build, tmp_path):
    defs, n_kernels = BUILDS[build]
    out = tmp_path / "fwd_bf16.s"
    flags = [f for f in BLD.FLAGS if f not in ("-fPIC", "-shared")]
    cmd = [BLD.HIPCC, *flags, *defs, "--cuda-device-only", "-S", SRC, "-o", str(out)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    ks = {n: b for n, b in kernels(out.read_text()).items() if "fwd_bf16_kernel" in n}
    assert len(ks) == n_kernels, sorted(ks)
    for name, body in ks.items():
        assert body.count("v_mfma_f32_32x32x16_bf16") > 100, name
        assert scan(body) == [], name


def test_every_few_query_instantiation_is_clean(tmp_path):
    """The few-query kernel's products are inline assembly too (head_dim 64/128 x one/two query blocks)."""
    src = os.path.join(ROOT, "streaming_video_diffusion_amd", "csrc", "fewq.hip")
    out = tmp_path / "fewq.s"
    flags = [f for f in BLD.FLAGS if f not in ("-fPIC", "-shared")]
    r = subprocess.run([BLD.HIPCC, *flags, "--cuda-device-only", "-S", src, "-o", str(out)], capture_output=True,
                       text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    ks = {n: b for n, b in kernels(out.read_text()).items() if "fewq_kernel" in n}
    assert len(ks) == 4, sorted(ks)
    for name, body in ks.items():
        assert body.count("v_mfma_f32_32x32x16_bf16") >= 32, name
        assert scan(body) == [], name


MFMA = "v_mfma_f32_32x32x16_bf16 a[0:15], v[0:3], v[4:7], a[0:15]"


def test_scan_sees_a_read_right_after_a_product():
    body = f"\t{MFMA}\n\ts_nop 3\n\tv_accvgpr_read_b32 v8, a2\n\ts_endpgm\n"
    assert len(scan(body)) == 1
    ok = f"\t{MFMA}\n\ts_nop 7\n\ts_nop 7\n\ts_nop 3\n\tv_accvgpr_read_b32 v8, a2\n\ts_endpgm\n"
    assert scan(ok) == []


def test_scan_follows_a_loop_back_edge_and_a_join():
    back = (f".LBB0_1:\n\tv_accvgpr_write_b32 a3, v9\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7\n\t{MFMA}\n"
            "\ts_cbranch_scc1 .LBB0_1\n\ts_nop 7\n\ts_nop 7\n\ts_endpgm\n")
    assert any("touches the result" in f for f in scan(back))
    join = (f"\ts_cbranch_scc1 .LBB0_2\n\t{MFMA}\n\ts_barrier\n.LBB0_2:\n\tv_accvgpr_mov_b32 a20, a0\n"
            "\ts_endpgm\n")
    assert any("touches the result" in f for f in scan(join))


def test_scan_sees_a_valu_write_just_before_a_product():
    body = f"\tv_mov_b32_e32 v5, v9\n\t{MFMA}\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_endpgm\n"
    assert any("writes an operand" in f for f in scan(body))
    body = f"\tv_mov_b32_e32 v5, v9\n\ts_nop 1\n\t{MFMA}\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_endpgm\n"
    assert scan(body) == []
