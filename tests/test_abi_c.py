"""The C ABI from a plain C program (no C++, no torch): the header compiles as
C11 with the host compiler, the program links against the in-tree library and
runs the calls that need no GPU (version, sizes, status strings, an argument
error with its message)."""

import os
import shutil
import subprocess

import pytest

from streaming_video_diffusion_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")

PROGRAM = r"""
#include <stdio.h>
#include "streamattn.h"

int main(void) {
    size_t bytes = 0;
    if (sa_abi_version() != SA_ABI_VERSION) return 1;
    if (sa_packed_bytes(40, 128, SA_BF16, 28480, &bytes) != SA_OK) return 2;
    sa_status st = sa_forward(NULL, NULL, 0, 0, 0, NULL, NULL, 1.0f, NULL, SA_BF16, 0, 0, (hipStream_t)0);
    printf("%d %zu %s %d %s\n", sa_abi_version(), bytes, sa_status_string(SA_ERR_NULL), (int)st, sa_last_error());
    return st == SA_ERR_NULL ? 0 : 3;
}
"""


@pytest.mark.skipif(shutil.which("gcc") is None or not os.path.isdir(os.path.join(ROCM, "include", "hip")),
                    reason="needs gcc and the HIP headers")
def test_plain_c_program_uses_the_abi(tmp_path):
    if not os.path.exists(B.LIB_PATH):
        from streaming_video_diffusion_amd import build
        build.build()
    src = tmp_path / "prog.c"
    src.write_text(PROGRAM)
    exe = tmp_path / "prog"
    libdir = os.path.dirname(B.LIB_PATH)
    cmd = ["gcc", "-std=c11", "-Wall", "-Werror=implicit-function-declaration", "-D__HIP_PLATFORM_AMD__",
           "-I" + os.path.join(ROOT, "include"), "-I" + os.path.join(ROCM, "include"), str(src),
           "-L" + libdir, "-l:" + os.path.basename(B.LIB_PATH), "-Wl,-rpath," + libdir, "-o", str(exe)]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    out = subprocess.run([str(exe)], check=True, capture_output=True, text=True).stdout.split()
    n_bytes = B.packed_bytes(40, 128, __import__("torch").bfloat16, 28480)
    assert out[0] == str(B.abi_version())
    assert int(out[1]) == n_bytes
    assert out[2] == "SA_ERR_NULL" and out[3] == "-1"
    assert "NULL" in " ".join(out[4:])
