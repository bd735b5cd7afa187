"""The library's host code (argument validation and dispatch in api.hip)
under AddressSanitizer and UndefinedBehaviorSanitizer.

The sanitizer build instruments host code only (device code is built as
usual and never runs here). The ABI and binding tests that need no GPU run
against it in a child process with the sanitizer runtime preloaded, and so
does the plain C program of test_abi_c; any report fails the test (the
build stops at the first report and the logs must stay empty)."""

import glob
import os
import shutil
import subprocess
import sys

import pytest

from streaming_video_diffusion_amd import build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def asan_runtime():
    hits = sorted(glob.glob(os.path.join(ROCM, "llvm", "lib", "clang", "*", "lib", "linux",
                                         "libclang_rt.asan-x86_64.so")))
    return hits[-1] if hits else None


def sanitizer_lib():
    """libstreamattn_san.so, rebuilt when older than any source or header."""
    srcs = build.sources() + glob.glob(os.path.join(build.CSRC, "*.h")) + glob.glob(os.path.join(build.INCLUDE, "*.h"))
    lib = build.SAN_LIB
    if not os.path.exists(lib) or os.path.getmtime(lib) < max(os.path.getmtime(s) for s in srcs):
        build.build(extra_flags=build.SAN_FLAGS, lib_path=lib)
    return lib


def sanitizer_env(tmp_path, lib):
    env = dict(os.environ)
    env["STREAMATTN_LIB"] = lib
    env["LD_PRELOAD"] = asan_runtime()
    # CPython itself leaks by design at exit; leak checking stays off
    env["ASAN_OPTIONS"] = f"detect_leaks=0:abort_on_error=1:log_path={tmp_path}/asan"
    env["UBSAN_OPTIONS"] = f"print_stacktrace=1:halt_on_error=1:log_path={tmp_path}/ubsan"
    return env


def reports(tmp_path):
    return sorted(glob.glob(str(tmp_path / "asan*")) + glob.glob(str(tmp_path / "ubsan*")))


pytestmark = pytest.mark.skipif(asan_runtime() is None or not os.path.exists(build.HIPCC),
                                reason="needs hipcc and the clang sanitizer runtime")


def test_abi_and_binding_checks_under_sanitizers(tmp_path):
    lib = sanitizer_lib()
    cmd = [sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
           os.path.join(ROOT, "tests", "test_abi_cpu.py"), os.path.join(ROOT, "tests", "test_binding_checks.py")]
    r = subprocess.run(cmd, cwd=ROOT, env=sanitizer_env(tmp_path, lib), capture_output=True, text=True, timeout=600)
    logs = reports(tmp_path)
    detail = "".join(open(p).read()[:3000] for p in logs)
    assert r.returncode == 0 and not logs, f"rc={r.returncode}\n{r.stdout[-2000:]}\n{r.stderr[-2000:]}\n{detail}"
    assert " passed" in r.stdout


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_plain_c_program_under_sanitizers(tmp_path):
    from test_abi_c import PROGRAM
    lib = sanitizer_lib()
    src = tmp_path / "prog.c"
    src.write_text(PROGRAM)
    exe = tmp_path / "prog"
    libdir = os.path.dirname(lib)
    cmd = ["gcc", "-std=c11", "-Wall", "-D__HIP_PLATFORM_AMD__", "-I" + os.path.join(ROOT, "include"),
           "-I" + os.path.join(ROCM, "include"), str(src), "-L" + libdir, "-l:" + os.path.basename(lib),
           "-Wl,-rpath," + libdir, "-Wl,--allow-shlib-undefined", "-o", str(exe)]  # runtime comes preloaded
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    r = subprocess.run([str(exe)], env=sanitizer_env(tmp_path, lib), capture_output=True, text=True, timeout=120)
    logs = reports(tmp_path)
    assert r.returncode == 0 and not logs, f"rc={r.returncode} {r.stdout} {r.stderr} {logs}"
    assert r.stdout.split()[2] == "SA_ERR_NULL"
