"""Build libstreamattn.so in-tree with hipcc for gfx950.

Usage: ``python -m streaming_video_diffusion_amd.build`` (or ``build()``).
Every HIP source under ``csrc/`` is compiled with ``--offload-arch=gfx950``
into one shared library next to this file.
"""

import glob
import os
import subprocess
import sys
import tempfile

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libstreamattn.so")
# the rotate-in-forward variant (keys rotated in the forward's key-tile load)
ROTK_LIB = os.path.join(PKG, "libstreamattn_rotk.so")
ROTK_FLAGS = ("-DSA_ROTATE_K_IN_FORWARD=1",)
# the host-sanitizer build: host code (argument validation, dispatch) with
# AddressSanitizer and UndefinedBehaviorSanitizer; device code as usual
SAN_LIB = os.path.join(PKG, "libstreamattn_san.so")
SAN_FLAGS = tuple("-Xarch_host -fsanitize=address -Xarch_host -fsanitize=undefined "
                  "-Xarch_host -fno-sanitize-recover=all -Xarch_host -fno-omit-frame-pointer -g".split())
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

FLAGS = [
    "-O3", "-std=c++17", "-fPIC", "-shared", f"--offload-arch={ARCH}",
    # No packed-fp32 VALU instructions in any kernel.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
    f"-I{INCLUDE}", f"-I{CSRC}",
]


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def build(verbose=False, extra_flags=(), lib_path=LIB):
    """Compile every csrc/*.hip into libstreamattn.so (always recompiles).

    ``extra_flags`` such as ``-DSA_ROTATE_K_IN_FORWARD=1`` (keys rotated in
    the forward's key-tile load instead of the pack) build a variant, usually
    with its own ``lib_path``; the binding loads a variant named by the
    STREAMATTN_LIB environment variable.
    """
    srcs = sources()
    if not srcs:
        raise RuntimeError(f"no HIP sources under {CSRC}")
    out_dir = os.path.dirname(os.path.abspath(lib_path))
    fd, tmp = tempfile.mkstemp(suffix=".so", dir=out_dir, prefix=".libstreamattn.")
    os.close(fd)
    cmd = [HIPCC, *FLAGS, *extra_flags, *srcs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    proc = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass warns that it does not know the packed-fp32 feature.
    noise = "is not a recognized feature for this target"
    err = "\n".join(line for line in proc.stderr.splitlines() if noise not in line)
    if proc.returncode != 0:
        os.unlink(tmp)
        raise RuntimeError(f"hipcc failed ({proc.returncode}):\n{err}")
    if verbose and err.strip():
        print(err, file=sys.stderr)
    os.replace(tmp, lib_path)
    return lib_path


if __name__ == "__main__":
    import argparse
    ap = argparse.ArgumentParser()
    ap.add_argument("--rotate-k-in-forward", action="store_true",
                    help="variant: keys rotated in the forward's key-tile load, not in the pack")
    ap.add_argument("--sanitize", action="store_true",
                    help="variant: host code with address and undefined-behaviour sanitizers")
    ap.add_argument("--out", default=None, help="library path to write")
    args = ap.parse_args()
    flags = ROTK_FLAGS if args.rotate_k_in_forward else ()
    out = args.out or LIB
    if args.sanitize:
        flags = flags + SAN_FLAGS
        out = args.out or SAN_LIB
    print(build(verbose=True, extra_flags=flags, lib_path=out))
