"""Build the HIP library libra_amd.so in-tree for gfx950.

    python -m ring_attention_blockwise_ra_amd.build

compiles csrc/*.hip with hipcc (one object per source, in parallel) and links
ring_attention_blockwise_ra_amd/_lib/libra_amd.so, then the plain-C client
_lib/ra_capi_ring (tests/capi_ring.c) that the GPU tests run. Every call
recompiles.
"""

from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIBDIR = os.path.join(PKG, "_lib")
LIB = os.path.join(LIBDIR, "libra_amd.so")
SOURCES = ["ra_kernels.hip", "ra_bwd.hip", "ra_rope.hip", "ra_api.hip"]
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

COMMON = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-I", INCLUDE, "-I", CSRC,
    # never emit packed fp32 (v_pk_*_f32) instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    # the host pass does not know the packed-fp32 target feature; that warning is noise
    out = "\n".join(line for line in r.stdout.splitlines()
                    if "packed-fp32-ops' is not a recognized feature" not in line)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{out}")
    return out


def build(verbose: bool = False, extra_flags=None) -> str:
    os.makedirs(LIBDIR, exist_ok=True)
    objdir = os.path.join(LIBDIR, "obj")
    os.makedirs(objdir, exist_ok=True)
    flags = COMMON + list(extra_flags or [])

    def compile_one(src):
        obj = os.path.join(objdir, src.replace(".hip", ".o"))
        out = _run([HIPCC, *flags, "-c", os.path.join(CSRC, src), "-o", obj])
        if verbose and out.strip():
            print(out)
        return obj

    with ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(compile_one, SOURCES))
    tmp = LIB + ".tmp"
    _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs])
    os.replace(tmp, LIB)
    build_c_client()
    return LIB


C_CLIENT_SRC = os.path.join(ROOT, "tests", "capi_ring.c")
C_CLIENT = os.path.join(LIBDIR, "ra_capi_ring")


def build_c_client() -> str | None:
    """The plain-C ring client the GPU tests run (tests/capi_ring.c): C99,
    the HIP runtime's C API and libra_amd.so only, found beside it."""
    if not os.path.exists(C_CLIENT_SRC):
        return None
    rocm = os.path.dirname(os.path.dirname(os.path.realpath(HIPCC)))
    tmp = C_CLIENT + ".tmp"
    _run(["gcc", "-std=c99", "-O2", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
          "-I", os.path.join(rocm, "include"), "-I", INCLUDE, C_CLIENT_SRC,
          "-L", LIBDIR, "-lra_amd", "-L", os.path.join(rocm, "lib"), "-lamdhip64",
          "-Wl,-rpath,$ORIGIN", "-Wl,-rpath," + os.path.join(rocm, "lib"), "-o", tmp])
    os.replace(tmp, C_CLIENT)
    return C_CLIENT


if __name__ == "__main__":
    path = build(verbose="-v" in sys.argv)
    print(path)
