"""include/ra.h from plain C: tests/capi_host.c is compiled as C99 with
warnings as errors against the header, linked against libra_amd.so and run.
It calls host-side entry points only (tile rule, workspace size, argument
validation), so no GPU is needed."""

import os
import shutil
import subprocess

import pytest

from ring_attention_blockwise_ra_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("gcc") is None, reason="no C compiler")
def test_header_compiles_as_c99_and_host_calls_work(tmp_path):
    if not os.path.exists(B.LIB_PATH):
        from ring_attention_blockwise_ra_amd import build
        build.build()
    libdir = os.path.dirname(B.LIB_PATH)
    exe = str(tmp_path / "capi_host")
    cmd = ["gcc", "-std=c99", "-Wall", "-Wextra", "-Werror", "-pedantic", "-I", os.path.join(ROOT, "include"),
           os.path.join(ROOT, "tests", "capi_host.c"), "-L", libdir, "-lra_amd",
           f"-Wl,-rpath,{libdir}", "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stdout + r.stderr
    r = subprocess.run([exe], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0 and r.stdout.strip().endswith("ok"), r.stdout + r.stderr
