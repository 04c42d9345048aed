"""The C ABI used from C: tests/c/abi_smoke.c is compiled with gcc against
include/linattn.h, linked to liblinattn.so and run.  It makes only calls that
need no GPU (argument rejections, sizes, the plan, version and status
strings), so it runs on the CPU."""

import os
import shutil
import subprocess

import pytest

import block_causal_linear_amd as la

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")

pytestmark = pytest.mark.skipif(
    not os.path.exists(la.LIB_PATH) or shutil.which("gcc") is None
    or not os.path.exists(os.path.join(ROCM, "include", "hip", "hip_runtime_api.h")),
    reason="needs the built library, gcc and the HIP headers")


def test_plain_c_program(tmp_path):
    exe = tmp_path / "abi_smoke"
    libdir = os.path.dirname(la.LIB_PATH)
    cmd = ["gcc", "-std=c99", "-Wall", "-Wextra", "-Werror", "-I", os.path.join(ROOT, "include"),
           "-I", os.path.join(ROCM, "include"), "-D__HIP_PLATFORM_AMD__",
           os.path.join(ROOT, "tests", "c", "abi_smoke.c"), "-L", libdir, "-llinattn",
           f"-Wl,-rpath,{libdir}", "-o", str(exe)]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0, r.stderr
    assert "abi_smoke ok" in r.stdout
