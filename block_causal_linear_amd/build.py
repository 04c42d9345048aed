"""Builds liblinattn.so (the library) and libla_probes.so (the benchmark's
HBM stream probes) in-tree for gfx950 with hipcc.

    python -m block_causal_linear_amd.build
"""

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_PATH = os.path.join(HERE, "liblinattn.so")
SOURCES = [os.path.join(CSRC, "linattn.hip")]
PROBE_LIB_PATH = os.path.join(HERE, "libla_probes.so")
PROBE_SOURCES = [os.path.join(CSRC, "probes.hip")]

HIPCC_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    # never emit packed fp32 VALU ops
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
]


def hipcc():
    exe = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(exe):
        raise RuntimeError("hipcc not found; the ROCm toolchain is required to build liblinattn")
    return exe


def build(verbose=False, extra_flags=()):
    """Builds both libraries; returns the attention library's path."""
    _build_one(PROBE_LIB_PATH, PROBE_SOURCES, verbose, extra_flags)
    return _build_one(LIB_PATH, SOURCES, verbose, extra_flags)


def _build_one(lib_path, sources, verbose, extra_flags):
    tmp = lib_path + ".tmp"
    cmd = [hipcc(), *HIPCC_FLAGS, *extra_flags, "-I", INCLUDE, "-I", CSRC, "-o", tmp, *sources]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"hipcc failed with exit code {res.returncode}")
    if verbose:
        # the host pass does not know the packed-fp32 feature flag; drop that noise
        noise = "is not a recognized feature for this target"
        lines = [l for l in (res.stdout + res.stderr).splitlines() if noise not in l]
        if lines:
            print("\n".join(lines))
    os.replace(tmp, lib_path)
    return lib_path


if __name__ == "__main__":
    print(build(verbose=True))
