"""Builds liblinattn.so (the library) and libla_probes.so (the benchmark's
HBM stream probes) in-tree for gfx950 with hipcc.

    python -m block_causal_linear_amd.build
    python -m block_causal_linear_amd.build --sanitize DIR   # host code under ASan + UBSan
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


# The host code under AddressSanitizer and UndefinedBehaviorSanitizer, for the
# CPU contract tests (argument checks, overlap tests, size arithmetic): each
# -fsanitize applies to the host pass only (-Xarch_host); the device code is
# built as usual and never runs in those tests.  The runtime's directory goes
# into the rpath; a process that loads the library must preload the ASan
# runtime (sanitizer_runtime()).
SANITIZE_FLAGS = [
    "-Xarch_host", "-fsanitize=address",
    "-Xarch_host", "-fsanitize=undefined",
    "-Xarch_host", "-fno-sanitize-recover=undefined",
    "-Xarch_host", "-fno-omit-frame-pointer",
    "-shared-libsan",
]


def sanitizer_runtime():
    """Path of the clang ASan runtime that ships with ROCm's compiler."""
    import glob

    root = os.environ.get("ROCM_PATH", "/opt/rocm")
    hits = sorted(glob.glob(os.path.join(root, "llvm", "lib", "clang", "*", "lib", "linux",
                                         "libclang_rt.asan-x86_64.so")))
    if not hits:
        raise RuntimeError("the clang ASan runtime was not found under " + root)
    return hits[-1]


def build_sanitized(out_dir, verbose=False):
    """liblinattn.so with the host code sanitized, in out_dir (not in-tree)."""
    os.makedirs(out_dir, exist_ok=True)
    rt_dir = os.path.dirname(sanitizer_runtime())
    flags = [f for f in HIPCC_FLAGS if f != "-O3"] + ["-O1", "-g"] + SANITIZE_FLAGS + [
        f"-Wl,-rpath,{rt_dir}"]
    out = os.path.join(out_dir, "liblinattn.so")
    cmd = [hipcc(), *flags, "-I", INCLUDE, "-I", CSRC, "-o", out, *SOURCES]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"hipcc failed with exit code {res.returncode}")
    return out


if __name__ == "__main__":
    if len(sys.argv) == 3 and sys.argv[1] == "--sanitize":
        print(build_sanitized(sys.argv[2], verbose=True))
    else:
        print(build(verbose=True))
