"""The host side of the C ABI under AddressSanitizer and
UndefinedBehaviorSanitizer: liblinattn.so is built with its host code
sanitized (block_causal_linear_amd.build.build_sanitized, into a temporary
directory), and the CPU contract tests (test_abi.py, test_plan.py,
test_c_abi.py: argument checks, overlap tests, size and plan arithmetic)
run against it in a child process with the ASan runtime preloaded.  Any
report ends the child with a nonzero status.  Needs no GPU."""

import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

pytestmark = pytest.mark.skipif(shutil.which("hipcc") is None
                                and not os.path.exists("/opt/rocm/bin/hipcc"),
                                reason="needs hipcc")


def test_contract_tests_pass_under_asan_and_ubsan(tmp_path):
    from block_causal_linear_amd import build as b

    lib = b.build_sanitized(str(tmp_path / "san"))
    env = dict(os.environ)
    env.update(LINATTN_LIB=lib, LD_PRELOAD=b.sanitizer_runtime(),
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    tests = [os.path.join(ROOT, "tests", t) for t in ("test_abi.py", "test_plan.py",
                                                     "test_c_abi.py")]
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider", *tests],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "ERROR: AddressSanitizer" not in out and "runtime error:" not in out, out[-4000:]
    assert " passed" in r.stdout
