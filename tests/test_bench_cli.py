"""bench.py's command line on the CPU: more than one GPU is refused with a
message and exit status 2 before anything touches a device, the commands the
profile summaries quote use options bench.py still accepts, and the tests the
docs name exist."""

import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr
    assert r.stdout == ""


def test_profile_commands_use_current_options():
    """Every bench.py command quoted in profiles/ and the docs names only
    options bench.py accepts, so each summary's command can be run again."""
    import glob
    import re

    accepted = set(re.findall(r'add_argument\("(--[\w-]+)"', open(os.path.join(ROOT, "bench.py")).read()))
    assert {"--workload", "--steps", "--warmup", "--no-cpu-baseline"} <= accepted
    files = sorted(glob.glob(os.path.join(ROOT, "profiles", "*.md")))
    files += [os.path.join(ROOT, n) for n in ("DESIGN.md", "README.md")]
    stale = []
    for f in files:
        text = open(f).read().replace("\\\n", " ")
        for m in re.finditer(r"bench\.py([^\n`]*)", text):
            bad = set(re.findall(r"(--[\w-]+)", m.group(1))) - accepted
            if bad:
                stale.append((os.path.basename(f), sorted(bad)))
    assert not stale, stale
    workloads = set(re.findall(r'"(\w+)"', open(os.path.join(ROOT, "bench.py")).read()))
    for f in files:
        for w in re.findall(r"--workload (\w+)", open(f).read()):
            assert w in workloads or w == "W", (os.path.basename(f), w)


def test_docs_name_existing_tests():
    """Every test function or test file the docs and profile summaries name
    exists under tests/."""
    import glob
    import re

    sources = sorted(glob.glob(os.path.join(ROOT, "tests", "*.py")))
    known = {os.path.basename(f)[:-3] for f in sources}
    for f in sources:
        known |= set(re.findall(r"def (test_\w+)", open(f).read()))
    files = sorted(glob.glob(os.path.join(ROOT, "profiles", "*.md")))
    files += [os.path.join(ROOT, n) for n in ("DESIGN.md", "README.md")]
    missing = []
    for f in files:
        for name in set(re.findall(r"\b(test_[a-z0-9_]+)\b", open(f).read())):
            if name not in known:
                missing.append((os.path.basename(f), name))
    assert not missing, missing
