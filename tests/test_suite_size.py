"""The GPU suite is registered: collecting tests/ with -m gpu selects at least
GPU_TESTS_MIN tests (a renamed or unregistered file must not empty the GPU run)."""

import os
import subprocess
import sys

from conftest import GPU_TESTS_MIN, ROOT


def test_gpu_suite_is_collected():
    r = subprocess.run([sys.executable, "-m", "pytest", os.path.join(ROOT, "tests"), "--collect-only", "-q", "-m",
                        "gpu", "-p", "no:cacheprovider"], capture_output=True, text=True, cwd=ROOT, timeout=300)
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-2000:]
    n = sum(1 for line in r.stdout.splitlines() if "::" in line)
    assert n >= GPU_TESTS_MIN, f"{n} GPU tests collected"
