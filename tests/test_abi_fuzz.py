"""Host-only fuzz of the C-ABI argument validation under AddressSanitizer and
UndefinedBehaviorSanitizer: gdn_api.cpp is compiled with g++ against stand-in launchers
(tests/host_fuzz/stubs.cpp, no device code, nothing reaches a GPU), and every entry point
is called with random and extreme shapes and NULL, misaligned and overlapping fake pointers
(tests/host_fuzz/harness.cpp).  The run must end without a sanitizer report, with only
documented return codes and with some calls accepted."""

import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIP_INCLUDE = "/opt/rocm/include"


@pytest.mark.skipif(shutil.which("g++") is None or not os.path.exists(os.path.join(HIP_INCLUDE, "hip")),
                    reason="needs g++ and the HIP headers")
def test_validation_fuzz_under_sanitizers(tmp_path):
    flags = ["-O1", "-g", "-std=c++17", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
             "-D__HIP_PLATFORM_AMD__", "-I", HIP_INCLUDE, "-I", os.path.join(ROOT, "include"),
             "-I", os.path.join(ROOT, "gated_deltanet_speculative_amd", "csrc")]
    srcs = [os.path.join(ROOT, "gated_deltanet_speculative_amd", "csrc", "gdn_api.cpp"),
            os.path.join(ROOT, "tests", "host_fuzz", "stubs.cpp"),
            os.path.join(ROOT, "tests", "host_fuzz", "harness.cpp")]
    exe = str(tmp_path / "harness")
    r = subprocess.run(["g++", *flags, *srcs, "-o", exe], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, (r.stdout + r.stderr)[-3000:]
    m = re.search(r"launches (\d+); codes:", r.stdout)
    assert m and int(m.group(1)) > 1000, r.stdout
