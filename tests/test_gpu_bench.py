"""bench.py on the GPU, briefly: each mode prints one JSON line whose roofline fields are
consistent (achieved / peak = frac, bytes / time = achieved) and whose workload is the
one asked for."""
import json
import os
import subprocess
import sys

import pytest

from gpu_util import log

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench(*extra):
    cmd = [sys.executable, os.path.join(ROOT, "bench.py"), "--steps", "2", "--warmup", "1", "--kernel-reps", "2",
           "--no-cpu-baseline", *extra]
    log(f"[bench] {' '.join(cmd[2:])}")
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=110, cwd=ROOT)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [ln for ln in r.stdout.splitlines() if ln.startswith("{")]
    assert len(lines) == 1, r.stdout[-2000:]
    return json.loads(lines[0])


@pytest.mark.gpu
@pytest.mark.parametrize("extra,workload", [((), "tree-c4-n16"), (("--mode", "decode", "--instances", "8"),
                                                                    "tree-c4-n16-decode"),
                                            (("--mode", "decode", "--route", "split", "--instances", "8"),
                                             "tree-c4-n16-decode"),
                                            (("--lanes", "8", "--instances", "8"), "tree-c4-n16-lanes8")])
def test_bench_line(extra, workload):
    d = _bench(*extra)
    assert d["n_gpus"] == 1 and d["steps"] == 2 and d["warmup"] == 1 and d["higher_is_better"] is True
    assert d["config"]["workload"] == workload and d["value"] > 0 and d["ms_per_step"] > 0
    assert d["cpu_baseline"] is None
    rl = d["roofline"]
    assert rl["bound"] == "hbm" and rl["unit"] == "GB/s" and rl["peak"] == 8000.0
    assert abs(rl["frac"] - rl["achieved"] / rl["peak"]) < 1e-3
    assert abs(rl["achieved"] - rl["bytes_per_launch"] / (rl["us_per_launch"] * 1e3)) / rl["achieved"] < 1e-2
    if "decode" in workload:
        assert rl["kernel"] == ("decode_step" if "split" in extra else "conv_decode")
    if "lanes8" in workload:
        assert d["config"]["lanes"] == 8 and d["config"]["slots"] == 8
    cp = d["copy_same_bytes"]  # a plain copy of the dominant kernel's bytes in the same run
    assert cp["bytes"] > 0 and cp["us"] > 0 and abs(cp["bytes"] - rl["bytes_per_launch"]) <= 8
    if "decode" not in workload:  # the dispatch floor of this machine, beside the kernel times
        fl = d["dispatch_floor"]
        assert 0 < fl["empty_kernel_us"] < fl["padding_lanes_same_grid_us"] < rl["us_per_launch"]
