"""Host-side checks of bench.py (no GPU): the one-GPU guard, and the algorithmic byte
counts behind the roofline figure, recomputed here tensor by tensor from the layouts of
the library header (fp32, every input read once, every output written once)."""
import os
import subprocess
import sys

import pytest

import bench
from workloads import WORKLOADS

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _elements(*shape):
    n = 1
    for s in shape:
        n *= s
    return n


def _tensors(wl):
    C, N, Ch, Hv, dk, dv = wl.n_seqs, wl.n_nodes, wl.channels, wl.n_v_heads, wl.d_k, wl.d_v
    W, R = wl.d_conv - 1, 1 + dk + dv
    return dict(
        x=_elements(C, N, Ch), conv_w=_elements(Ch, wl.d_conv), hist_rows=_elements(C, Ch, W),
        conv_out=_elements(C, N, Ch), windows=_elements(C, N, Ch, W), gates=2 * _elements(C, N, Hv),
        dt_A=2 * Hv, state_blocks=_elements(C, Hv, dk, dv), out=_elements(C, N, Hv, dv),
        log=_elements(C, N, Hv, R), R=R)


@pytest.mark.parametrize("name", ["tree-c4-n16", "chains-c5-n8-l48", "stress-c64-n32-l48", "tiny-chain"])
def test_round_bytes_tensor_by_tensor(name):
    wl = WORKLOADS[name]
    t = _tensors(wl)
    ab = bench.algorithmic_bytes(wl, accept_depths=[0] * wl.n_seqs)
    conv = t["x"] + t["conv_w"] + t["hist_rows"] + t["conv_out"] + t["windows"]
    verify = t["conv_out"] + t["gates"] + t["dt_A"] + t["state_blocks"] + t["out"] + t["log"]
    fused = t["x"] + t["conv_w"] + t["hist_rows"] + t["windows"] + t["gates"] + t["dt_A"] + t["state_blocks"] \
        + t["out"] + t["log"]
    assert ab["conv"] == 4 * conv
    assert ab["verify"] == 4 * verify
    assert ab["conv_verify"] == 4 * fused
    assert ab["commit"] == 0  # nothing accepted: nothing moves


def test_bench_shape_figure():
    """The byte count the bench line reports for the fused launch at its workload."""
    assert bench.algorithmic_bytes(WORKLOADS["tree-c4-n16"], [0] * 4)["conv_verify"] == 20472064


def test_commit_bytes_follow_the_accepted_paths():
    wl = WORKLOADS["tree-c4-n16"]
    t = _tensors(wl)
    depths = [0, 1, 3, 16]
    Hv, dk, dv, Ch, W = wl.n_v_heads, wl.d_k, wl.d_v, wl.channels, wl.d_conv - 1
    per_lane = [0 if a == 0 else 2 * Hv * dk * dv + 2 * Ch * W + a * Hv * t["R"] for a in depths]
    assert bench.algorithmic_bytes(wl, depths)["commit"] == 4 * sum(per_lane)


def test_ragged_counts_scale_the_node_terms():
    wl = WORKLOADS["tree-c4-n16"]
    full = bench.algorithmic_bytes(wl, [0] * 4)
    half = bench.algorithmic_bytes(wl, [0] * 4, lane_counts=[8] * 4)
    t = _tensors(wl)
    node_terms = t["x"] + t["windows"] + t["gates"] + t["out"] + t["log"]  # per node, in the fused launch
    assert full["conv_verify"] - half["conv_verify"] == 4 * node_terms // 2


def test_decode_bytes_tensor_by_tensor():
    wl = WORKLOADS["tree-c4-n16"]
    C, Ch, Hv, dk, dv, W = wl.n_seqs, wl.channels, wl.n_v_heads, wl.d_k, wl.d_v, wl.d_conv - 1
    db = bench.decode_bytes(wl)
    # conv step: history rows read and written, one token read, conv row written, taps
    assert db["conv_step"] == 4 * (2 * C * Ch * W + C * Ch + C * Ch + Ch * wl.d_conv)
    # recurrence: state read and written, conv row, two gates, dt and A, output row
    assert db["decode_step"] == 4 * (2 * C * Hv * dk * dv + C * Ch + 2 * C * Hv + 2 * Hv + C * Hv * dv)
    # fused: both, without the conv row written by one and read by the other
    assert db["conv_decode"] == 4 * (2 * C * Ch * W + C * Ch + Ch * wl.d_conv + 2 * C * Hv * dk * dv + 2 * C * Hv
                                     + 2 * Hv + C * Hv * dv)


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in r.stdout + r.stderr


@pytest.mark.parametrize("fn,unit", [("cpu_baseline", "verify tokens/s"), ("cpu_baseline_decode", "decode tokens/s"),
                                     ("cpu_baseline_prefill", "prompt tokens/s")])
def test_cpu_baselines_report_their_sample(fn, unit):
    r = getattr(bench, fn)(WORKLOADS["tiny-chain"], 0.05, 0)
    assert r["unit"] == unit and r["kind"] == "oracle" and r["cores"] == 1
    assert r["value"] > 0 and "fp64" in r["sample"]
    # the host it ran on: logical CPUs, usable CPUs, model, and one BLAS thread in the baseline
    assert r["host_cpu_count"] == os.cpu_count() and 1 <= r["host_cpus_usable"] <= r["host_cpu_count"]
    assert "cpu_model" in r
    assert all(b["threads"] == 1 for b in r["blas_in_baseline"])
    if fn == "cpu_baseline":  # also one layer of the single-lane grouped chain
        c1 = r["grouped_chain_n8"]
        assert c1["unit"] == "verify tokens/s" and c1["value"] > 0
        assert abs(c1["value"] - 8 / c1["seconds"]) / c1["value"] < 1e-2
