"""Host-side checks of the rocprofv3 summary script on synthetic counter files: the copy
calibration scales FETCH_SIZE and WRITE_SIZE so that a plain copy of M MiB reads and writes
M MiB, and each kernel's bytes per dispatch are its mean counters times those factors."""
import csv
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = ["Correlation_Id", "Dispatch_Id", "Grid_Size", "Kernel_Name", "Counter_Name", "Counter_Value"]


def _write(path, counter, rows):
    with open(path, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(HEADER)
        for i, (name, grid, value) in enumerate(rows):
            w.writerow([i, i, grid, name, counter, value])


def test_traffic_scaling(tmp_path):
    mib = 256
    kib = mib * 1024.0
    verify = "void gdn::(anonymous namespace)::conv_tree_verify_kernel<128, 128, 16, false, false>(gdn::VerifyArgs)"
    commit = "void gdn::(anonymous namespace)::replay_commit_kernel<128, 128>(gdn::Dims)"
    # the counters of this machine: FETCH_SIZE reads half of a copy's bytes, WRITE_SIZE all of them
    fetch_rows = [("__amd_rocclr_copyBuffer", 512, 2.5), ("__amd_rocclr_copyBuffer", 131072, kib / 2),
                  ("__amd_rocclr_copyBuffer", 131072, kib / 2), (verify, 1024, 5000.0), (verify, 1024, 5200.0),
                  (commit, 4096, 300000.0)]
    write_rows = [("__amd_rocclr_copyBuffer", 512, 2.5), ("__amd_rocclr_copyBuffer", 131072, kib),
                  ("__amd_rocclr_copyBuffer", 131072, kib), (verify, 1024, 9000.0), (verify, 1024, 9400.0),
                  (commit, 4096, 500000.0)]
    fcsv, wcsv, js = tmp_path / "f.csv", tmp_path / "w.csv", tmp_path / "t.json"
    _write(fcsv, "FETCH_SIZE", fetch_rows)
    _write(wcsv, "WRITE_SIZE", write_rows)
    r = subprocess.run([sys.executable, "-m", "gated_deltanet_speculative_amd.rocprof_summary", "traffic", str(fcsv),
                        str(wcsv), "--copy-mib", str(mib), "--workload", "w", "--cmd-fetch", "f", "--cmd-write", "w",
                        "--json-out", str(js)], capture_output=True, text=True, cwd=ROOT, timeout=120)
    assert r.returncode == 0, r.stderr
    rec = json.loads(js.read_text())
    assert abs(rec["fetch_scale"] - 2.0) < 1e-12 and abs(rec["write_scale"] - 1.0) < 1e-12
    v = rec["kernels"]["conv_tree_verify"]
    assert v["dispatches"] == 2
    assert abs(v["read_bytes"] - 5100.0 * 2.0 * 1024) < 1e-6
    assert abs(v["write_bytes"] - 9200.0 * 1024) < 1e-6
    c = rec["kernels"]["replay_commit"]
    assert abs(c["read_bytes"] - 600000.0 * 1024) < 1e-6 and abs(c["write_bytes"] - 500000.0 * 1024) < 1e-6
    assert "| conv_tree_verify | 2 |" in r.stdout


def test_stats_table(tmp_path):
    p = tmp_path / "s.csv"
    with open(p, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Name", "Calls", "TotalDurationNs", "AverageNs", "Percentage", "MinNs", "MaxNs"])
        w.writerow(["void gdn::(anonymous namespace)::replay_commit_kernel<128, 128>(gdn::Dims)", 3, 30000, 10000,
                    75.0, 9000, 11000])
    r = subprocess.run([sys.executable, "-m", "gated_deltanet_speculative_amd.rocprof_summary", "stats", str(p),
                        "--workload", "w", "--cmd", "c"], capture_output=True, text=True, cwd=ROOT, timeout=120)
    assert r.returncode == 0, r.stderr
    assert "| replay_commit | 3 | 10.000 | 9.000 | 11.000 | 75.0% |" in r.stdout


def test_source_hash_covers_included_headers():
    """A kernel's recorded hash covers the headers it includes, so a change to a shared
    device helper invalidates the counter summaries of every kernel built from it."""
    sys.path.insert(0, ROOT)
    from gated_deltanet_speculative_amd import rocprof_summary as rs

    for k in rs.KERNEL_SOURCES:
        names = [os.path.basename(p) for p in rs.source_files(k)]
        assert names[0] == os.path.basename(rs.KERNEL_SOURCES[k])
        assert {"gdn_device.h", "gdn_internal.h", "gdn_verify.h"} <= set(names), (k, names)
        assert len(names) == len(set(names))
    # kernels built from the same file share a hash; different files differ
    assert rs.source_sha256("prefill_prep") == rs.source_sha256("prefill_state")
    assert rs.source_sha256("prefill_prep") != rs.source_sha256("decode_step")


def test_source_hash_ignores_comments_only():
    """Comments and layout do not enter the hash; code does."""
    sys.path.insert(0, ROOT)
    from gated_deltanet_speculative_amd import rocprof_summary as rs

    base = "int f(int x) {\n    return x + 1;  // one more\n}\n/* a\n   block */\n"
    same = "int f(int x) {\n    return x + 1;  // one MORE, reworded\n}\n/* another\n   block */\n"
    other = "int f(int x) {\n    return x + 2;  // one more\n}\n/* a\n   block */\n"
    assert rs.strip_comments(base) == rs.strip_comments(same)
    assert rs.strip_comments(base) != rs.strip_comments(other)
    assert "return x + 1;" in rs.strip_comments(base) and "one more" not in rs.strip_comments(base)
    relaid = "int f(int x)\n{\n    return x + 1;\n\n}\n"
    assert rs.strip_comments(base) == rs.strip_comments(relaid)

