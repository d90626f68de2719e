"""Turn rocprofv3 CSV output into the short summaries kept under profiles/.

    python -m gated_deltanet_speculative_amd.rocprof_summary stats KERNEL_STATS_CSV --workload NAME --cmd "..."
    python -m gated_deltanet_speculative_amd.rocprof_summary traffic FETCH_CSV WRITE_CSV --copy-mib M \
        --workload NAME --cmd-fetch "..." --cmd-write "..."

`stats` prints a markdown table of per-kernel dispatch counts and durations.
`traffic` averages FETCH_SIZE and WRITE_SIZE (KiB per dispatch) per kernel, scales
each by what the same counter reads for the calibration copy (M MiB read and M MiB
written by one plain copy kernel), and writes both a markdown table and a JSON
record that bench.py uses for the roofline's `traffic` field.  The JSON carries the
SHA-256 of each kernel's source file and the project headers it includes (comments and
layout removed), so a later change to a kernel's code makes bench.py report its traffic as
unknown instead of stale.
"""

from __future__ import annotations

import argparse
import csv
import hashlib
import json
import os
import re
import statistics
from collections import defaultdict

PKG = os.path.dirname(os.path.abspath(__file__))
KERNEL_SOURCES = {  # (matched in this order: conv_tree_verify before tree_verify)
    "conv_tree_verify": "csrc/tree_verify.hip",
    "conv_tree_step": "csrc/conv_tree_step.hip",
    "tree_verify": "csrc/tree_verify.hip",
    "replay_commit": "csrc/replay_commit.hip",
    "conv_decode": "csrc/decode_step.hip",  # the fused plain step (conv_decode_group_kernel, or conv_decode_kernel)
    "decode_step": "csrc/decode_step.hip",
    "prefill_prep": "csrc/prefill.hip",
    "prefill_state": "csrc/prefill.hip",
    "conv_step": "csrc/decode_step.hip",
}
INCLUDE_DIRS = (os.path.join(PKG, "csrc"), os.path.join(os.path.dirname(PKG), "include"))


def source_files(kernel: str) -> list:
    """The kernel's source file and every project header it includes, directly or through
    another header (quoted includes found in csrc/ or include/), in a fixed order."""
    out, todo = [], [os.path.join(PKG, KERNEL_SOURCES[kernel])]
    while todo:
        path = todo.pop(0)
        if path in out:
            continue
        out.append(path)
        with open(path, encoding="utf-8") as f:
            for name in re.findall(r'^\s*#\s*include\s+"([^"]+)"', f.read(), re.M):
                for d in INCLUDE_DIRS:
                    if os.path.exists(os.path.join(d, name)):
                        todo.append(os.path.join(d, name))
                        break
    return out


_COMMENT = re.compile(r"//[^\n]*|/\*.*?\*/", re.S)


def strip_comments(text: str) -> str:
    """The source with its // and /* */ comments removed and every run of white space made
    one space, so that an edit of comments or layout leaves the hash alone.  (A '//' inside a
    string literal would be cut too, the same way every time, which keeps the hash
    deterministic.)"""
    return " ".join(_COMMENT.sub(" ", text).split())


def source_sha256(kernel: str) -> str:
    """sha256 over the kernel's source and the project headers it includes, comments removed:
    a counter summary taken under another hash no longer describes the built kernel."""
    h = hashlib.sha256()
    for path in source_files(kernel):
        with open(path, encoding="utf-8") as f:
            h.update(strip_comments(f.read()).encode())
    return h.hexdigest()


# kernels reported under another kernel's name (the same call, another launch shape)
KERNEL_ALIASES = {"conv_decode_group": "conv_decode"}


def short_name(name: str) -> str:
    for k, v in KERNEL_ALIASES.items():
        if k + "_kernel" in name:
            return v
    for k in KERNEL_SOURCES:
        if k + "_kernel" in name:
            return k
    return "copy" if "copyBuffer" in name else name.split("(")[0][-60:]


def stats(path: str) -> list:
    rows = []
    for r in csv.DictReader(open(path)):
        rows.append((short_name(r["Name"]), int(r["Calls"]), float(r["AverageNs"]) / 1e3, float(r["MinNs"]) / 1e3,
                     float(r["MaxNs"]) / 1e3, float(r["Percentage"])))
    return rows


def counters(path: str) -> dict:
    per = defaultdict(list)
    for r in csv.DictReader(open(path)):
        key = short_name(r["Kernel_Name"])
        if key == "copy":
            key = f"copy:grid{r['Grid_Size']}"
        per[key].append(float(r["Counter_Value"]))
    return per


def main():
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="mode", required=True)
    a = sub.add_parser("stats")
    a.add_argument("csv")
    a.add_argument("--workload", required=True)
    a.add_argument("--cmd", required=True)
    b = sub.add_parser("traffic")
    b.add_argument("fetch_csv")
    b.add_argument("write_csv")
    b.add_argument("--copy-mib", type=int, required=True)
    b.add_argument("--workload", required=True)
    b.add_argument("--cmd-fetch", required=True)
    b.add_argument("--cmd-write", required=True)
    b.add_argument("--json-out", required=True)
    args = ap.parse_args()

    if args.mode == "stats":
        print(f"# Kernel durations, {args.workload}\n\nCommand:\n\n    {args.cmd}\n")
        print("| kernel | dispatches | mean us | min us | max us | share of GPU time |")
        print("|---|---|---|---|---|---|")
        for name, calls, avg, mn, mx, pct in stats(args.csv):
            print(f"| {name} | {calls} | {avg:.3f} | {mn:.3f} | {mx:.3f} | {pct:.1f}% |")
        return

    fetch, write = counters(args.fetch_csv), counters(args.write_csv)
    copy_kib = args.copy_mib * 1024.0
    big = max((k for k in fetch if k.startswith("copy:")), key=lambda k: statistics.mean(fetch[k]))
    f_scale = copy_kib / statistics.mean(fetch[big])
    w_scale = copy_kib / statistics.mean(write[big])
    rec = {"workload": args.workload, "fetch_scale": f_scale, "write_scale": w_scale,
           "calibration": f"{args.copy_mib} MiB plain copy ({big}): FETCH_SIZE {statistics.mean(fetch[big]):.1f} KiB, "
                          f"WRITE_SIZE {statistics.mean(write[big]):.1f} KiB", "kernels": {}}
    print(f"# Fabric traffic per dispatch, {args.workload}\n")
    print(f"Commands:\n\n    {args.cmd_fetch}\n    {args.cmd_write}\n")
    print(f"Calibration: {rec['calibration']}; scale factors fetch x{f_scale:.4f}, write x{w_scale:.4f}.\n")
    print("| kernel | dispatches | FETCH_SIZE KiB | WRITE_SIZE KiB | read MB (scaled) | written MB (scaled) |")
    print("|---|---|---|---|---|---|")
    for k in KERNEL_SOURCES:
        if k not in fetch or k not in write:
            continue
        fk, wk = statistics.mean(fetch[k]), statistics.mean(write[k])
        rb, wb = fk * f_scale * 1024, wk * w_scale * 1024
        rec["kernels"][k] = {"read_bytes": rb, "write_bytes": wb, "source_sha256": source_sha256(k),
                             "dispatches": len(fetch[k])}
        print(f"| {k} | {len(fetch[k])} | {fk:.1f} | {wk:.1f} | {rb / 1e6:.3f} | {wb / 1e6:.3f} |")
    with open(args.json_out, "w") as f:
        json.dump(rec, f, indent=1)
        f.write("\n")


if __name__ == "__main__":
    main()
