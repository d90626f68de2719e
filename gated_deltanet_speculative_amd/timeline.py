"""Per-phase timeline of the fused conv + verify launch, from an instrumented build.

    python -m gated_deltanet_speculative_amd.timeline build
    python -m gated_deltanet_speculative_amd.timeline run [--workload tree-c4-n16] [--instances 64] [--lanes N]

`build` (no GPU needed) writes a copy of csrc/tree_verify.hip in which thread 0 of every
workgroup records the shader clock (s_memtime) at the start of the verify body, once its
first loads are back and the tree is walked, after every LDS barrier of the body, and at
its end (the window workgroups at their start and end), plus the constant 100 MHz clock
(s_memrealtime) at start and end to convert cycles to microseconds.  Stamps go to a
fixed device array with ordinary vector stores.  The copy is linked with the other
sources into libgdntimeline.so beside this file; the library's own sources are not
changed, and nothing in the library loads the instrumented copy.

`run` (on the GPU) replays the launch over the workload's layer instances as the bench
does, reads the stamps of the last launch and prints, per phase, the median, p10 and p90
over the verify workgroups.  The shader clock runs per XCD, so only differences within one
workgroup are meaningful; the constant clock is common to the chip and places every
workgroup's start and end (verify and window workgroups) on one time line.  Wave 4 also
stamps the start of its state product, once its state chunks are all back (it waits for
them there anyway).  The stamps cost time themselves (each waits
for the LDS counters); the launch time printed last is the instrumented one.
"""

from __future__ import annotations

import argparse
import ctypes
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libgdntimeline.so")
MAX_WG = 4096  # workgroups whose stamps are kept

PHASES = [  # (stamp slot, name) in the order a verify workgroup passes them
    (1, "first loads back, tree walked"),
    (2, "token rows staged"),
    (3, "conv + SiLU"),
    (4, "Gram + state product"),
    (5, "coefficients"),
    (6, "solve + rhs"),
    (7, "epilogue staged"),
    (10, "stores issued"),
]

_STAMP_DEFS = f"""
#define GDN_TL_MAX_WG {MAX_WG}
__device__ unsigned long long gdn_tl_stamps[GDN_TL_MAX_WG][16];
#define GDN_STAMP(k) do {{ if (threadIdx.x == 0 && blockIdx.x < GDN_TL_MAX_WG) \\
    __builtin_nontemporal_store(__builtin_amdgcn_s_memtime(), &gdn_tl_stamps[blockIdx.x][k]); }} while (0)
#define GDN_STAMP_ARRIVAL(r) do {{ if (threadIdx.x == 256 && blockIdx.x < GDN_TL_MAX_WG) {{ \
    asm volatile("" :: "v"(r[0][0]), "v"(r[LCQ - 1][3])); \
    __builtin_nontemporal_store(__builtin_amdgcn_s_memtime(), &gdn_tl_stamps[blockIdx.x][11]); }} }} while (0)
#define GDN_RSTAMP(k) do {{ if (threadIdx.x == 0 && blockIdx.x < GDN_TL_MAX_WG) \\
    __builtin_nontemporal_store(__builtin_amdgcn_s_memrealtime(), &gdn_tl_stamps[blockIdx.x][k]); }} while (0)
extern "C" int gdn_timeline_read(unsigned long long *host) {{
    return (int)hipMemcpyFromSymbol(host, HIP_SYMBOL(gdn_tl_stamps), sizeof(gdn_tl_stamps), 0, hipMemcpyDeviceToHost);
}}
"""


def _instrument(src: str) -> str:
    """The verify kernels' source with the stamps inserted (asserts that every anchor exists)."""

    def sub(a: str, b: str) -> None:
        nonlocal src
        assert a in src, f"instrumentation anchor not found: {a[:70]!r}"
        src = src.replace(a, b, 1)

    sub("namespace gdn {\nnamespace {", _STAMP_DEFS + "\nnamespace gdn {\nnamespace {")
    body = src.index("__device__ __forceinline__ void verify_body")
    end = src.index("__global__ __launch_bounds__(kThreads) void tree_verify_kernel")
    part = src[body:end]
    out, k = [], 2
    for line in part.split("\n"):
        out.append(line)
        if line.strip() == "lds_barrier();":
            out.append(f"    GDN_STAMP({k});")
            k += 1
    assert k == 8, f"expected 6 barriers in the verify body, found {k - 2}"
    part = "\n".join(out)
    close = part.rindex("}\n", 0, part.rindex("template <int DK, int DV, int NP, bool RAGGED, bool WIDE>"))
    part = part[:close] + "    GDN_STAMP(10); GDN_RSTAMP(13);\n" + part[close:]
    src = src[:body] + part + src[end:]
    sub("    auto state_product = [&]() {\n", "    auto state_product = [&]() {\n        GDN_STAMP_ARRIVAL(sreg);\n")
    sub("    const Dims d = args.d;\n    // every kernel argument used for an address",
        "    GDN_STAMP(0); GDN_RSTAMP(12);\n    const Dims d = args.d;\n    // every kernel argument used for an address")
    sub("    // fused: stage the raw token rows for the tree conv\n",
        "    GDN_STAMP(1);\n    // fused: stage the raw token rows for the tree conv\n")
    sub("    constexpr int GPB = kThreads / NP;  // 4-channel groups per workgroup\n",
        "    constexpr int GPB = kThreads / NP;  // 4-channel groups per workgroup\n    GDN_STAMP(0); GDN_RSTAMP(12);\n")
    wb = src.index("void window_body")
    wend = src.index("void conv_tree_verify_kernel(")
    wclose = src.rindex("}\n", wb, src.rindex("template", wb, wend))
    src = src[:wclose] + "    GDN_STAMP(10); GDN_RSTAMP(13);\n" + src[wclose:]
    return src


def build() -> str:
    from gated_deltanet_speculative_amd.build import HIPCC_FLAGS, SOURCE_FLAGS, SOURCES, _hipcc

    tmp = os.path.join(ROOT, "_build", "timeline")
    os.makedirs(tmp, exist_ok=True)
    objs = []
    for name in SOURCES:
        path = os.path.join(CSRC, name)
        if name == "tree_verify.hip":
            path = os.path.join(tmp, name)
            with open(path, "w") as f:
                f.write(_instrument(open(os.path.join(CSRC, name)).read()))
        obj = os.path.join(tmp, name + ".o")
        cmd = [_hipcc(), *HIPCC_FLAGS, *SOURCE_FLAGS.get(name, []), "-x", "hip", "-c", path, "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode:
            raise RuntimeError(f"hipcc failed on {name}:\n{r.stderr[-3000:]}")
        objs.append(obj)
    r = subprocess.run([_hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", LIB], capture_output=True,
                       text=True)
    if r.returncode:
        raise RuntimeError(f"link failed:\n{r.stderr[-3000:]}")
    print(f"built {LIB}")
    return LIB


def run(workload: str, instances: int, lanes: int | None = None) -> None:
    import dataclasses

    import numpy as np
    import torch

    if ROOT not in sys.path:
        sys.path.insert(0, ROOT)
    import gated_deltanet_speculative_amd as gdn
    from gated_deltanet_speculative_amd import _lib
    from workloads import WORKLOADS, layer_params, round_inputs, round_structure

    if not os.path.exists(LIB):
        raise RuntimeError(f"{LIB} is missing: run `python -m gated_deltanet_speculative_amd.timeline build`")
    lib = _lib.load_library(LIB)
    _lib._lib = lib  # the binding's calls go to the instrumented build
    lib.gdn_timeline_read.argtypes = [ctypes.c_void_p]
    wl = WORKLOADS[workload]
    if lanes is not None:  # the workload's head shape and trees with this many lanes, as in bench.py
        wl = dataclasses.replace(wl, name=f"{wl.name}-lanes{lanes}", n_seqs=lanes, n_slots=max(lanes, wl.n_slots))
    sh = gdn.Shape(**wl.shape_dict())
    C, N, Ch, Hv, dv = sh.n_seqs, sh.n_nodes, sh.channels, sh.n_v_heads, sh.d_v
    dev = torch.device("cuda:0")

    def d(a):
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    st = round_structure(wl, 0)
    slots, parents = d(st["slot_ids"]), d(st["parents"])
    status = torch.zeros(1, dtype=torch.int32, device=dev)
    inst = []
    for layer in range(instances):
        lp, ri = layer_params(wl, layer), round_inputs(wl, layer, 0)
        ba = d(ri["ba"])
        inst.append(dict(x=d(ri["x"]), beta=ba[..., :Hv], alpha=ba[..., Hv:], w=d(lp["conv_w"]),
                         hist=d(lp["conv_hist"]), state=d(lp["state"]), dt=d(lp["dt_bias"]), A=d(lp["A"]),
                         out=torch.empty((C, N, Hv, dv), device=dev),
                         log=torch.empty((C, N, Hv, sh.log_row), device=dev),
                         win=torch.empty((C, N, Ch, 3), device=dev)))

    def launches():
        for b in inst:
            gdn.conv_tree_verify(sh, b["x"], b["w"], b["hist"], b["beta"], b["alpha"], b["dt"], b["A"], b["state"],
                                 slots, parents, out=b["out"], replay_log=b["log"], commit_win=b["win"], status=status)

    launches()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        launches()
    for _ in range(3):
        g.replay()
    torch.cuda.synchronize()
    assert int(status.item()) == 0, "device status bits set"
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    g.replay()
    e1.record()
    torch.cuda.synchronize()
    stamps = np.zeros((MAX_WG, 16), np.uint64)
    assert lib.gdn_timeline_read(stamps.ctypes.data) == 0
    wide = dv == 128 and C * Hv >= 256
    n_verify = (1 if wide else max(dv // 64, 1)) * Hv * C
    s = stamps[:n_verify].astype(np.int64)
    per_us = np.median((s[:, 10] - s[:, 0]) / ((s[:, 13] - s[:, 12]) / 100.0))  # shader cycles per us
    print(f"{wl.name}: {n_verify} verify workgroups, shader clock {per_us / 1e3:.2f} GHz")
    print(f"{'phase':32s} {'median':>7s} {'p10':>7s} {'p90':>7s}  (us, per verify workgroup)")
    prev = s[:, 0]
    for slot, name in PHASES:
        dt = (s[:, slot] - prev) / per_us
        print(f"{name:32s} {np.median(dt):7.2f} {np.percentile(dt, 10):7.2f} {np.percentile(dt, 90):7.2f}")
        prev = s[:, slot]
    span = (s[:, 10] - s[:, 0]) / per_us
    print(f"{'whole body':32s} {np.median(span):7.2f} {np.percentile(span, 10):7.2f} {np.percentile(span, 90):7.2f}")
    arr = (s[:, 11] - s[:, 2]) / per_us
    print(f"{'state product starts, from staging':32s} {np.median(arr):7.2f} {np.percentile(arr, 10):7.2f} "
          f"{np.percentile(arr, 90):7.2f}  (wave 4)")
    # the common clock: every workgroup's start and end against the first start of the launch
    n_window = 0 if (wide and C * Hv >= 512) else C * -(-Ch // (4 * (512 // (8 if N <= 8 else (16 if N <= 16 else 32)))))
    allw = stamps[:n_verify + n_window].astype(np.int64)
    t0 = allw[:, 12].min()
    print(f"{'common clock (us from first start)':36s} {'start p10/p50/p90':>20s} {'end p10/p50/p90':>20s}")
    for name, blk in (("verify workgroups", allw[:n_verify]), ("window workgroups", allw[n_verify:])):
        if len(blk) == 0:
            continue
        st, en = (blk[:, 12] - t0) / 100.0, (blk[:, 13] - t0) / 100.0
        print(f"{name:36s} {np.percentile(st, 10):6.2f} {np.median(st):6.2f} {np.percentile(st, 90):6.2f} "
              f"{np.percentile(en, 10):6.2f} {np.median(en):6.2f} {np.percentile(en, 90):6.2f}  (last {en.max():.2f})")
    print(f"instrumented launch: {e0.elapsed_time(e1) * 1e3 / instances:.2f} us (graph of {instances})")


def main() -> None:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("mode", choices=("build", "run"))
    ap.add_argument("--workload", default="tree-c4-n16")
    ap.add_argument("--instances", type=int, default=64)
    ap.add_argument("--lanes", type=int, default=None, help="this many lanes at the workload's head shape")
    args = ap.parse_args()
    if args.mode == "build":
        build()
    else:
        run(args.workload, args.instances, args.lanes)


if __name__ == "__main__":
    main()
