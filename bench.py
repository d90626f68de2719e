#!/usr/bin/env python3
"""Throughput of the speculative-verify GDN route on one MI355X.

One step = one speculative round over L independent layer instances of the
workload (default: 4 lanes in an 8-slot pool, 16-node random draft trees,
H_k=16, H_v=32, d_k=d_v=128, 8192 conv channels): for every instance the fused
tree conv + verify (or, with --route split, the separate conv step and verify),
then the replay commit of the round's accepted paths for all instances in one
multi-layer launch (or, with --commit per-layer, one commit launch per instance).  All instances share the round's slot ids,
parents, accept nodes and status word, as the layers of one model round do.
L=64 instances (~1.9 GB) keep the working set far above the 256 MB last-level
cache, so every layer reads its inputs from HBM.

value = C*N*L / step time: verified draft tokens per second, each instance
counted as one single-layer verify.  Inputs are resident in HBM before timing.

The JSON line also carries the roofline of the dominant kernel (algorithmic
bytes per launch / mean launch time measured with HIP events on the launch
stream) and the fp64 CPU oracle timed on a bounded sample of the same workload.
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, vendor figure
MFMA_FP32_PEAK_TFLOPS = 157.3  # MI355X dense fp32 matrix, vendor figure


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="tree-c4-n16")
    ap.add_argument("--instances", type=int, default=None,
                    help="independent layer instances per step (default 64; 8 for --mode prefill)")
    ap.add_argument("--rounds", type=int, default=4, help="distinct tree/acceptance draws cycled over steps")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--kernel-reps", type=int, default=20, help="repetitions of each per-kernel timing loop")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="budget of the CPU oracle sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--profile-only", action="store_true", help="skip the CPU oracle and per-kernel loops")
    ap.add_argument("--no-floor", action="store_true",
                    help="skip the dispatch-floor launches (so a kernel trace holds only the kernels' real launches)")
    ap.add_argument("--eager", action="store_true", help="launch every call directly instead of replaying graphs")
    ap.add_argument("--route", choices=("fused", "split"), default="fused",
                    help="fused conv + verify (decode mode: conv + recurrence) call, or the separate calls")
    ap.add_argument("--commit", choices=("layers", "per-layer"), default="layers",
                    help="one multi-layer commit launch per round, or one commit launch per instance")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="after the run, launch 4 plain device copies of this many MiB (counter calibration)")
    ap.add_argument("--ragged", action="store_true",
                    help="verify mode: each round draws every lane's node count uniformly from 1..N (seeded) and "
                         "accepts the lane's last node; throughput counts the present nodes")
    ap.add_argument("--mode", choices=("verify", "decode", "prefill"), default="verify",
                    help="the speculative round (headline metric); the plain decode step of a lane "
                         "without a draft (conv step + one-token recurrence per instance, state in place); "
                         "or a prompt filling the slots (conv step + chunked prefill per instance)")
    ap.add_argument("--prompt", type=int, default=1024, help="--mode prefill: prompt tokens per lane")
    ap.add_argument("--lanes", type=int, default=None,
                    help="verify mode: run the workload's head shape and trees with this many lanes "
                         "(slots = max(lanes, the workload's pool)); the workload is then named <name>-lanes<N>")
    return ap.parse_args()


def algorithmic_bytes(wl, accept_depths, lane_counts=None):
    """Every input read once and every output written once, at the library's layouts (fp32).
    lane_counts: nodes present per lane (ragged lanes; default N each)."""
    C, N, Ch, Hv, dk, dv = wl.n_seqs, wl.n_nodes, wl.channels, wl.n_v_heads, wl.d_k, wl.d_v
    W, R = wl.d_conv - 1, wl.log_row
    n = C * N if lane_counts is None else int(np.sum(lane_counts))  # present nodes of the round
    conv = 4 * Ch * (C * W + n * (1 + 1 + W) + wl.d_conv)
    verify = 4 * (C * Hv * dk * dv + n * Ch + 2 * n * Hv + 2 * Hv + n * Hv * dv + n * Hv * R)
    commit = sum(4 * (2 * Hv * dk * dv + 2 * W * Ch) + a * 4 * Hv * R for a in accept_depths if a > 0)
    # fused: the conv output is neither written nor read back
    return dict(conv=conv, verify=verify, conv_verify=conv + verify - 2 * 4 * n * Ch, commit=commit)


def calibrate_copy(mib, dev):
    """Four plain device copies of `mib` MiB: the counter-calibration reference of a
    rocprofv3 --pmc run (no-op for 0)."""
    if not mib:
        return
    import torch

    n = mib * (1 << 20) // 4
    src = torch.ones(n, device=dev)
    dst = torch.empty(n, device=dev)
    for _ in range(4):
        dst.copy_(src)
    torch.cuda.synchronize()


def decode_bytes(wl):
    """Algorithmic bytes of the plain decode step (one token per lane), every input read
    once and every output written once: conv step = history read + written, token,
    conv output, taps; recurrence = state read + written, conv row, gates, dt/A, output."""
    C, Ch, Hv, dk, dv = wl.n_seqs, wl.channels, wl.n_v_heads, wl.d_k, wl.d_v
    W = wl.d_conv - 1
    conv = 4 * Ch * (C * (W + 1 + 1 + W) + wl.d_conv)
    decode = 4 * (2 * C * Hv * dk * dv + C * Ch + 2 * C * Hv + 2 * Hv + C * Hv * dv)
    # the fused call: the conv output row is neither written nor read back
    return dict(conv_step=conv, decode_step=decode, conv_decode=conv + decode - 2 * 4 * C * Ch)


def prefill_cost(wl, T, chunk=16):
    """Algorithmic flops and bytes of the chunked prefill over T tokens per lane.  Flops: the
    dense products of the chunked form per token and value head -- [K; Q] S0 (4 d_k d_v), the
    state update K^T W D (2 d_k d_v), the Gram products (4 B d_k) and D = T rhs, Cq D
    (4 B d_v) with B = 16-token chunks.  Bytes: the conv output rows, gates and outputs once,
    the state read and written once."""
    C, Ch, Hv, dk, dv = wl.n_seqs, wl.channels, wl.n_v_heads, wl.d_k, wl.d_v
    flops = C * T * Hv * (6 * dk * dv + 4 * chunk * (dk + dv))
    bytes_ = 4 * (C * T * Ch + 2 * C * T * Hv + C * T * Hv * dv + 2 * C * Hv * dk * dv + 2 * Hv)
    conv = 4 * Ch * (2 * C * T + 2 * 3 * C + wl.d_conv)  # tokens in, conv out, history in + out, taps
    return dict(flops=flops, bytes=bytes_, conv_bytes=conv)


def percentiles(xs):
    """p10, median and p90 of a list of timings, rounded."""
    return [round(float(v), 4) for v in np.percentile(np.asarray(xs, dtype=np.float64), [10, 50, 90])]


def measured_traffic(workload, kernel):
    """Fabric bytes per launch of `kernel` from the committed counter summary
    (profiles/traffic_<workload>.json: FETCH_SIZE + WRITE_SIZE, copy-calibrated), or
    None when there is none or the kernel's source changed since it was measured."""
    from gated_deltanet_speculative_amd.rocprof_summary import source_sha256

    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "profiles", f"traffic_{workload}.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path)).get("kernels", {}).get(kernel)
    if not rec or rec.get("source_sha256") != source_sha256(kernel):
        return None
    return int(round(rec["read_bytes"] + rec["write_bytes"]))


def host_description():
    """The host the CPU baseline ran on: logical CPUs, those this process may use, the CPU
    model, and the BLAS libraries numpy loaded with the thread count each uses inside the
    baseline (limited to one)."""
    from threadpoolctl import threadpool_info, threadpool_limits

    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    with threadpool_limits(limits=1):
        blas = [dict(library=i.get("internal_api"), threads=i.get("num_threads")) for i in threadpool_info()
                if i.get("user_api") == "blas"]
    return dict(host_cpu_count=os.cpu_count(), host_cpus_usable=len(os.sched_getaffinity(0)), cpu_model=model,
                blas_in_baseline=blas)


def _oracle_round_seconds(wl, layer, seed):
    """Seconds of one single-layer round (conv + verify + commit) of the fp64 oracle."""
    from oracle import gdn_oracle as O
    from workloads import layer_params, round_inputs, round_structure

    st = round_structure(wl, 0, seed)
    lp, ri = layer_params(wl, layer, seed), round_inputs(wl, layer, 0, seed)
    t0 = time.perf_counter()
    r = O.verify_round(ri["x"], ri["ba"], lp["conv_w"], lp["conv_hist"], lp["state"], lp["dt_bias"], lp["A"],
                       st["slot_ids"], st["parents"], wl.n_k_heads)
    pool, hist = lp["state"].astype(np.float64), lp["conv_hist"].astype(np.float64)
    O.replay_commit(r["replay_log"], r["commit_win"], st["slot_ids"], st["parents"], st["accept_node"], pool, hist)
    return time.perf_counter() - t0


def cpu_baseline(wl, seconds, seed):
    """The fp64 oracle on single-layer instances of the workload, until `seconds` of CPU work,
    and on one layer of the single-lane grouped chain (median of 3 after a warm-up)."""
    from threadpoolctl import threadpool_limits

    from workloads import WORKLOADS

    done, t_used = 0, 0.0
    with threadpool_limits(limits=1):
        while t_used < seconds:
            t_used += _oracle_round_seconds(wl, done, seed)
            done += 1
        c1 = WORKLOADS["grouped-chain-n8"]
        _oracle_round_seconds(c1, 0, seed)
        t1 = float(np.median([_oracle_round_seconds(c1, k, seed) for k in range(3)]))
    return dict(value=wl.n_seqs * wl.n_nodes * done / t_used, unit="verify tokens/s", cores=1, kind="oracle",
                sample=f"{done} single-layer rounds (conv+verify+commit) of {wl.name}, fp64 numpy, 1 BLAS thread, "
                       f"{t_used:.1f} s",
                grouped_chain_n8=dict(value=round(c1.n_seqs * c1.n_nodes / t1, 1), unit="verify tokens/s",
                                      sample="one layer (1 lane, 8-token chain, H_k 16, H_v 32, d 128; "
                                             "conv+verify+commit), median of 3 after a warm-up",
                                      seconds=round(t1, 4)),
                **host_description())


def cpu_baseline_decode(wl, seconds, seed):
    """The fp64 oracle's plain decode step (conv step, then the one-token recurrence) on one
    layer instance of the workload, repeated on its in-place history and state until
    `seconds` of CPU work."""
    from threadpoolctl import threadpool_limits

    from oracle import gdn_oracle as O
    from workloads import layer_params, round_inputs, round_structure

    C, Ch, Hv, dv = wl.n_seqs, wl.channels, wl.n_v_heads, wl.d_v
    slots = round_structure(wl, 0, seed)["slot_ids"]
    lp, ri = layer_params(wl, 0, seed), round_inputs(wl, 0, 0, seed)
    ba = ri["ba"][:, 0]
    hist, pool = lp["conv_hist"].astype(np.float64), lp["state"].astype(np.float64)
    conv_out, out = np.zeros((C, 1, Ch)), np.zeros((C, Hv, dv))
    done, t_used = 0, 0.0
    with threadpool_limits(limits=1):
        while t_used < seconds:
            t0 = time.perf_counter()
            O.conv_step(ri["x"][:, :1], lp["conv_w"], hist, slots, conv_out)
            O.decode_step(conv_out[:, 0], ba[:, :Hv], ba[:, Hv:], lp["dt_bias"], lp["A"], pool, slots, wl.n_k_heads,
                          out)
            t_used += time.perf_counter() - t0
            done += 1
    return dict(value=C * done / t_used, unit="decode tokens/s", cores=1, kind="oracle",
                sample=f"{done} single-layer decode steps (conv step + recurrence) of {wl.name}, fp64 numpy, "
                       f"1 BLAS thread, {t_used:.1f} s", **host_description())


def cpu_baseline_prefill(wl, seconds, seed, tokens=32):
    """The fp64 oracle's prompt path (conv step over the prompt, then the token-by-token
    recurrence) on `tokens`-token prompts of the workload's lanes, until `seconds` of CPU
    work (one layer instance, its history and state carried over from prompt to prompt):
    the oracle's cost is linear in the prompt length, so a short prompt measures its rate."""
    from threadpoolctl import threadpool_limits

    from oracle import gdn_oracle as O
    from workloads import layer_params, round_structure

    C, Ch, Hv, dv = wl.n_seqs, wl.channels, wl.n_v_heads, wl.d_v
    slots = round_structure(wl, 0, seed)["slot_ids"]
    lp = layer_params(wl, 0, seed)
    rng = np.random.default_rng([seed, 7])
    x = rng.standard_normal((C, tokens, Ch)).astype(np.float32)
    ba = rng.standard_normal((C, tokens, 2 * Hv)).astype(np.float32)
    hist, pool = lp["conv_hist"].astype(np.float64), lp["state"].astype(np.float64)
    conv_out, out = np.zeros((C, tokens, Ch)), np.zeros((C, tokens, Hv, dv))
    done, t_used = 0, 0.0
    with threadpool_limits(limits=1):
        while t_used < seconds:
            t0 = time.perf_counter()
            O.conv_step(x, lp["conv_w"], hist, slots, conv_out)
            O.prefill(conv_out, ba[..., :Hv], ba[..., Hv:], lp["dt_bias"], lp["A"], pool, slots, wl.n_k_heads, out)
            t_used += time.perf_counter() - t0
            done += 1
    return dict(value=C * tokens * done / t_used, unit="prompt tokens/s", cores=1, kind="oracle",
                sample=f"{done} single-layer {tokens}-token prompts of {wl.name} (conv step + recurrence), "
                       f"fp64 numpy, 1 BLAS thread, {t_used:.1f} s", **host_description())


def copy_reference(nbytes, dev):
    """A plain device copy moving `nbytes` (half read, half written): 64 back-to-back copies of
    distinct buffers replayed as a graph; microseconds per copy and the rate."""
    import torch

    nb = int(nbytes) // 8
    srcs = [torch.ones(nb, dtype=torch.float32, device=dev) for _ in range(64)]
    dsts = [torch.empty(nb, dtype=torch.float32, device=dev) for _ in range(64)]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for d_, s_ in zip(dsts, srcs):
            d_.copy_(s_)
    g.replay()
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record()
    for _ in range(5):
        g.replay()
    ev1.record()
    torch.cuda.synchronize()
    copy_us = ev0.elapsed_time(ev1) * 1e3 / (5 * 64)
    return dict(bytes=8 * nb, us=round(copy_us, 3), gbs=round(8 * nb / (copy_us * 1e-6) / 1e9, 1),
                what="torch device copy_ of the same byte count, 64 buffers, graph replay")


def decode_main(args):
    """The plain decode step at the workload's head shape: one token per lane, for every
    layer instance the conv step (history written in place) and the one-token recurrence
    (state updated in place), in one fused launch (--route split: the two calls).
    value = C * L / step time."""
    import torch

    import gated_deltanet_speculative_amd as gdn
    from workloads import WORKLOADS, layer_params, round_inputs, round_structure

    wl = WORKLOADS[args.workload]
    sh = gdn.Shape(**dict(wl.shape_dict(), n_nodes=1))
    C, P, Ch, Hv, dk, dv = sh.n_seqs, sh.n_slots, sh.channels, sh.n_v_heads, sh.d_k, sh.d_v
    L = args.instances
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    def d(a):
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    t_gen = time.time()
    slot_ids = d(round_structure(wl, 0, args.seed)["slot_ids"])
    status = torch.zeros(1, dtype=torch.int32, device=dev)
    sync = torch.zeros((C, wl.n_k_heads, gdn.SYNC_STRIDE), dtype=torch.int32, device=dev)  # the fused call's counters
    inst = []
    for l in range(L):
        lp, ri = layer_params(wl, l, args.seed), round_inputs(wl, l, 0, args.seed)
        ba = d(ri["ba"][:, 0])
        inst.append(dict(x=d(ri["x"][:, :1]), beta=ba[:, :Hv], alpha=ba[:, Hv:], conv_w=d(lp["conv_w"]),
                         conv_hist=d(lp["conv_hist"]), state=d(lp["state"]), dt_bias=d(lp["dt_bias"]), A=d(lp["A"]),
                         qkv=torch.empty((C, 1, Ch), device=dev), out=torch.empty((C, Hv, dv), device=dev)))
    torch.cuda.synchronize()
    t_gen = time.time() - t_gen

    def conv(b):
        gdn.conv_step(sh, b["x"], b["conv_w"], b["conv_hist"], slot_ids, status, conv_out=b["qkv"])

    def rec(b):
        gdn.decode_step(sh, b["qkv"][:, 0], b["beta"], b["alpha"], b["dt_bias"], b["A"], b["state"], slot_ids,
                        status, out=b["out"])

    def fused(b):
        gdn.conv_decode_step(sh, b["x"][:, 0], b["conv_w"], b["conv_hist"], b["beta"], b["alpha"], b["dt_bias"],
                             b["A"], b["state"], slot_ids, sync, status, out=b["out"])

    def step():
        for b in inst:
            if args.route == "fused":
                fused(b)
            else:
                conv(b)
                rec(b)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    assert int(status.item()) == 0, "device status bits set"

    def timed_graph(fn, reps):
        run = fn
        if not args.eager:
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                fn()
            run = g.replay
        run()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            run()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps  # ms per replay

    ms_step = timed_graph(step, args.steps)
    kern = {}
    if not args.profile_only:
        if args.route == "fused":
            kern["conv_decode"] = timed_graph(lambda: [fused(b) for b in inst], args.kernel_reps) * 1e3 / L
        else:
            kern["conv_step"] = timed_graph(lambda: [conv(b) for b in inst], args.kernel_reps) * 1e3 / L
            kern["decode_step"] = timed_graph(lambda: [rec(b) for b in inst], args.kernel_reps) * 1e3 / L
    assert int(status.item()) == 0, "device status bits set"
    assert not sync.any(), "sync counters left non-zero"
    calibrate_copy(args.calibrate_copy, dev)
    kb = decode_bytes(wl)
    # split: the recurrence moves 14x the conv step's bytes; both launches are near the dispatch
    # floor, so which one times longer over a few replays is noise, and the roofline stays with
    # the recurrence
    dom = "conv_decode" if args.route == "fused" else "decode_step"
    # context for the dominant kernel: a plain copy of its bytes (mostly the state block read and written)
    copy_ref = None if args.profile_only else copy_reference(kb[dom], dev)
    roofline = None
    if kern:
        achieved = kb[dom] / (kern[dom] * 1e-6) / 1e9
        traffic_wl = wl.name + ("-decode" if args.route == "fused" else "-decode-split")
        roofline = dict(bound="hbm", kernel=dom, achieved=round(achieved, 1), peak=HBM_PEAK_GBS, unit="GB/s",
                        frac=round(achieved / HBM_PEAK_GBS, 4), traffic=measured_traffic(traffic_wl, dom),
                        bytes_per_launch=int(kb[dom]), us_per_launch=round(kern[dom], 3))
    line = {
        "metric": "GDN plain decode tokens/s (one token per lane, state committed in place)",
        "value": round(C * L / (ms_step * 1e-3), 1),
        "unit": "decode tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "timing": ("eager launches" if args.eager else "HIP graph replay of the whole step")
                  + "; inputs resident in HBM",
        "config": {"workload": wl.name + "-decode", "lanes": C, "tokens_per_lane": 1, "slots": P,
                   "k_heads": wl.n_k_heads, "v_heads": Hv, "d_k": dk, "d_v": dv, "conv_channels": Ch,
                   "layer_instances": L,
                   "step": ("fused conv step + one-token recurrence per instance" if args.route == "fused"
                            else "conv step + one-token recurrence per instance")},
        "step_gbs": round(L * (kb["conv_decode"] if args.route == "fused" else kb["conv_step"] + kb["decode_step"])
                          / (ms_step * 1e-3) / 1e9, 1),
        "kernel_us": {k: round(v, 3) for k, v in kern.items()},
        "kernel_gbs": {k: round(kb[k] / (kern[k] * 1e-6) / 1e9, 1) for k in kern},
        "copy_same_bytes": copy_ref,
        "roofline": roofline,
        "cpu_baseline": (None if args.no_cpu_baseline or args.profile_only
                         else cpu_baseline_decode(wl, args.cpu_seconds, args.seed)),
        "setup_s": round(t_gen, 1),
    }
    print(json.dumps(line), flush=True)


def prefill_main(args):
    """A prompt of T tokens per lane filling the slots at the workload's head shape: for every
    layer instance the chain conv step over the prompt (history written in place), then the
    chunked prefill (state updated in place).  value = C * T * L / step time."""
    import torch

    import gated_deltanet_speculative_amd as gdn
    from workloads import WORKLOADS, layer_params, round_structure

    wl = WORKLOADS[args.workload]
    T, L = args.prompt, args.instances
    sh = gdn.Shape(**dict(wl.shape_dict(), n_nodes=T))
    C, P, Ch, Hv, dk, dv = sh.n_seqs, sh.n_slots, sh.channels, sh.n_v_heads, sh.d_k, sh.d_v
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    def d(a):
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    t_gen = time.time()
    gen = torch.Generator(device=dev)
    slot_ids = d(round_structure(wl, 0, args.seed)["slot_ids"])
    status = torch.zeros(1, dtype=torch.int32, device=dev)
    # one workspace for every instance: their prefills run one after another on the stream
    workspace = torch.empty(gdn.prefill_workspace_size(sh) // 4, dtype=torch.float32, device=dev)
    inst = []
    for l in range(L):
        lp = layer_params(wl, l, args.seed)
        gen.manual_seed(args.seed * 1000003 + l)  # prompt tokens ~ N(0,1), b|a logits ~ N(0,1)
        ba = torch.randn((C, T, 2 * Hv), generator=gen, device=dev)
        inst.append(dict(x=torch.randn((C, T, Ch), generator=gen, device=dev), beta=ba[..., :Hv], alpha=ba[..., Hv:],
                         conv_w=d(lp["conv_w"]), conv_hist=d(lp["conv_hist"]), state=d(lp["state"]),
                         dt_bias=d(lp["dt_bias"]), A=d(lp["A"]), qkv=torch.empty((C, T, Ch), device=dev),
                         out=torch.empty((C, T, Hv, dv), device=dev)))
    torch.cuda.synchronize()
    t_gen = time.time() - t_gen

    def conv(b):
        gdn.conv_step(sh, b["x"], b["conv_w"], b["conv_hist"], slot_ids, status, conv_out=b["qkv"])

    def rec(b):
        gdn.prefill(sh, b["qkv"], b["beta"], b["alpha"], b["dt_bias"], b["A"], b["state"], slot_ids, status,
                    out=b["out"], workspace=workspace)

    def step():
        for b in inst:
            conv(b)
            rec(b)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    assert int(status.item()) == 0, "device status bits set"

    def timed(fn, reps):
        run = fn
        if not args.eager:
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                fn()
            run = g.replay
        run()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            run()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps  # ms per run

    ms_step = timed(step, args.steps)
    kern = {}
    if not args.profile_only:
        kern["conv_step"] = timed(lambda: [conv(b) for b in inst], args.kernel_reps) * 1e3 / L
        kern["prefill"] = timed(lambda: [rec(b) for b in inst], args.kernel_reps) * 1e3 / L
    assert int(status.item()) == 0, "device status bits set"
    calibrate_copy(args.calibrate_copy, dev)
    cost = prefill_cost(wl, T)
    roofline = None
    if kern:
        tflops = cost["flops"] / (kern["prefill"] * 1e-6) / 1e12
        parts = [measured_traffic(wl.name + "-prefill", k) for k in ("prefill_prep", "prefill_state")]
        roofline = dict(bound="mfma", kernel="prefill (prefill_prep + prefill_state launches of one call)",
                        achieved=round(tflops, 2), peak=MFMA_FP32_PEAK_TFLOPS, unit="TFLOP/s",
                        frac=round(tflops / MFMA_FP32_PEAK_TFLOPS, 4),
                        traffic=None if None in parts else sum(parts), flops_per_launch=cost["flops"],
                        us_per_launch=round(kern["prefill"], 3))
    line = {
        "metric": "GDN prefill tokens/s (prompt filling the slots)",
        "value": round(C * T * L / (ms_step * 1e-3), 1),
        "unit": "prompt tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "timing": ("eager launches" if args.eager else "HIP graph replay of the whole step")
                  + "; inputs resident in HBM",
        "config": {"workload": wl.name + "-prefill", "lanes": C, "prompt_tokens": T, "slots": P,
                   "k_heads": wl.n_k_heads, "v_heads": Hv, "d_k": dk, "d_v": dv, "conv_channels": Ch,
                   "layer_instances": L, "step": "conv step over the prompt + chunked prefill per instance"},
        "kernel_us": {k: round(v, 3) for k, v in kern.items()},
        "kernel_gbs": ({"conv_step": round(cost["conv_bytes"] / (kern["conv_step"] * 1e-6) / 1e9, 1),
                        "prefill": round(cost["bytes"] / (kern["prefill"] * 1e-6) / 1e9, 1)} if kern else {}),
        "roofline": roofline,
        "cpu_baseline": (None if args.no_cpu_baseline or args.profile_only
                         else cpu_baseline_prefill(wl, args.cpu_seconds, args.seed)),
        "setup_s": round(t_gen, 1),
    }
    print(json.dumps(line), flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); the route needs no collective, "
              "so multi-GPU throughput is the per-GPU figure times the lane-sharded GPU count.", file=sys.stderr)
        sys.exit(2)
    if args.instances is None:
        args.instances = 8 if args.mode == "prefill" else 64
    if args.mode == "decode":
        decode_main(args)
        return
    if args.mode == "prefill":
        prefill_main(args)
        return

    import torch

    import gated_deltanet_speculative_amd as gdn
    from workloads import WORKLOADS, layer_params, path_to_root, round_inputs, round_structure

    wl = WORKLOADS[args.workload]
    if args.lanes is not None:
        import dataclasses

        wl = dataclasses.replace(wl, name=f"{wl.name}-lanes{args.lanes}", n_seqs=args.lanes,
                                 n_slots=max(args.lanes, wl.n_slots))
    sh = gdn.Shape(**wl.shape_dict())
    C, N, P, Ch, Hv, dk, dv = sh.n_seqs, sh.n_nodes, sh.n_slots, sh.channels, sh.n_v_heads, sh.d_k, sh.d_v
    L = args.instances
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    def d(a):
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    t_gen = time.time()
    rounds = [round_structure(wl, r, args.seed) for r in range(args.rounds)]
    slot_ids = d(rounds[0]["slot_ids"])
    if args.ragged:  # per-lane node counts, and each lane accepts its last present node
        for r, rd in enumerate(rounds):
            rd["lane_nodes"] = np.random.default_rng([args.seed, 77, r]).integers(1, N + 1, size=C).astype(np.int32)
            rd["accept_node"] = rd["lane_nodes"] - 1
    parents = [d(r["parents"]) for r in rounds]
    accepts = [d(r["accept_node"]) for r in rounds]
    counts = [d(r["lane_nodes"]) if args.ragged else None for r in rounds]
    depths = [[len(path_to_root(r["parents"][c], int(e))) if e >= 0 else 0 for c, e in enumerate(r["accept_node"])]
              for r in rounds]
    status = torch.zeros(1, dtype=torch.int32, device=dev)  # the round's status word, shared by every layer
    inst = []
    for l in range(L):
        lp, ri = layer_params(wl, l, args.seed), round_inputs(wl, l, 0, args.seed)
        ba = d(ri["ba"])
        inst.append(dict(
            x=d(ri["x"]), ba=ba, beta=ba[..., :Hv], alpha=ba[..., Hv:], conv_w=d(lp["conv_w"]),
            conv_hist=d(lp["conv_hist"]), state=d(lp["state"]), dt_bias=d(lp["dt_bias"]), A=d(lp["A"]),
            conv_out=torch.empty((C, N, Ch), device=dev), commit_win=torch.empty((C, N, Ch, 3), device=dev),
            out=torch.empty((C, N, Hv, dv), device=dev), log=torch.empty((C, N, Hv, sh.log_row), device=dev),
        ))
    torch.cuda.synchronize()
    t_gen = time.time() - t_gen

    def conv(b, r):
        gdn.conv_tree_step(sh, b["x"], b["conv_w"], b["conv_hist"], slot_ids, parents[r], conv_out=b["conv_out"],
                           commit_win=b["commit_win"], status=status, lane_nodes=counts[r])

    def verify(b, r):
        gdn.tree_verify(sh, b["conv_out"], b["beta"], b["alpha"], b["dt_bias"], b["A"], b["state"], slot_ids,
                        parents[r], out=b["out"], replay_log=b["log"], status=status, lane_nodes=counts[r])

    def conv_verify(b, r):
        gdn.conv_tree_verify(sh, b["x"], b["conv_w"], b["conv_hist"], b["beta"], b["alpha"], b["dt_bias"], b["A"],
                             b["state"], slot_ids, parents[r], out=b["out"], replay_log=b["log"],
                             commit_win=b["commit_win"], status=status, lane_nodes=counts[r])

    def commit(b, r):
        gdn.replay_commit(sh, b["log"], b["commit_win"], slot_ids, parents[r], accepts[r], b["state"], b["conv_hist"],
                          status, lane_nodes=counts[r])

    if L > gdn.MAX_LAYERS and args.commit == "layers":
        raise SystemExit(f"--instances {L} exceeds the {gdn.MAX_LAYERS} layers of one multi-layer commit")
    layer_bufs = {k: [b[k] for b in inst] for k in ("log", "commit_win", "state", "conv_hist")}

    def commit_layers(r):
        gdn.replay_commit_layers(sh, layer_bufs["log"], layer_bufs["commit_win"], slot_ids, parents[r], accepts[r],
                                 layer_bufs["state"], layer_bufs["conv_hist"], status, lane_nodes=counts[r])

    def step(r):
        for b in inst:
            if args.route == "fused":
                conv_verify(b, r)
            else:
                conv(b, r)
                verify(b, r)
        if args.commit == "layers":
            commit_layers(r)
        else:
            for b in inst:
                commit(b, r)

    # Warm up eagerly (also runs every kernel's one-time setup), then capture one HIP
    # graph per round draw: a decode loop launches a whole round as one graph replay,
    # so the timed region measures the GPU, not per-call Python launch overhead.
    for k in range(args.warmup):
        step(k % args.rounds)
    torch.cuda.synchronize()
    assert int(status.item()) == 0, "device status bits set"

    def capture(fn):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            fn()
        return g

    if args.eager:
        graphs = [type("Eager", (), {"replay": (lambda self, r=r: step(r))})() for r in range(args.rounds)]
    else:
        graphs = [capture(lambda r=r: step(r)) for r in range(args.rounds)]
    for r in range(args.rounds):
        graphs[r].replay()
    torch.cuda.synchronize()

    # K steps back to back; an event between consecutive steps gives each step's own time
    # (events only record, they add no synchronisation)
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    evs[0].record()
    for k in range(args.steps):
        graphs[k % args.rounds].replay()
        evs[k + 1].record()
    torch.cuda.synchronize()
    ms_step = evs[0].elapsed_time(evs[-1]) / args.steps
    step_ms = [evs[k].elapsed_time(evs[k + 1]) for k in range(args.steps)]
    assert int(status.item()) == 0, "device status bits set"
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    # per-kernel mean time per layer instance: each kernel alone over the L instances (one
    # graph of L back-to-back launches, or of one multi-layer commit launch), HIP events
    # on the stream the graph runs on
    kern, kern_pct, cold_us, copy_ref, floor = {}, {}, {}, None, None
    ab0 = algorithmic_bytes(wl, [1] * C, rounds[0].get("lane_nodes"))
    kernel_bytes_est = {"conv_tree_verify": ab0["conv_verify"], "tree_verify": ab0["verify"]}
    if not args.profile_only:
        if args.route == "fused":
            timed = [("conv_tree_verify", lambda: [conv_verify(b, 0) for b in inst])]
        else:
            timed = [("conv_tree_step", lambda: [conv(b, 0) for b in inst]),
                     ("tree_verify", lambda: [verify(b, 0) for b in inst])]
        # the multi-layer commit is one launch: 8 of them per graph, so that the gap between
        # graph replays is not charged to a single kernel
        timed.append(("replay_commit", (lambda: [commit_layers(0) for _ in range(8)]) if args.commit == "layers"
                      else (lambda: [commit(b, 0) for b in inst])))
        for name, fn in timed:
            g = capture(fn)
            g.replay()
            torch.cuda.synchronize()
            kev = [torch.cuda.Event(enable_timing=True) for _ in range(args.kernel_reps + 1)]
            kev[0].record()
            for rep in range(args.kernel_reps):
                g.replay()
                kev[rep + 1].record()
            torch.cuda.synchronize()
            per = L * (8 if (name == "replay_commit" and args.commit == "layers") else 1)  # layers per replay
            kern[name] = kev[0].elapsed_time(kev[-1]) * 1e3 / (args.kernel_reps * per)  # us per layer instance
            kern_pct[name] = percentiles([kev[r].elapsed_time(kev[r + 1]) * 1e3 / per for r in range(args.kernel_reps)])
        # one call each right after a 1 GiB device write has flushed the caches (eager
        # launches; the write is still running while the call is enqueued, so the host's
        # launch latency is not in the measurement)
        flush = torch.empty(1 << 28, dtype=torch.float32, device=dev)
        for name, fn in timed:
            one = {"conv_tree_verify": lambda: conv_verify(inst[0], 0), "conv_tree_step": lambda: conv(inst[0], 0),
                   "tree_verify": lambda: verify(inst[0], 0), "replay_commit": lambda: commit(inst[0], 0)}[name]
            one()  # the first launch of a kernel in the process also loads it: not timed
            torch.cuda.synchronize()
            flush.fill_(1.0)
            ev0.record()
            one()
            ev1.record()
            torch.cuda.synchronize()
            cold_us[name] = ev0.elapsed_time(ev1) * 1e3
        del flush
        # context for the dominant kernel's fraction: a plain device copy moving the same
        # number of bytes (read + write), 64 back-to-back copies of distinct buffers replayed
        # as a graph, and an empty graph replay's cost per launch of a one-kernel graph
        copy_ref = copy_reference(kernel_bytes_est["conv_tree_verify" if args.route == "fused" else "tree_verify"], dev)
    if not args.profile_only and not args.no_floor:
        # the dispatch floor on this machine: 64 launches of an empty one-workgroup kernel (torch's
        # clock spin for 0 cycles), and 64 launches of the fused kernel's own grid with every lane
        # a padding lane (its workgroups issue their slot-independent loads and return)
        g = capture(lambda: [torch.cuda._sleep(0) for _ in range(64)])
        g.replay()
        torch.cuda.synchronize()
        ev0.record()
        for _ in range(5):
            g.replay()
        ev1.record()
        torch.cuda.synchronize()
        floor = dict(empty_kernel_us=round(ev0.elapsed_time(ev1) * 1e3 / (5 * 64), 3))
        if args.route == "fused":
            pad = torch.full((C,), -1, dtype=torch.int32, device=dev)
            g = capture(lambda: [gdn.conv_tree_verify(sh, b["x"], b["conv_w"], b["conv_hist"], b["beta"], b["alpha"],
                                                      b["dt_bias"], b["A"], b["state"], pad, parents[0], out=b["out"],
                                                      replay_log=b["log"], commit_win=b["commit_win"], status=status,
                                                      lane_nodes=counts[0]) for b in inst])
            g.replay()
            torch.cuda.synchronize()
            ev0.record()
            for _ in range(5):
                g.replay()
            ev1.record()
            torch.cuda.synchronize()
            floor["padding_lanes_same_grid_us"] = round(ev0.elapsed_time(ev1) * 1e3 / (5 * L), 3)
        floor["what"] = ("per launch in graph replays of back-to-back launches: an empty one-workgroup kernel, and "
                         "the fused launch with every lane a padding lane (same grid; each workgroup issues its "
                         "slot-independent loads, then returns)")
        del g

    calibrate_copy(args.calibrate_copy, dev)

    mean_depths = np.mean([np.mean(dd) for dd in depths]) if depths else 0.0
    # per-kernel times are taken on round 0: with ragged lanes its node counts set the bytes
    ab = algorithmic_bytes(wl, [int(round(mean_depths))] * C, rounds[0].get("lane_nodes"))
    ab_rounds = [algorithmic_bytes(wl, dd, rd.get("lane_nodes")) for dd, rd in zip(depths, rounds)]
    commit_bytes = float(np.mean([a["commit"] for a in ab_rounds]))  # a step's commit: the rounds cycle
    # the per-kernel loop times every kernel on round 0's trees and accepted paths
    kernel_bytes = {"conv_tree_step": ab["conv"], "tree_verify": ab["verify"], "conv_tree_verify": ab["conv_verify"],
                    "replay_commit": ab_rounds[0]["commit"]}
    roofline = None
    if kern:
        dom = max(kern, key=lambda k: kern[k])
        bytes_per = kernel_bytes[dom]
        layers_per_launch = L if (dom == "replay_commit" and args.commit == "layers") else 1
        achieved = bytes_per / (kern[dom] * 1e-6) / 1e9
        traffic = measured_traffic(wl.name + ("-split" if args.route == "split" else ""), dom)
        roofline = dict(bound="hbm", kernel=dom, achieved=round(achieved, 1), peak=HBM_PEAK_GBS, unit="GB/s",
                        frac=round(achieved / HBM_PEAK_GBS, 4), traffic=traffic,
                        bytes_per_launch=int(bytes_per * layers_per_launch),
                        us_per_launch=round(kern[dom] * layers_per_launch, 3))

    cpu = None
    if not args.no_cpu_baseline and not args.profile_only:
        cpu = cpu_baseline(wl, args.cpu_seconds, args.seed)

    present = [int(np.sum(rd["lane_nodes"])) if args.ragged else C * N for rd in rounds]
    tokens = float(np.mean(present)) * L  # verified tokens per step (rounds cycle over the steps)
    kv = [(a["conv_verify"] if args.route == "fused" else a["conv"] + a["verify"]) for a in ab_rounds]
    step_bytes = L * float(np.mean(kv)) + L * commit_bytes
    line = {
        "metric": "GDN verify tokens/s (C=4, 16-node trees, d=128); achieved HBM GB/s vs peak",
        "value": round(tokens / (ms_step * 1e-3), 1),
        "unit": "verify tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "timing": "HIP graph replay of the whole step; inputs resident in HBM",
        "config": {"workload": wl.name, "lanes": C, "nodes": N, "slots": P, "k_heads": wl.n_k_heads,
                   "v_heads": Hv, "d_k": dk, "d_v": dv, "conv_channels": Ch, "layer_instances": L,
                   "step": ("fused conv+verify" if args.route == "fused" else "conv step + verify")
                           + " per instance, then " + ("one multi-layer commit" if args.commit == "layers"
                                                      else "commit per instance"),
                   **({"ragged": "lane node counts uniform in 1..N, mean "
                                 + f"{np.mean(present) / C:.2f} per lane"} if args.ragged else {})},
        "step_gbs": round(step_bytes / (ms_step * 1e-3) / 1e9, 1),
        "step_ms_p10_p50_p90": percentiles(step_ms),
        "kernel_us": {k: round(v, 3) for k, v in kern.items()},
        "kernel_us_p10_p50_p90": kern_pct,
        "kernel_cold_call_us": {k: round(v, 2) for k, v in cold_us.items()},
        "copy_same_bytes": copy_ref,
        "dispatch_floor": floor,
        "kernel_gbs": {k: round(kernel_bytes[k] / (kern[k] * 1e-6) / 1e9, 1) for k in kern},
        "verify_only_tokens_per_s": (round(present[0] / (sum(v for k, v in kern.items() if k != "replay_commit")
                                                         * 1e-6), 1) if kern else None),
        "roofline": roofline,
        "cpu_baseline": cpu,
        "setup_s": round(t_gen, 1),
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
