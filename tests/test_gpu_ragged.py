"""Ragged lanes on the GPU: each lane drafts its own number of nodes (lane_nodes[c]).
Present nodes match the fp64 oracle to the usual bars (conv 1e-5; output, log and
committed state 2e-4; windows and history bit-exact); absent nodes' outputs are never
written (guarded sentinel), their parents are never checked, and the commit accepts only
present nodes."""

import numpy as np
import pytest
import torch

import gated_deltanet_speculative_amd as gdn
from gpu_util import SENTINEL, GpuRound, dev, err_metric, log, oracle_commit, oracle_round
from workloads import synth_case

pytestmark = pytest.mark.gpu

CONV_TOL, REC_TOL = 1e-5, 2e-4

CASES = [
    # name, C, N, P, Hk, Hv, dk, dv, tree, lane node counts
    ("headline-heads", 4, 16, 8, 16, 32, 128, 128, True, [16, 5, 0, 11]),
    ("np32", 3, 32, 5, 2, 4, 64, 32, True, [32, 17, 1]),
    ("chains-d16", 5, 8, 7, 2, 2, 16, 16, False, [8, 3, 0, 1, 6]),
    # C * H_v >= 256 with d_v = 128: the variant whose verify workgroups write the windows
    ("wide", 8, 16, 9, 16, 32, 128, 128, True, [16, 5, 0, 11, 1, 16, 9, 3]),
    ("wide-np32", 4, 32, 5, 4, 64, 64, 128, True, [32, 17, 1, 25]),
    ("wide-windows", 16, 16, 17, 16, 32, 128, 128, True, [16, 5, 0, 11, 1, 16, 9, 3, 2, 14, 16, 7, 8, 0, 12, 6]),
    ("wide-windows-np32", 8, 32, 9, 4, 64, 64, 128, True, [32, 17, 1, 25, 0, 32, 9, 30]),
]


def _case(C, N, P, Hk, Hv, dk, dv, tree, counts, seed):
    case = synth_case(C, N, P, Hk, Hv, dk, dv, seed=seed, tree=tree)
    parents = case["parents"].copy()
    rng = np.random.default_rng(seed)
    for c, n in enumerate(counts):  # absent nodes hold garbage parents: they must not be checked
        parents[c, n:] = rng.choice([99, -7, N], size=N - n)
    case["parents"] = parents
    return case


def _check_lanes(g, ref, counts):
    """Present nodes against the oracle, absent nodes untouched."""
    errs = dict(conv=0.0, out=0.0, log=0.0)
    bufs = [("commit_win", g.commit_win, None), ("out", g.out, REC_TOL), ("log", g.replay_log, REC_TOL)]
    if not g.fused:
        bufs.append(("conv", g.conv_out, CONV_TOL))
    ref_name = {"commit_win": "commit_win", "out": "out", "log": "replay_log", "conv": "conv_out"}
    for c, n in enumerate(counts):
        for name, buf, tol in bufs:
            gv = buf.np()[c]
            assert (gv[n:] == np.float32(SENTINEL)).all(), f"lane {c}: absent nodes of {name} written"
            rv = ref[ref_name[name]][c, :n]
            if tol is None:
                assert np.array_equal(gv[:n], rv.astype(np.float32)), f"lane {c}: commit windows differ"
            elif n:
                e = err_metric(gv[:n], rv)
                assert e <= tol, f"lane {c}: {name} error {e}"
                errs[name] = max(errs[name], e)
    if g.fused:
        assert (g.conv_out.np() == np.float32(SENTINEL)).all()
    assert g.guards_intact()
    return errs


@pytest.mark.parametrize("route", ["split", "fused"])
@pytest.mark.parametrize("name,C,N,P,Hk,Hv,dk,dv,tree,counts", CASES)
def test_ragged_parity_and_commit(name, C, N, P, Hk, Hv, dk, dv, tree, counts, route):
    sh = gdn.Shape(C, N, P, Hk, Hv, dk, dv)
    case = _case(C, N, P, Hk, Hv, dk, dv, tree, counts, seed=100 + N)
    log(f"[ragged] {name} route={route} counts={counts} slots={case['slot_ids'].tolist()}")
    g = GpuRound(sh, case["x"], case["ba"], case["conv_w"], case["conv_hist"], case["state"], case["dt_bias"],
                 case["A"], case["slot_ids"], case["parents"], fused=route == "fused", lane_nodes=counts).verify()
    torch.cuda.synchronize()
    ref = oracle_round(sh, case["x"], case["ba"], case["conv_w"], case["conv_hist"], case["state"], case["dt_bias"],
                       case["A"], case["slot_ids"], case["parents"], lane_nodes=counts)
    assert int(g.status.item()) == 0 and ref["status"] == 0
    errs = _check_lanes(g, ref, counts)
    assert torch.equal(g.state.cpu(), torch.from_numpy(case["state"]))
    # commit the deepest present node of every lane (-1 for an empty lane)
    accept = np.array([n - 1 for n in counts], np.int32)
    g.commit(accept)
    torch.cuda.synchronize()
    assert int(g.status.item()) == 0
    st, pool, hist = oracle_commit(sh, ref, case["slot_ids"], case["parents"], accept, case["state"],
                                   case["conv_hist"], lane_nodes=counts)
    assert st == 0
    gpool, ghist = g.state.cpu().numpy(), g.conv_hist.cpu().numpy()
    slots = case["slot_ids"]
    e_state = err_metric(gpool[slots], pool[slots])
    assert e_state <= REC_TOL, f"committed state error {e_state}"
    assert np.array_equal(ghist[slots], hist[slots].astype(np.float32))
    untouched = np.setdiff1d(np.arange(P), slots[np.asarray(counts) > 0])  # unused slots and empty lanes
    assert np.array_equal(gpool[untouched], case["state"][untouched])
    assert np.array_equal(ghist[untouched], case["conv_hist"][untouched])
    log(f"[ragged] {name}: conv {errs['conv']:.2e} out {errs['out']:.2e} log {errs['log']:.2e} state {e_state:.2e}")


@pytest.mark.parametrize("route", ["split", "fused"])
def test_ragged_count_out_of_range(route):
    name, C, N, P, Hk, Hv, dk, dv, tree, counts = CASES[2]
    counts = list(counts)
    counts[1] = N + 1
    sh = gdn.Shape(C, N, P, Hk, Hv, dk, dv)
    case = _case(C, N, P, Hk, Hv, dk, dv, tree, [min(n, N) for n in counts], seed=7)
    log(f"[ragged] count out of range, route={route}, counts={counts}")
    g = GpuRound(sh, case["x"], case["ba"], case["conv_w"], case["conv_hist"], case["state"], case["dt_bias"],
                 case["A"], case["slot_ids"], case["parents"], fused=route == "fused", lane_nodes=counts).verify()
    torch.cuda.synchronize()
    assert int(g.status.item()) == gdn.STATUS_NODES
    for buf in (g.out, g.replay_log, g.commit_win):
        assert (buf.np()[1] == np.float32(SENTINEL)).all()
        assert not (buf.np()[0] == np.float32(SENTINEL)).any()
    g.commit(np.full(C, 0, np.int32))  # the round's status is set: the commit must change nothing
    torch.cuda.synchronize()
    assert np.array_equal(g.state.cpu().numpy(), case["state"])
    assert np.array_equal(g.conv_hist.cpu().numpy(), case["conv_hist"])


def test_ragged_commit_rejects_an_absent_accept_node():
    name, C, N, P, Hk, Hv, dk, dv, tree, counts = CASES[2]
    sh = gdn.Shape(C, N, P, Hk, Hv, dk, dv)
    case = _case(C, N, P, Hk, Hv, dk, dv, tree, counts, seed=8)
    log("[ragged] accept node past the lane's count")
    g = GpuRound(sh, case["x"], case["ba"], case["conv_w"], case["conv_hist"], case["state"], case["dt_bias"],
                 case["A"], case["slot_ids"], case["parents"], lane_nodes=counts).verify()
    torch.cuda.synchronize()
    assert int(g.status.item()) == 0
    accept = np.array([n - 1 for n in counts], np.int32)
    accept[3] = 1  # lane 3 has one node: node 1 is absent
    g.commit(accept)
    torch.cuda.synchronize()
    assert int(g.status.item()) & gdn.STATUS_ACCEPT
    assert np.array_equal(g.state.cpu().numpy(), case["state"])
    assert np.array_equal(g.conv_hist.cpu().numpy(), case["conv_hist"])
