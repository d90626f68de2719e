"""GPU parity: the HIP route through the C ABI against the fp64 oracle, element by element.

Bars: commit windows, committed conv history, slot mapping and untouched pools
bit-exact; conv output within 1e-5 and recurrence output / replay log / committed
state within 2e-4 of max|g - r| / max(1, |r|)."""

import numpy as np
import pytest
import torch

import gated_deltanet_speculative_amd as gdn
from gpu_util import (SENTINEL, GpuRound, compare_verify, dev, err_metric, log, oracle_commit, oracle_round)
from workloads import WORKLOADS, layer_params, round_inputs, round_structure, synth_case

pytestmark = pytest.mark.gpu

REC_TOL = 2e-4


def _shape(C, N, P, Hk, Hv, dk, dv):
    return gdn.Shape(C, N, P, Hk, Hv, dk, dv)


ROUTES = ["split", "fused"]


def _run_case(sh, case, accept=None, lanes=None, route="split"):
    """Verify on the GPU (separate conv + verify calls, or the fused call) and in the oracle;
    returns both sides."""
    g = GpuRound(sh, case["x"], case["ba"], case["conv_w"], case["conv_hist"], case["state"], case["dt_bias"],
                 case["A"], case["slot_ids"], case["parents"], fused=route == "fused").verify()
    torch.cuda.synchronize()
    sel = slice(None) if lanes is None else np.asarray(lanes)
    ref = oracle_round(sh, case["x"][sel], case["ba"][sel], case["conv_w"], case["conv_hist"], case["state"],
                       case["dt_bias"], case["A"], case["slot_ids"][sel], case["parents"][sel])
    return g, ref, sel


@pytest.mark.parametrize("route", ROUTES)
@pytest.mark.parametrize("name,layer,lanes", [
    ("tiny-chain", 0, None),
    ("grouped-chain-n8", 0, None),
    ("tree-c4-n16", 0, None),
    ("chains-c5-n8-l48", 0, None),
    ("chains-c5-n8-l48", 47, None),
    ("stress-c64-n32-l48", 0, [0, 17, 40, 63]),
])
def test_workload_parity(name, layer, lanes, route):
    wl = WORKLOADS[name]
    sh = gdn.Shape(**wl.shape_dict())
    log(f"[parity] {name} layer={layer} lanes={lanes} route={route} shape={tuple(sh)}")
    case = dict(layer_params(wl, layer), **round_structure(wl, 0), **round_inputs(wl, layer, 0))
    g, ref, sel = _run_case(sh, case, lanes=lanes, route=route)
    assert int(g.status.item()) == 0 and ref["status"] == 0
    assert g.guards_intact()
    errs = compare_verify(g, ref, lanes=sel, ref_is_subset=True)
    # persistent pools are read-only during verify
    assert torch.equal(g.state.cpu(), torch.from_numpy(case["state"]))
    assert torch.equal(g.conv_hist.cpu(), torch.from_numpy(case["conv_hist"]))
    # commit the accepted paths
    accept = case["accept_node"]
    g.commit(accept)
    torch.cuda.synchronize()
    assert int(g.status.item()) == 0
    st, pool, hist = oracle_commit(sh, ref, case["slot_ids"][sel], case["parents"][sel], accept[sel], case["state"],
                                   case["conv_hist"])
    assert st == 0
    gpool, ghist = g.state.cpu().numpy(), g.conv_hist.cpu().numpy()
    slots = case["slot_ids"][sel]
    e_state = err_metric(gpool[slots], pool[slots])
    assert e_state <= REC_TOL, f"committed state error {e_state}"
    assert np.array_equal(ghist[slots], hist[slots].astype(np.float32))
    unused = np.setdiff1d(np.arange(sh.n_slots), case["slot_ids"])
    assert np.array_equal(gpool[unused], case["state"][unused])
    assert np.array_equal(ghist[unused], case["conv_hist"][unused])
    log(f"[parity] {name}: conv {errs['conv']:.2e} out {errs['out']:.2e} log {errs['log']:.2e} state {e_state:.2e}")


SWEEP = [
    # C, N, P, Hk, Hv, dk, dv, tree
    (1, 1, 1, 1, 1, 16, 16, True),
    (3, 5, 4, 1, 2, 16, 32, True),
    (2, 7, 5, 2, 2, 32, 16, True),
    (3, 9, 3, 2, 4, 64, 64, True),
    (2, 17, 4, 1, 3, 128, 64, True),
    (1, 32, 2, 2, 2, 128, 128, True),
    (2, 32, 2, 1, 2, 16, 128, False),
    (3, 31, 5, 2, 4, 64, 32, True),
    (5, 12, 9, 3, 3, 32, 128, True),
    (2, 16, 2, 4, 8, 128, 32, True),
    # 256 <= C * H_v < 512 with d_v = 128 and at most 16 nodes: one workgroup per (lane, value
    # head), split state product, window workgroups
    (9, 13, 10, 8, 32, 128, 128, True),
    (7, 16, 8, 4, 40, 32, 128, True),
    # C * H_v >= 256 with d_v = 128: one workgroup per (lane, value head) over all columns
    (8, 16, 9, 16, 32, 128, 128, True),
    (16, 9, 16, 4, 16, 64, 128, True),
    (4, 25, 5, 8, 64, 32, 128, True),
    # C * H_v >= 512 with d_v = 128: those workgroups also write the commit windows
    (16, 16, 17, 16, 32, 128, 128, True),
    (8, 27, 9, 2, 64, 64, 128, True),
    (8, 25, 9, 8, 64, 32, 128, False),
    (16, 8, 17, 32, 32, 128, 128, False),  # H_k = H_v: each workgroup writes its whole q/k slab
    (32, 4, 33, 4, 16, 16, 128, True),
]


@pytest.mark.parametrize("route", ROUTES)
@pytest.mark.parametrize("C,N,P,Hk,Hv,dk,dv,tree", SWEEP)
def test_shape_sweep(C, N, P, Hk, Hv, dk, dv, tree, route):
    sh = _shape(C, N, P, Hk, Hv, dk, dv)
    log(f"[sweep] shape={tuple(sh)} tree={tree} route={route}")
    case = synth_case(C, N, P, Hk, Hv, dk, dv, seed=7, tree=tree)
    g, ref, _ = _run_case(sh, case, route=route)
    assert int(g.status.item()) == 0 and g.guards_intact()
    compare_verify(g, ref)
    rng = np.random.default_rng(C * 100 + N)
    accept = rng.integers(-1, N, size=C).astype(np.int32)
    g.commit(accept)
    torch.cuda.synchronize()
    st, pool, hist = oracle_commit(sh, ref, case["slot_ids"], case["parents"], accept, case["state"],
                                   case["conv_hist"])
    assert int(g.status.item()) == 0 and st == 0
    assert err_metric(g.state.cpu().numpy(), pool) <= REC_TOL
    assert np.array_equal(g.conv_hist.cpu().numpy(), hist.astype(np.float32))


@pytest.mark.parametrize("route", ROUTES)
def test_many_lanes_small_heads(route):
    C, N, P = 1024, 3, 1100
    sh = _shape(C, N, P, 1, 1, 16, 16)
    log(f"[max-lanes] shape={tuple(sh)} route={route}")
    case = synth_case(C, N, P, 1, 1, 16, 16, seed=3)
    lanes = [0, 511, 1023]
    g, ref, sel = _run_case(sh, case, lanes=lanes, route=route)
    assert int(g.status.item()) == 0 and g.guards_intact()
    compare_verify(g, ref, lanes=sel, ref_is_subset=True)


@pytest.mark.parametrize("route", ROUTES)
@pytest.mark.parametrize("C,N,P,Hk,Hv,dk,dv", [
    (6, 5, 8, 1, 2, 32, 32),
    (16, 5, 20, 4, 32, 64, 128),  # C * H_v = 512: the verify workgroups write the windows
])
def test_padding_and_invalid_lanes_write_nothing(C, N, P, Hk, Hv, dk, dv, route):
    sh = _shape(C, N, P, Hk, Hv, dk, dv)
    log(f"[lanes] padding / invalid parent / duplicate slot / slot out of range, C={C} H_v={Hv} route={route}")
    slots = [2, -1, 3, 5, 5, P] + list(range(6, C))  # lanes 1..5 padding or invalid
    case = synth_case(C, N, P, Hk, Hv, dk, dv, seed=11, slots=slots)
    case["parents"][2, 3] = 3  # not before its child
    g, ref, _ = _run_case(sh, case, route=route)
    want = gdn.STATUS_PARENT | gdn.STATUS_SLOT_DUP | gdn.STATUS_SLOT_RANGE
    assert int(g.status.item()) == want == ref["status"]
    assert g.guards_intact()
    for buf in (g.conv_out, g.commit_win, g.out, g.replay_log):
        a = buf.np()
        assert (a[1:6] == np.float32(SENTINEL)).all(), "an invalid or padding lane was written"
    compare_verify(g, ref, lanes=[0] + list(range(6, C)))
    # the round's status makes the commit a no-op for every lane, including the valid ones
    state0, hist0 = g.state.clone(), g.conv_hist.clone()
    g.commit(np.array([4] + [0] * (C - 1), np.int32))
    torch.cuda.synchronize()
    assert torch.equal(g.state, state0) and torch.equal(g.conv_hist, hist0)


@pytest.mark.parametrize("bad", ["accept_high", "accept_low"])
def test_commit_preflight_is_all_or_nothing(bad):
    C, N, P = 3, 6, 4
    sh = _shape(C, N, P, 1, 2, 32, 32)
    log(f"[transaction] {bad}")
    case = synth_case(C, N, P, 1, 2, 32, 32, seed=12)
    g, ref, _ = _run_case(sh, case)
    assert int(g.status.item()) == 0
    accept = np.array([2, N if bad == "accept_high" else -2, 1], np.int32)
    state0, hist0 = g.state.clone(), g.conv_hist.clone()
    g.commit(accept)
    torch.cuda.synchronize()
    assert int(g.status.item()) == gdn.STATUS_ACCEPT
    assert torch.equal(g.state, state0) and torch.equal(g.conv_hist, hist0)


def test_slot_permutation_equivariance_bit_exact():
    C, N, P = 3, 9, 6
    sh = _shape(C, N, P, 2, 4, 64, 64)
    case = synth_case(C, N, P, 2, 4, 64, 64, seed=13)
    pi = np.array([4, 2, 0, 5, 1, 3])
    g1 = GpuRound(sh, case["x"], case["ba"], case["conv_w"], case["conv_hist"], case["state"], case["dt_bias"],
                  case["A"], case["slot_ids"], case["parents"]).verify()
    pool2, hist2 = np.empty_like(case["state"]), np.empty_like(case["conv_hist"])
    pool2[pi], hist2[pi] = case["state"], case["conv_hist"]
    g2 = GpuRound(sh, case["x"], case["ba"], case["conv_w"], hist2, pool2, case["dt_bias"], case["A"],
                  pi[case["slot_ids"]].astype(np.int32), case["parents"]).verify()
    torch.cuda.synchronize()
    for a, b in ((g1.conv_out, g2.conv_out), (g1.commit_win, g2.commit_win), (g1.out, g2.out),
                 (g1.replay_log, g2.replay_log)):
        assert torch.equal(a.t, b.t)
    accept = np.array([8, -1, 3], np.int32)
    g1.commit(accept)
    g2.commit(accept)
    torch.cuda.synchronize()
    assert torch.equal(g1.state.cpu()[torch.from_numpy(np.arange(P))], g2.state.cpu()[torch.from_numpy(pi)])
    assert torch.equal(g1.conv_hist.cpu(), g2.conv_hist.cpu()[torch.from_numpy(pi)])


def test_rounds_back_to_back_without_host_sync():
    """Three verify -> commit rounds queued on one stream with no host synchronisation,
    then compared with the oracle run round by round on its own pools (slot reuse)."""
    C, N, P, Hk, Hv, d = 2, 6, 3, 1, 2, 32
    sh = _shape(C, N, P, Hk, Hv, d, d)
    base = synth_case(C, N, P, Hk, Hv, d, d, seed=14)
    rounds = [synth_case(C, N, P, Hk, Hv, d, d, seed=100 + r) for r in range(3)]
    accepts = [np.array([5, 2], np.int32), np.array([-1, 4], np.int32), np.array([3, 0], np.int32)]
    g = GpuRound(sh, base["x"], base["ba"], base["conv_w"], base["conv_hist"], base["state"], base["dt_bias"],
                 base["A"], base["slot_ids"], base["parents"])
    outs = []
    for r in range(3):
        g.x.copy_(dev(rounds[r]["x"]))
        g.ba.copy_(dev(rounds[r]["ba"]))
        g.parents.copy_(dev(rounds[r]["parents"]))
        g.verify()
        outs.append(g.out.t.clone())
        g.commit(accepts[r])
    torch.cuda.synchronize()
    assert int(g.status.item()) == 0
    pool, hist = base["state"].astype(np.float64), base["conv_hist"].astype(np.float64)
    for r in range(3):
        ref = oracle_round(sh, rounds[r]["x"], rounds[r]["ba"], base["conv_w"], hist, pool, base["dt_bias"],
                           base["A"], base["slot_ids"], rounds[r]["parents"])
        assert err_metric(outs[r].cpu().numpy(), ref["out"]) <= REC_TOL
        st, pool, hist = oracle_commit(sh, ref, base["slot_ids"], rounds[r]["parents"], accepts[r], pool, hist)
        assert st == 0
    assert err_metric(g.state.cpu().numpy(), pool) <= REC_TOL
    assert err_metric(g.conv_hist.cpu().numpy(), hist) == 0.0


def test_cancelled_round_changes_nothing():
    """A verified round that is never committed leaves the next round's inputs as they were."""
    C, N, P = 2, 8, 4
    sh = _shape(C, N, P, 2, 2, 128, 128)
    case = synth_case(C, N, P, 2, 2, 128, 128, seed=15)
    g = GpuRound(sh, case["x"], case["ba"], case["conv_w"], case["conv_hist"], case["state"], case["dt_bias"],
                 case["A"], case["slot_ids"], case["parents"]).verify()
    first = g.out.t.clone()
    g.verify()  # same inputs again: identical outputs, pools untouched
    torch.cuda.synchronize()
    assert torch.equal(first, g.out.t)
    assert torch.equal(g.state.cpu(), torch.from_numpy(case["state"]))


def test_alias_rejected_on_device():
    C, N, P = 1, 4, 2
    sh = _shape(C, N, P, 1, 1, 16, 16)
    case = synth_case(C, N, P, 1, 1, 16, 16, seed=16)
    x = dev(case["x"])
    with pytest.raises(gdn.GdnError) as ei:
        gdn.conv_tree_step(sh, x, dev(case["conv_w"]), dev(case["conv_hist"]), dev(case["slot_ids"]),
                           dev(case["parents"]), conv_out=x)
    assert ei.value.code == 4


def test_graph_replay_matches_eager():
    """The route captured in a HIP graph: every replay, with eager work and host
    synchronisation between replays, is bit-identical to the eager call."""
    C, N, P = 3, 12, 5
    sh = _shape(C, N, P, 2, 4, 128, 128)
    log("[graph] conv + verify + commit captured and replayed")
    case = synth_case(C, N, P, 2, 4, 128, 128, seed=17)
    accept = dev(np.array([11, -1, 4], np.int32))
    g = GpuRound(sh, case["x"], case["ba"], case["conv_w"], case["conv_hist"], case["state"], case["dt_bias"],
                 case["A"], case["slot_ids"], case["parents"])
    state0, hist0 = g.state.clone(), g.conv_hist.clone()
    bufs = (g.conv_out.t, g.commit_win.t, g.out.t, g.replay_log.t)

    def run():
        g.verify()
        gdn.replay_commit(sh, g.replay_log.t, g.commit_win.t, g.slot_ids, g.parents, accept, g.state, g.conv_hist,
                          g.status)

    run()
    torch.cuda.synchronize()
    ref = [b.clone() for b in bufs] + [g.state.clone(), g.conv_hist.clone()]
    g.state.copy_(state0)
    g.conv_hist.copy_(hist0)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run()
    for rep in range(3):
        for b in bufs:
            b.fill_(0.0)  # eager work between replays
        g.state.copy_(state0)
        g.conv_hist.copy_(hist0)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert int(g.status.item()) == 0
        for a, b in zip(list(bufs) + [g.state, g.conv_hist], ref):
            assert torch.equal(a, b), f"replay {rep} differs from the eager result"


def _layer_rounds(wl, layers):
    sh = gdn.Shape(**wl.shape_dict())
    rs = round_structure(wl, 0)
    rounds, cases = [], []
    for layer in layers:
        case = dict(layer_params(wl, layer), **rs, **round_inputs(wl, layer, 0))
        rounds.append(GpuRound(sh, case["x"], case["ba"], case["conv_w"], case["conv_hist"], case["state"],
                               case["dt_bias"], case["A"], case["slot_ids"], case["parents"]).verify())
        cases.append(case)
    torch.cuda.synchronize()
    return sh, rs, rounds, cases


def test_commit_layers_matches_per_layer_and_oracle():
    """Every layer of chains-c5-n8-l48 committed in one launch: bit-identical to one
    commit launch per layer, and within the recurrence bar of the oracle on sampled layers."""
    wl = WORKLOADS["chains-c5-n8-l48"]
    layers = list(range(wl.n_layers))
    log(f"[commit-layers] {wl.name} L={len(layers)}")
    sh, rs, rounds, cases = _layer_rounds(wl, layers)
    accept = dev(rs["accept_node"])
    pools = [g.state.clone() for g in rounds]
    hists = [g.conv_hist.clone() for g in rounds]
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    gdn.replay_commit_layers(sh, [g.replay_log.t for g in rounds], [g.commit_win.t for g in rounds], rounds[0].slot_ids,
                             rounds[0].parents, accept, pools, hists, status)
    for g in rounds:
        g.commit(rs["accept_node"])
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    for l, g in enumerate(rounds):
        assert int(g.status.item()) == 0
        assert torch.equal(pools[l], g.state), f"layer {l} state"
        assert torch.equal(hists[l], g.conv_hist), f"layer {l} history"
    for l in (0, 23, 47):
        c = cases[l]
        ref = oracle_round(sh, c["x"], c["ba"], c["conv_w"], c["conv_hist"], c["state"], c["dt_bias"], c["A"],
                           c["slot_ids"], c["parents"])
        st, pool, hist = oracle_commit(sh, ref, c["slot_ids"], c["parents"], c["accept_node"], c["state"],
                                       c["conv_hist"])
        assert st == 0
        assert err_metric(pools[l].cpu().numpy(), pool) <= REC_TOL
        assert err_metric(hists[l].cpu().numpy(), hist) == 0.0


@pytest.mark.parametrize("bad", ["accept", "slot"])
def test_commit_layers_all_or_nothing(bad):
    """One bad lane cancels the commit of every layer in the launch."""
    wl = WORKLOADS["tree-c4-n16"]
    log(f"[commit-layers transaction] {bad}")
    sh, rs, rounds, _ = _layer_rounds(wl, [0, 0, 0])  # same inputs, three distinct sets of pools
    accept = rs["accept_node"].copy()
    slots = rounds[0].slot_ids.clone()
    if bad == "accept":
        accept[2] = sh.n_nodes
    else:
        slots[1] = sh.n_slots  # out of range
    before = [(g.state.clone(), g.conv_hist.clone()) for g in rounds]
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    gdn.replay_commit_layers(sh, [g.replay_log.t for g in rounds], [g.commit_win.t for g in rounds], slots,
                             rounds[0].parents, dev(accept), [g.state for g in rounds],
                             [g.conv_hist for g in rounds], status)
    torch.cuda.synchronize()
    want = gdn.STATUS_ACCEPT if bad == "accept" else gdn.STATUS_SLOT_RANGE
    assert int(status.item()) & want
    for g, (s0, h0) in zip(rounds, before):
        assert torch.equal(g.state, s0) and torch.equal(g.conv_hist, h0)


def test_fused_matches_split_route():
    """The fused call and the two separate calls on the same inputs: commit windows
    bit-identical, out and replay log within the recurrence bar of each other, and the
    commits that follow give the same pools within that bar."""
    wl = WORKLOADS["tree-c4-n16"]
    sh = gdn.Shape(**wl.shape_dict())
    log("[fused-vs-split] tree-c4-n16")
    case = dict(layer_params(wl, 0), **round_structure(wl, 0), **round_inputs(wl, 0, 0))
    args = (sh, case["x"], case["ba"], case["conv_w"], case["conv_hist"], case["state"], case["dt_bias"], case["A"],
            case["slot_ids"], case["parents"])
    a, b = GpuRound(*args).verify(), GpuRound(*args, fused=True).verify()
    torch.cuda.synchronize()
    assert int(a.status.item()) == 0 and int(b.status.item()) == 0
    assert torch.equal(a.commit_win.t, b.commit_win.t)
    assert err_metric(b.out.np(), a.out.np()) <= REC_TOL
    assert err_metric(b.replay_log.np(), a.replay_log.np()) <= REC_TOL
    a.commit(case["accept_node"])
    b.commit(case["accept_node"])
    torch.cuda.synchronize()
    assert err_metric(b.state.cpu().numpy(), a.state.cpu().numpy()) <= REC_TOL
    assert torch.equal(a.conv_hist, b.conv_hist)


@pytest.mark.parametrize("layer", [0, 47])
def test_stress_two_rounds_on_sampled_lanes(layer):
    """The bandwidth-stress workload (64 lanes in 128 slots, 32-node trees) over two
    verify -> commit rounds of one layer: the GPU runs every lane (fused route), the oracle
    4 sampled lanes on their own slots; outputs, windows and log each round, then the
    committed state and history, are compared."""
    wl = WORKLOADS["stress-c64-n32-l48"]
    sh = gdn.Shape(**wl.shape_dict())
    lanes = np.array([3, 22, 51, 60])
    log(f"[parity] stress two rounds, layer {layer}, lanes {lanes.tolist()}")
    lp = layer_params(wl, layer)
    rs = [round_structure(wl, r) for r in range(2)]
    ri = [round_inputs(wl, layer, r) for r in range(2)]
    g = GpuRound(sh, ri[0]["x"], ri[0]["ba"], lp["conv_w"], lp["conv_hist"], lp["state"], lp["dt_bias"], lp["A"],
                 rs[0]["slot_ids"], rs[0]["parents"], fused=True)
    slots = rs[0]["slot_ids"][lanes]
    local = np.arange(len(lanes), dtype=np.int32)
    pool, hist = lp["state"][slots].astype(np.float64), lp["conv_hist"][slots].astype(np.float64)
    for r in range(2):
        if r:
            g.x.copy_(dev(ri[r]["x"]))
            g.ba.copy_(dev(ri[r]["ba"]))
            g.parents.copy_(dev(rs[r]["parents"]))
        g.verify()
        torch.cuda.synchronize()
        assert int(g.status.item()) == 0
        ref = oracle_round(sh, ri[r]["x"][lanes], ri[r]["ba"][lanes], lp["conv_w"], hist, pool, lp["dt_bias"],
                           lp["A"], local, rs[r]["parents"][lanes])
        errs = compare_verify(g, ref, lanes=lanes, ref_is_subset=True)
        g.commit(rs[r]["accept_node"])
        st, pool, hist = oracle_commit(sh, ref, local, rs[r]["parents"][lanes], rs[r]["accept_node"][lanes], pool,
                                       hist)
        assert st == 0
        log(f"[parity] stress round {r}: {errs}")
    torch.cuda.synchronize()
    assert int(g.status.item()) == 0
    e_state = err_metric(g.state.cpu().numpy()[slots], pool)
    assert e_state <= REC_TOL, f"committed state error {e_state}"
    assert np.array_equal(g.conv_hist.cpu().numpy()[slots], hist.astype(np.float32))
