"""GPU parity at the extremes of the gates and of the q/k scale, and of the prompt path at
the prefill bench shape, through the C ABI against the fp64 oracle.

The gates are beta = sigmoid(b) and g = exp(softplus(a + dt_bias) * A) ("qwen35: DSpark
speculative decoding", raw-gate commit message); the kernels evaluate them on the
hardware transcendental units and form decay ratios from cumulative log-decays, and
normalise q and k with a clamped reciprocal square root.  Each case of
`workloads.EDGE_KINDS` drives one of those paths to its limit: beta -> 1 or 0, g -> 0
(exp(-480)) or 1, mixed extremes along 16- and 32-node paths with A = -exp(U(0, 3)),
near-parallel keys with beta = g = 1 (the triangular solve at its worst conditioning), and
q/k rows scaled by 1e-3 and 1e3.

Bars as everywhere: commit windows and committed history bit-exact; recurrence output,
replay log and committed state within 2e-4 of max|g - r| / max(1, |r|); conv output within
1e-5 of the same metric, where for q|k inputs scaled by 1e3 the q|k channels are compared
after dividing by that scale (a float32 sum of four products carries a rounding error
proportional to its terms, about 1e-4 at that scale when the sum itself is near zero).
"""

import functools

import numpy as np
import pytest
import torch

import gated_deltanet_speculative_amd as gdn
from gpu_util import SENTINEL, Guarded, GpuRound, dev, err_metric, log, oracle_commit, oracle_round
from oracle import gdn_oracle as O
from workloads import EDGE_KINDS, edge_case, synth_case

pytestmark = pytest.mark.gpu

CONV_TOL, REC_TOL = 1e-5, 2e-4

EDGE_SHAPES = [
    # C, N, P, Hk, Hv, d, tree
    (4, 16, 8, 16, 32, 128, True),    # the bench shape: 64-column blocks and window workgroups
    (2, 32, 3, 2, 4, 128, False),     # 32-node chains
    (8, 32, 9, 16, 32, 128, True),    # C * H_v = 256: one workgroup per (lane, value head)
    (16, 16, 17, 16, 32, 128, True),  # C * H_v = 512: those workgroups also write the windows
    (16, 32, 17, 16, 32, 128, True),  # the same with 32-node trees (the stress layer's variant)
]


def _qk_scale(kind):
    return 1e3 if kind == "qk_large" else 1.0


def _conv_err(g, r, kind, Hk, dk):
    """The conv bar's metric; q|k channels of 1e3-scaled inputs compared at the inputs' scale."""
    g = np.asarray(g, np.float64).copy()
    r = np.asarray(r, np.float64).copy()
    s = _qk_scale(kind)
    g[..., :2 * Hk * dk] /= s
    r[..., :2 * Hk * dk] /= s
    return err_metric(g, r)


@functools.lru_cache(maxsize=None)
def _edge_case(kind, shape):
    C, N, P, Hk, Hv, d, tree = shape
    base = synth_case(C, N, P, Hk, Hv, d, d, seed=300 + N, tree=tree)
    case = edge_case(base, kind, Hk, d, seed=1)
    rng = np.random.default_rng(400 + N)
    accept = np.empty(C, np.int32)  # a random node's whole root path, or nothing
    for c in range(C):
        accept[c] = int(rng.integers(-1, N))
    case["accept_node"] = accept
    return case


@functools.lru_cache(maxsize=None)
def _edge_oracle(kind, shape):
    C, N, P, Hk, Hv, d, tree = shape
    case = _edge_case(kind, shape)
    sh = gdn.Shape(C, N, P, Hk, Hv, d, d)
    with np.errstate(over="ignore"):
        ref = oracle_round(sh, case["x"], case["ba"], case["conv_w"], case["conv_hist"], case["state"],
                           case["dt_bias"], case["A"], case["slot_ids"], case["parents"])
        st, pool, hist = oracle_commit(sh, ref, case["slot_ids"], case["parents"], case["accept_node"], case["state"],
                                       case["conv_hist"])
    assert ref["status"] == 0 and st == 0
    return ref, pool, hist


@pytest.mark.parametrize("route", ["split", "fused"])
@pytest.mark.parametrize("shape", EDGE_SHAPES, ids=lambda s: "C{}-N{}-Hv{}-{}".format(s[0], s[1], s[4], "tree" if s[6] else "chain"))
@pytest.mark.parametrize("kind", EDGE_KINDS)
def test_edge_verify_and_commit(kind, shape, route):
    C, N, P, Hk, Hv, d, tree = shape
    sh = gdn.Shape(C, N, P, Hk, Hv, d, d)
    log(f"[edge] {kind} shape={tuple(sh)} tree={tree} route={route}")
    case = _edge_case(kind, shape)
    g = GpuRound(sh, case["x"], case["ba"], case["conv_w"], case["conv_hist"], case["state"], case["dt_bias"],
                 case["A"], case["slot_ids"], case["parents"], fused=route == "fused").verify()
    torch.cuda.synchronize()
    ref, pool, hist = _edge_oracle(kind, shape)
    assert int(g.status.item()) == 0 and g.guards_intact()
    if route == "split":
        e_conv = _conv_err(g.conv_out.np(), ref["conv_out"], kind, Hk, d)
        assert e_conv <= CONV_TOL, f"conv_out error {e_conv}"
    else:
        e_conv = 0.0
        assert (g.conv_out.np() == np.float32(SENTINEL)).all()
    assert np.array_equal(g.commit_win.np(), ref["commit_win"].astype(np.float32)), "commit windows differ"
    e_out = err_metric(g.out.np(), ref["out"])
    e_log = err_metric(g.replay_log.np(), ref["replay_log"])
    assert e_out <= REC_TOL, f"out error {e_out}"
    assert e_log <= REC_TOL, f"replay_log error {e_log}"
    assert torch.equal(g.state.cpu(), torch.from_numpy(case["state"]))
    g.commit(case["accept_node"])
    torch.cuda.synchronize()
    assert int(g.status.item()) == 0
    e_state = err_metric(g.state.cpu().numpy(), pool)
    assert e_state <= REC_TOL, f"committed state error {e_state}"
    assert np.array_equal(g.conv_hist.cpu().numpy(), hist.astype(np.float32))
    log(f"[edge] {kind}: conv {e_conv:.2e} out {e_out:.2e} log {e_log:.2e} state {e_state:.2e}")


# ---------------------------------------------------------------- plain decode step

@pytest.mark.parametrize("kind", EDGE_KINDS)
def test_edge_decode_steps(kind):
    """Three plain steps (conv step + one-token recurrence in place) at the headline head
    shape on edge inputs, and the fused call beside them, bit for bit."""
    C, T, P, Hk, Hv, d = 4, 3, 8, 16, 32, 128
    case = edge_case(synth_case(C, T, P, Hk, Hv, d, d, seed=320, tree=False), kind, Hk, d, seed=2)
    sh1 = gdn.Shape(C, 1, P, Hk, Hv, d, d)
    log(f"[edge] decode {kind} shape={tuple(sh1)}")
    slots = case["slot_ids"]
    hist, state = dev(case["conv_hist"]), dev(case["state"])
    w, dt, A, slot_t = dev(case["conv_w"]), dev(case["dt_bias"]), dev(case["A"]), dev(slots)
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    rhist, rstate = case["conv_hist"].astype(np.float64), case["state"].astype(np.float64)
    # the fused call on its own copies of the pools: bit for bit the two calls
    fhist, fstate = dev(case["conv_hist"]), dev(case["state"])
    sync = torch.zeros((C, Hk, gdn.SYNC_STRIDE), dtype=torch.int32, device="cuda")
    worst_conv = worst_out = 0.0
    for t in range(T):
        ba_f = dev(case["ba"][:, t])
        fout = gdn.conv_decode_step(sh1, dev(case["x"][:, t]), w, fhist, ba_f[:, :Hv], ba_f[:, Hv:], dt, A, fstate,
                                    slot_t, sync, status)
        qkv = Guarded((C, 1, sh1.channels))
        gdn.conv_step(sh1, dev(case["x"][:, t:t + 1]), w, hist, slot_t, status, conv_out=qkv.t)
        ba = dev(case["ba"][:, t])
        out = Guarded((C, Hv, d))
        gdn.decode_step(sh1, qkv.t[:, 0], ba[:, :Hv], ba[:, Hv:], dt, A, state, slot_t, status, out=out.t)
        torch.cuda.synchronize()
        assert int(status.item()) == 0
        rq = np.full((C, 1, sh1.channels), np.nan)
        ro = np.full((C, Hv, d), np.nan)
        with np.errstate(over="ignore"):
            assert O.conv_step(case["x"][:, t:t + 1], case["conv_w"], rhist, slots, rq) == 0
            assert O.decode_step(rq[:, 0], case["ba"][:, t, :Hv], case["ba"][:, t, Hv:], case["dt_bias"], case["A"],
                                 rstate, slots, Hk, ro) == 0
        assert torch.equal(fout, out.t), f"fused step, token {t}"
        worst_conv = max(worst_conv, _conv_err(qkv.np(), rq, kind, Hk, d))
        worst_out = max(worst_out, err_metric(out.np(), ro))
        assert qkv.guards_intact() and out.guards_intact()
    assert worst_conv <= CONV_TOL, f"conv_out error {worst_conv}"
    assert worst_out <= REC_TOL, f"out error {worst_out}"
    assert np.array_equal(hist.cpu().numpy(), rhist.astype(np.float32))
    e_state = err_metric(state.cpu().numpy(), rstate)
    assert e_state <= REC_TOL, f"state error {e_state}"
    assert torch.equal(fhist, hist) and torch.equal(fstate, state) and not sync.any()
    log(f"[edge] decode {kind}: conv {worst_conv:.2e} out {worst_out:.2e} state {e_state:.2e}")


# ---------------------------------------------------------------- prefill

def _prefill_case(C, T, P, Hk, Hv, d, seed, kind=None):
    case = synth_case(C, T, P, Hk, Hv, d, d, seed=seed, tree=False)
    rng = np.random.default_rng(seed)
    case["qkv"] = rng.standard_normal(case["x"].shape).astype(np.float32)  # a prompt's conv output rows
    case["z"] = rng.standard_normal((C, T, Hv, d)).astype(np.float32)
    return case if kind is None else edge_case(case, kind, Hk, d, seed=3)


def _oracle_prefill_lanes(case, Hk, lanes, qkv=None, gate=None):
    """The oracle's prefill of the given lanes on float64 copies of their slots' states."""
    Hv = case["state"].shape[1]
    sel = np.asarray(lanes)
    slots = case["slot_ids"][sel]
    pool = case["state"][slots].astype(np.float64)
    q = case["qkv"] if qkv is None else qkv
    out = np.full((len(sel),) + case["z"].shape[1:], np.nan)
    st = O.prefill(q[sel], case["ba"][sel][..., :Hv], case["ba"][sel][..., Hv:], case["dt_bias"], case["A"], pool,
                   np.arange(len(sel), dtype=np.int32), Hk, out, None if gate is None else case["z"][sel],
                   gate or 0)
    assert st == 0
    return pool, out


@pytest.mark.parametrize("kind", EDGE_KINDS)
def test_edge_prefill(kind):
    """The chunked prefill over 64 tokens (4 chunks) on edge inputs: the per-chunk
    cumulative log-decays and the chunk coefficients at their extremes."""
    C, T, P, Hk, Hv, d = 2, 64, 3, 2, 4, 128
    case = _prefill_case(C, T, P, Hk, Hv, d, seed=330, kind=kind)
    sh = gdn.Shape(C, T, P, Hk, Hv, d, d)
    log(f"[edge] prefill {kind} shape={tuple(sh)}")
    state = dev(case["state"])
    ba = dev(case["ba"])
    out = Guarded((C, T, Hv, d))
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    gdn.prefill(sh, dev(case["qkv"]), ba[..., :Hv], ba[..., Hv:], dev(case["dt_bias"]), dev(case["A"]), state,
                dev(case["slot_ids"]), status, gate_z=dev(case["z"]), gate_mode=1, out=out.t)
    torch.cuda.synchronize()
    assert int(status.item()) == 0 and out.guards_intact()
    pool, ref = _oracle_prefill_lanes(case, Hk, range(C), gate=1)
    e_out = err_metric(out.np(), ref)
    e_state = err_metric(state.cpu().numpy()[case["slot_ids"]], pool)
    assert e_out <= REC_TOL, f"out error {e_out}"
    assert e_state <= REC_TOL, f"state error {e_state}"
    log(f"[edge] prefill {kind}: out {e_out:.2e} state {e_state:.2e}")


PROMPT_C, PROMPT_T, PROMPT_P, PROMPT_HK, PROMPT_HV, PROMPT_D = 4, 1024, 8, 16, 32, 128


@functools.lru_cache(maxsize=None)
def _bench_prompt():
    """The prefill bench shape (4 lanes x 1024 tokens, H_k 16, H_v 32, d 128) through the GPU
    prompt path once: the chain conv step over the prompt, then the prefill on its output
    (ungated, SiLU-gated and sigmoid-gated from the same state)."""
    C, T, P, Hk, Hv, d = PROMPT_C, PROMPT_T, PROMPT_P, PROMPT_HK, PROMPT_HV, PROMPT_D
    case = _prefill_case(C, T, P, Hk, Hv, d, seed=340)
    sh = gdn.Shape(C, T, P, Hk, Hv, d, d)
    hist = dev(case["conv_hist"])
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    qkv = gdn.conv_step(sh, dev(case["x"]), dev(case["conv_w"]), hist, dev(case["slot_ids"]), status)
    ba = dev(case["ba"])
    res = {}
    for gate in (None, 0, 1):
        state = dev(case["state"])
        out = torch.empty((C, T, Hv, d), device="cuda")
        gdn.prefill(sh, qkv, ba[..., :Hv], ba[..., Hv:], dev(case["dt_bias"]), dev(case["A"]), state,
                    dev(case["slot_ids"]), status, gate_z=None if gate is None else dev(case["z"]),
                    gate_mode=gate or 0, out=out)
        res[gate] = (state.cpu().numpy(), out.cpu().numpy())
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    return case, qkv.cpu().numpy(), hist.cpu().numpy(), res


def test_prompt_conv_at_bench_shape():
    """The chain conv step over 4 x 1024 tokens of 8192 channels (32-token runs): every lane's
    conv output within 1e-5 and its history bit-exact."""
    C, Hk = PROMPT_C, PROMPT_HK
    log(f"[prompt] conv step C={C} T={PROMPT_T} Ch={2 * Hk * PROMPT_D + PROMPT_HV * PROMPT_D}")
    case, qkv, hist, _ = _bench_prompt()
    rq = np.full(case["x"].shape, np.nan)
    rhist = case["conv_hist"].astype(np.float64)
    assert O.conv_step(case["x"], case["conv_w"], rhist, case["slot_ids"], rq) == 0
    e_conv = err_metric(qkv, rq)
    assert e_conv <= CONV_TOL, f"conv error {e_conv}"
    assert np.array_equal(hist, rhist.astype(np.float32))
    log(f"[prompt] conv {e_conv:.2e}")


@pytest.mark.parametrize("gate,lanes", [(None, (0, 3)), (0, (1,)), (1, (2,))])
def test_prefill_at_bench_shape(gate, lanes):
    """The prefill at the bench shape (64 chunks per lane) against the oracle on sampled lanes,
    ungated and with either closing gate, on the GPU's own conv output of the prompt."""
    log(f"[prompt] prefill at the bench shape gate={gate} lanes={lanes}")
    case, qkv, _, res = _bench_prompt()
    state, out = res[gate]
    pool, ref = _oracle_prefill_lanes(case, PROMPT_HK, lanes, qkv=qkv, gate=gate)
    sel = np.asarray(lanes)
    e_out = err_metric(out[sel], ref)
    e_state = err_metric(state[case["slot_ids"][sel]], pool)
    assert e_out <= REC_TOL, f"out error {e_out}"
    assert e_state <= REC_TOL, f"state error {e_state}"
    log(f"[prompt] prefill gate={gate}: out {e_out:.2e} state {e_state:.2e}")
