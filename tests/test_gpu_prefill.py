"""GPU parity of the prefill (the recurrence over a chain of T tokens per lane, the slot's
state updated in place, optional closing output gate) through the C ABI against the fp64
oracle.  Bars: output and state within 2e-4 of max|g - r| / max(1, |r|); conv output of
the prompt within 1e-5 and its history bit-exact; untouched slots and padding lanes
bit-exact."""

import numpy as np
import pytest
import torch

import gated_deltanet_speculative_amd as gdn
from gpu_util import SENTINEL, Guarded, dev, err_metric, log
from oracle import gdn_oracle as O
from workloads import synth_case

pytestmark = pytest.mark.gpu

CONV_TOL, REC_TOL = 1e-5, 2e-4


def _inputs(C, T, P, Hk, Hv, dk, dv, seed, pad=None):
    case = synth_case(C, T, P, Hk, Hv, dk, dv, seed=seed, tree=False)
    rng = np.random.default_rng(seed)
    case["qkv"] = rng.standard_normal(case["x"].shape).astype(np.float32)  # the prompt's conv output rows
    case["z"] = rng.standard_normal((C, T, Hv, dv)).astype(np.float32)
    if pad is not None:
        case["slot_ids"] = case["slot_ids"].copy()
        case["slot_ids"][pad] = -1
    return case


def _gpu_prefill(case, Hk, qkv=None, gate=False, mode=0, status=None, workspace=None):
    C, T, Ch = case["x"].shape
    P, Hv, dk, dv = case["state"].shape
    sh = gdn.Shape(C, T, P, Hk, Hv, dk, dv)
    state = dev(case["state"])
    ba = dev(case["ba"])
    out = Guarded((C, T, Hv, dv))
    status = torch.zeros(1, dtype=torch.int32, device="cuda") if status is None else status
    gdn.prefill(sh, dev(case["qkv"]) if qkv is None else qkv, ba[..., :Hv], ba[..., Hv:], dev(case["dt_bias"]),
                dev(case["A"]), state, dev(case["slot_ids"]), status, gate_z=dev(case["z"]) if gate else None,
                gate_mode=mode, out=out.t, workspace=workspace)
    return state, out, status


def _oracle_prefill(case, Hk, qkv=None, gate=False, mode=0):
    P, Hv, dk, dv = case["state"].shape
    pool = case["state"].astype(np.float64)
    out = np.full(case["z"].shape, np.nan)
    st = O.prefill(case["qkv"] if qkv is None else qkv, case["ba"][..., :Hv], case["ba"][..., Hv:], case["dt_bias"],
                   case["A"], pool, case["slot_ids"], Hk, out, case["z"] if gate else None, mode)
    assert st == 0
    return pool, out


def _check(case, state, out, pool, ref, label):
    slots = case["slot_ids"]
    live = slots >= 0
    gout = out.np()
    e_out = err_metric(gout[live], ref[live])
    assert e_out <= REC_TOL, f"{label}: out error {e_out}"
    assert (gout[~live] == np.float32(SENTINEL)).all(), f"{label}: padding lane written"
    assert out.guards_intact()
    gstate = state.cpu().numpy()
    used = slots[live]
    e_state = err_metric(gstate[used], pool[used])
    assert e_state <= REC_TOL, f"{label}: state error {e_state}"
    unused = np.setdiff1d(np.arange(gstate.shape[0]), used)
    assert np.array_equal(gstate[unused], case["state"][unused]), f"{label}: unused slot touched"
    return e_out, e_state


CASES = [
    # C, T, P, Hk, Hv, dk, dv, padding lane, gate
    (3, 37, 5, 1, 2, 32, 64, 1, None),     # three chunks with a 5-token tail
    (2, 1, 3, 2, 2, 16, 16, None, None),   # a single token
    (2, 16, 4, 2, 4, 16, 16, 0, 1),        # exactly one chunk, sigmoid gate
    (3, 100, 4, 1, 2, 64, 32, None, 0),    # SiLU gate
    (2, 48, 4, 16, 32, 128, 128, None, None),  # the headline head shape
    (2, 48, 4, 16, 32, 128, 128, 1, 1),
]


@pytest.mark.parametrize("C,T,P,Hk,Hv,dk,dv,pad,gate", CASES)
def test_prefill_parity(C, T, P, Hk, Hv, dk, dv, pad, gate):
    case = _inputs(C, T, P, Hk, Hv, dk, dv, seed=200 + T + dk, pad=pad)
    log(f"[prefill] C={C} T={T} Hk={Hk} Hv={Hv} dk={dk} dv={dv} gate={gate} slots={case['slot_ids'].tolist()}")
    state, out, status = _gpu_prefill(case, Hk, gate=gate is not None, mode=gate or 0)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    pool, ref = _oracle_prefill(case, Hk, gate=gate is not None, mode=gate or 0)
    e_out, e_state = _check(case, state, out, pool, ref, "prefill")
    log(f"[prefill] out {e_out:.2e} state {e_state:.2e}")


@pytest.mark.parametrize("T", [512, 513])
def test_prefill_long_prompt(T):
    """512 tokens (32 chunks) and 513 (33 chunks, a one-token tail: the chunk loop runs in
    pairs, so an odd count ends with a step past the last chunk) at d = 128: the error stays
    within the bar."""
    case = _inputs(1, T, 2, 1, 2, 128, 128, seed=210 + T % 2)
    log(f"[prefill] {T}-token prompt")
    state, out, status = _gpu_prefill(case, 1)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    pool, ref = _oracle_prefill(case, 1)
    e_out, e_state = _check(case, state, out, pool, ref, "long prompt")
    log(f"[prefill] {T} tokens: out {e_out:.2e} state {e_state:.2e}")


def test_prompt_conv_then_prefill():
    """A prompt end to end: the chain conv step over 300 tokens (history in place), then the
    prefill on its output."""
    C, T, P, Hk, Hv, dk, dv = 2, 300, 3, 2, 2, 32, 32
    case = _inputs(C, T, P, Hk, Hv, dk, dv, seed=220)
    sh = gdn.Shape(C, T, P, Hk, Hv, dk, dv)
    log("[prefill] conv step over 300 tokens, then prefill")
    hist = dev(case["conv_hist"])
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    qkv = gdn.conv_step(sh, dev(case["x"]), dev(case["conv_w"]), hist, dev(case["slot_ids"]), status)
    state, out, _ = _gpu_prefill(case, Hk, qkv=qkv, status=status)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    ref_qkv = np.full(case["x"].shape, np.nan)
    ref_hist = case["conv_hist"].astype(np.float64)
    assert O.conv_step(case["x"], case["conv_w"], ref_hist, case["slot_ids"], ref_qkv) == 0
    e_conv = err_metric(qkv.cpu().numpy(), ref_qkv)
    assert e_conv <= CONV_TOL, f"conv error {e_conv}"
    assert np.array_equal(hist.cpu().numpy(), ref_hist.astype(np.float32))
    pool, ref = _oracle_prefill(case, Hk, qkv=ref_qkv)
    e_out, e_state = _check(case, state, out, pool, ref, "prompt")
    log(f"[prefill] prompt: conv {e_conv:.2e} out {e_out:.2e} state {e_state:.2e}")


def test_prefill_equals_decode_steps_on_gpu():
    """GPU against GPU at the headline head shape: the prefill of T tokens leaves the state
    and gives the outputs of T plain decode steps."""
    C, T, P, Hk, Hv, dk, dv = 2, 21, 4, 16, 32, 128, 128
    case = _inputs(C, T, P, Hk, Hv, dk, dv, seed=230)
    log("[prefill] prefill vs 21 decode steps")
    state, out, status = _gpu_prefill(case, Hk)
    sh1 = gdn.Shape(C, 1, P, Hk, Hv, dk, dv)
    st_d = dev(case["state"])
    slots = dev(case["slot_ids"])
    outs = []
    for t in range(T):
        ba = dev(case["ba"][:, t])
        outs.append(gdn.decode_step(sh1, dev(case["qkv"][:, t]), ba[:, :Hv], ba[:, Hv:], dev(case["dt_bias"]),
                                    dev(case["A"]), st_d, slots, status))
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    e_state = err_metric(state.cpu().numpy(), st_d.cpu().numpy())
    e_out = max(err_metric(out.np()[:, t], outs[t].cpu().numpy()) for t in range(T))
    assert e_state <= REC_TOL and e_out <= REC_TOL, (e_state, e_out)
    log(f"[prefill] vs decode steps: out {e_out:.2e} state {e_state:.2e}")


def test_prefill_workspace_contents_do_not_matter():
    """A workspace holding NaN (and larger than needed) gives the results of a fresh one,
    bit for bit, on two calls in a row with different prompt lengths."""
    for T in (53, 20):
        case = _inputs(2, T, 4, 2, 4, 32, 32, seed=250 + T)
        sh = gdn.Shape(2, T, 4, 2, 4, 32, 32)
        log(f"[prefill] NaN workspace, T={T}")
        ws = torch.full((gdn.prefill_workspace_size(sh) // 4 + 100,), float("nan"), device="cuda")
        st_a, out_a, status_a = _gpu_prefill(case, 2, gate=True, workspace=ws)
        st_b, out_b, status_b = _gpu_prefill(case, 2, gate=True)
        torch.cuda.synchronize()
        assert int(status_a.item()) == 0 and int(status_b.item()) == 0
        assert torch.equal(st_a, st_b) and np.array_equal(out_a.np(), out_b.np())


@pytest.mark.parametrize("bad", ["slot_dup", "status_in"])
def test_prefill_is_all_or_nothing(bad):
    case = _inputs(3, 20, 4, 1, 2, 32, 32, seed=240)
    case["slot_ids"] = np.array([0, 2, 2] if bad == "slot_dup" else [0, 1, 2], np.int32)
    status = torch.full((1,), 0x100 if bad == "status_in" else 0, dtype=torch.int32, device="cuda")
    log(f"[prefill] transaction {bad}")
    state, out, status = _gpu_prefill(case, 1, status=status)
    torch.cuda.synchronize()
    st = int(status.item())
    assert st & (gdn.STATUS_SLOT_DUP if bad == "slot_dup" else 0x100)
    assert (out.np() == np.float32(SENTINEL)).all()
    assert np.array_equal(state.cpu().numpy(), case["state"])


def test_prompt_graph_replay_matches_eager():
    """The prompt path (chain conv step, then prefill with a gate) captured in a HIP graph:
    every replay, with eager work and host synchronisation between replays, is
    bit-identical to the eager calls."""
    C, T, P, Hk, Hv, dk, dv = 2, 40, 3, 2, 4, 64, 64
    case = _inputs(C, T, P, Hk, Hv, dk, dv, seed=260)
    sh = gdn.Shape(C, T, P, Hk, Hv, dk, dv)
    log("[prefill] conv step + prefill captured and replayed")
    x, w, ba = dev(case["x"]), dev(case["conv_w"]), dev(case["ba"])
    hist, state, slots = dev(case["conv_hist"]), dev(case["state"]), dev(case["slot_ids"])
    z, dt, A = dev(case["z"]), dev(case["dt_bias"]), dev(case["A"])
    hist0, state0 = hist.clone(), state.clone()
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    qkv = torch.empty((C, T, sh.channels), device="cuda")
    out = torch.empty((C, T, Hv, dv), device="cuda")
    ws = torch.empty(gdn.prefill_workspace_size(sh) // 4, device="cuda")

    def run():
        gdn.conv_step(sh, x, w, hist, slots, status, conv_out=qkv)
        gdn.prefill(sh, qkv, ba[..., :Hv], ba[..., Hv:], dt, A, state, slots, status, gate_z=z, gate_mode=0,
                    out=out, workspace=ws)

    run()
    torch.cuda.synchronize()
    ref = [qkv.clone(), out.clone(), hist.clone(), state.clone()]
    hist.copy_(hist0)
    state.copy_(state0)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run()
    for rep in range(3):
        qkv.fill_(0.0)  # eager work between replays
        out.fill_(0.0)
        ws.fill_(float("nan"))
        hist.copy_(hist0)
        state.copy_(state0)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert int(status.item()) == 0
        for a, b in zip([qkv, out, hist, state], ref):
            assert torch.equal(a, b), f"replay {rep} differs from the eager result"
