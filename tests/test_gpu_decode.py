"""GPU parity of the plain decode step (chain conv step with in-place history write-back,
one-token recurrence applied to the slot's state in place) through the C ABI against the
fp64 oracle.

Bars: conv output within 1e-5, recurrence output and state within 2e-4 of
max|g - r| / max(1, |r|); conv history, untouched slots and padding lanes bit-exact."""

import numpy as np
import pytest
import torch

import gated_deltanet_speculative_amd as gdn
from gpu_util import SENTINEL, Guarded, dev, err_metric, log
from oracle import gdn_oracle as O
from workloads import synth_case

pytestmark = pytest.mark.gpu

CONV_TOL, REC_TOL = 1e-5, 2e-4


class PlainStep:
    """Device pools and guarded outputs of one layer; conv(t0) runs the conv step over
    tokens t0 .. t0+n-1, decode(t) the recurrence for token t (after a one-token conv)."""

    def __init__(self, case, Hk, slots=None):
        self.case = case
        self.slots = np.asarray(case["slot_ids"] if slots is None else slots, np.int32)
        self.C, self.Ch = case["x"].shape[0], case["x"].shape[2]
        self.P, self.Hv, self.dk, self.dv = case["state"].shape
        self.Hk = Hk
        self.hist, self.state = dev(case["conv_hist"]), dev(case["state"])
        self.conv_w, self.dt, self.A = dev(case["conv_w"]), dev(case["dt_bias"]), dev(case["A"])
        self.slot_t = dev(self.slots)
        self.status = torch.zeros(1, dtype=torch.int32, device="cuda")

    def shape(self, n):
        return gdn.Shape(self.C, n, self.P, self.Hk, self.Hv, self.dk, self.dv)

    def conv(self, t0, n):
        out = Guarded((self.C, n, self.Ch))
        gdn.conv_step(self.shape(n), dev(self.case["x"][:, t0:t0 + n]), self.conv_w, self.hist, self.slot_t,
                      self.status, conv_out=out.t)
        return out

    def decode(self, t):
        qkv = self.conv(t, 1)
        ba = dev(self.case["ba"][:, t])
        out = Guarded((self.C, self.Hv, self.dv))
        gdn.decode_step(self.shape(1), qkv.t[:, 0], ba[:, :self.Hv], ba[:, self.Hv:], self.dt, self.A, self.state,
                        self.slot_t, self.status, out=out.t)
        return qkv, out


    def fused(self, t):
        """conv_decode_step on token t (both parts in one launch)."""
        if not hasattr(self, "sync"):
            self.sync = torch.zeros((self.C, self.Hk, gdn.SYNC_STRIDE), dtype=torch.int32, device="cuda")
        ba = dev(self.case["ba"][:, t])
        out = Guarded((self.C, self.Hv, self.dv))
        gdn.conv_decode_step(self.shape(1), dev(self.case["x"][:, t]), self.conv_w, self.hist, ba[:, :self.Hv],
                             ba[:, self.Hv:], self.dt, self.A, self.state, self.slot_t, self.sync, self.status,
                             out=out.t)
        return out


class OraclePlain:
    """The same steps in the oracle, on float64 copies of the pools."""

    def __init__(self, case, Hk, slots):
        self.case, self.Hk, self.slots = case, Hk, np.asarray(slots, np.int32)
        self.hist = case["conv_hist"].astype(np.float64)
        self.state = case["state"].astype(np.float64)

    def conv(self, t0, n):
        x = self.case["x"][:, t0:t0 + n]
        out = np.full(x.shape, np.nan)
        assert O.conv_step(x, self.case["conv_w"], self.hist, self.slots, out) == 0
        return out

    def decode(self, t):
        qkv = self.conv(t, 1)
        Hv = self.state.shape[1]
        out = np.full((qkv.shape[0], Hv, self.state.shape[3]), np.nan)
        ba = self.case["ba"][:, t]
        assert O.decode_step(qkv[:, 0], ba[:, :Hv], ba[:, Hv:], self.case["dt_bias"], self.case["A"], self.state,
                             self.slots, self.Hk, out) == 0
        return qkv, out


def _check_pools(g, ref, label):
    ghist, gstate = g.hist.cpu().numpy(), g.state.cpu().numpy()
    used = g.slots[g.slots >= 0]
    unused = np.setdiff1d(np.arange(g.P), used)
    assert np.array_equal(ghist[used], ref.hist[used].astype(np.float32)), f"{label}: history"
    e_state = err_metric(gstate[used], ref.state[used])
    assert e_state <= REC_TOL, f"{label}: state error {e_state}"
    assert np.array_equal(ghist[unused], g.case["conv_hist"][unused]), f"{label}: unused history touched"
    assert np.array_equal(gstate[unused], g.case["state"][unused]), f"{label}: unused state touched"
    return e_state


def _compare_rows(gbuf, ref, slots, tol, label):
    """Rows of non-padding lanes within tol; padding lanes untouched; guard bands intact."""
    gv = gbuf.np()
    live = slots >= 0
    e = err_metric(gv[live], ref[live])
    assert e <= tol, f"{label}: error {e}"
    assert (gv[~live] == np.float32(SENTINEL)).all(), f"{label}: padding lane written"
    assert gbuf.guards_intact(), f"{label}: guard band written"
    return e


@pytest.mark.parametrize("n", [1, 2, 5, 19, 70])
def test_conv_step_parity(n):
    """Chain conv step over n tokens: 2 leaves a history mixing old columns and tokens, 19
    spans three 8-token loads with a ragged tail, 70 three 32-token runs of threads."""
    C, P, Hk, Hv, dk, dv = 3, 6, 2, 4, 32, 16
    case = synth_case(C, max(n, 20), P, Hk, Hv, dk, dv, seed=40 + n, tree=False)
    slots = np.array([4, -1, 1], np.int32)
    log(f"[plain] conv_step n={n} C={C} Ch={case['x'].shape[2]} slots={slots.tolist()}")
    g, r = PlainStep(case, Hk, slots), OraclePlain(case, Hk, slots)
    out = g.conv(0, n)
    torch.cuda.synchronize()
    assert int(g.status.item()) == 0
    e = _compare_rows(out, r.conv(0, n), slots, CONV_TOL, "conv_out")
    _check_pools(g, r, "conv_step")
    log(f"[plain] conv_step n={n}: conv {e:.2e}")


DECODE_SHAPES = [
    # C, P, Hk, Hv, dk, dv, padding lane
    (1, 2, 2, 2, 16, 16, None),
    (3, 5, 1, 2, 32, 64, 1),
    (2, 4, 2, 4, 64, 16, None),
    (3, 4, 1, 1, 128, 32, 0),
    (4, 8, 16, 32, 128, 128, None),   # the headline head shape (C=4 lanes in 8 slots)
    (5, 16, 32, 32, 128, 128, 4),     # non-grouped heads
]


@pytest.mark.parametrize("C,P,Hk,Hv,dk,dv,pad", DECODE_SHAPES)
def test_decode_step_parity(C, P, Hk, Hv, dk, dv, pad):
    case = synth_case(C, 1, P, Hk, Hv, dk, dv, seed=50 + C + dk, tree=False)
    slots = case["slot_ids"].copy()
    if pad is not None:
        slots[pad] = -1
    log(f"[plain] decode_step C={C} P={P} Hk={Hk} Hv={Hv} dk={dk} dv={dv} slots={slots.tolist()}")
    g, r = PlainStep(case, Hk, slots), OraclePlain(case, Hk, slots)
    gq, go = g.decode(0)
    torch.cuda.synchronize()
    assert int(g.status.item()) == 0
    rq, ro = r.decode(0)
    e_conv = _compare_rows(gq, rq, slots, CONV_TOL, "conv_out")
    e_out = _compare_rows(go, ro, slots, REC_TOL, "out")
    e_state = _check_pools(g, r, "decode_step")
    log(f"[plain] decode_step: conv {e_conv:.2e} out {e_out:.2e} state {e_state:.2e}")


def test_decode_steps_accumulate_within_tolerance():
    """Eight consecutive plain steps at the headline head shape stay within the bar."""
    C, P, Hk, Hv, dk, dv, T = 4, 8, 16, 32, 128, 128, 8
    case = synth_case(C, T, P, Hk, Hv, dk, dv, seed=61, tree=False)
    slots = case["slot_ids"]
    log(f"[plain] {T} consecutive steps, slots={slots.tolist()}")
    g, r = PlainStep(case, Hk, slots), OraclePlain(case, Hk, slots)
    worst = 0.0
    for t in range(T):
        _, go = g.decode(t)
        _, ro = r.decode(t)
        torch.cuda.synchronize()
        worst = max(worst, _compare_rows(go, ro, slots, REC_TOL, f"out step {t}"))
    assert int(g.status.item()) == 0
    e_state = _check_pools(g, r, "after 8 steps")
    log(f"[plain] 8 steps: out {worst:.2e} state {e_state:.2e}")


@pytest.mark.parametrize("bad", ["slot_dup", "slot_range", "status_in"])
def test_plain_step_is_all_or_nothing(bad):
    C, P, Hk, Hv, dk, dv = 3, 5, 1, 2, 32, 32
    case = synth_case(C, 1, P, Hk, Hv, dk, dv, seed=70, tree=False)
    slots = {"slot_dup": [0, 3, 3], "slot_range": [0, 5, 2], "status_in": [0, 3, 2]}[bad]
    bit = {"slot_dup": gdn.STATUS_SLOT_DUP, "slot_range": gdn.STATUS_SLOT_RANGE, "status_in": 0x100}[bad]
    log(f"[plain] transaction {bad}: slots={slots}")
    g = PlainStep(case, Hk, slots)
    if bad == "status_in":
        g.status.fill_(0x100)
    gq, go = g.decode(0)
    torch.cuda.synchronize()
    st = int(g.status.item())
    assert st & bit
    if bad == "status_in":
        assert st == 0x100
    assert (gq.np() == np.float32(SENTINEL)).all() and (go.np() == np.float32(SENTINEL)).all()
    assert np.array_equal(g.hist.cpu().numpy(), case["conv_hist"])
    assert np.array_equal(g.state.cpu().numpy(), case["state"])


def test_plain_steps_equal_chain_verify_then_commit():
    """GPU against GPU at the headline head shape: k plain steps leave the pools a k-token
    chain verify followed by the commit of all k tokens leaves, and give its outputs."""
    C, P, Hk, Hv, dk, dv, k = 4, 8, 16, 32, 128, 128, 5
    case = synth_case(C, k, P, Hk, Hv, dk, dv, seed=80, tree=False)
    sh = gdn.Shape(C, k, P, Hk, Hv, dk, dv)
    log(f"[plain] {k} plain steps vs chain verify + commit")
    st_v, hist_v = dev(case["state"]), dev(case["conv_hist"])
    slots, parents = dev(case["slot_ids"]), dev(case["parents"])
    ba = dev(case["ba"])
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    out_v, log_v, win_v, _ = gdn.conv_tree_verify(sh, dev(case["x"]), dev(case["conv_w"]), hist_v, ba[..., :Hv],
                                                  ba[..., Hv:], dev(case["dt_bias"]), dev(case["A"]), st_v, slots,
                                                  parents, status=status)
    gdn.replay_commit(sh, log_v, win_v, slots, parents, dev(np.full(C, k - 1, np.int32)), st_v, hist_v, status)
    g = PlainStep(case, Hk)
    outs = [g.decode(t)[1] for t in range(k)]
    torch.cuda.synchronize()
    assert int(status.item()) == 0 and int(g.status.item()) == 0
    assert torch.equal(g.hist, hist_v)
    e_state = err_metric(g.state.cpu().numpy(), st_v.cpu().numpy())
    assert e_state <= REC_TOL, f"state error {e_state}"
    ov = out_v.cpu().numpy()
    e_out = max(err_metric(outs[t].np(), ov[:, t]) for t in range(k))
    assert e_out <= REC_TOL, f"output error {e_out}"
    log(f"[plain] plain vs verify+commit: out {e_out:.2e} state {e_state:.2e}")


def test_plain_step_graph_replay_matches_eager():
    """Two plain steps (conv step + recurrence each) captured in a HIP graph: every replay,
    with eager work and host synchronisation between replays, is bit-identical to the
    eager calls."""
    C, P, Hk, Hv, dk, dv = 4, 8, 16, 32, 128, 128
    case = synth_case(C, 2, P, Hk, Hv, dk, dv, seed=90, tree=False)
    log("[plain] two plain steps captured and replayed")
    g = PlainStep(case, Hk)
    hist0, state0 = g.hist.clone(), g.state.clone()
    sh1 = g.shape(1)
    xs = [dev(case["x"][:, t:t + 1]) for t in range(2)]
    bas = [dev(case["ba"][:, t]) for t in range(2)]
    qkv = [torch.empty((C, 1, g.Ch), device="cuda") for _ in range(2)]
    outs = [torch.empty((C, Hv, dv), device="cuda") for _ in range(2)]

    def run():
        for t in range(2):
            gdn.conv_step(sh1, xs[t], g.conv_w, g.hist, g.slot_t, g.status, conv_out=qkv[t])
            gdn.decode_step(sh1, qkv[t][:, 0], bas[t][:, :Hv], bas[t][:, Hv:], g.dt, g.A, g.state, g.slot_t,
                            g.status, out=outs[t])

    run()
    torch.cuda.synchronize()
    bufs = qkv + outs + [g.hist, g.state]
    ref = [b.clone() for b in bufs]
    g.hist.copy_(hist0)
    g.state.copy_(state0)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run()
    for rep in range(3):
        for b in qkv + outs:
            b.fill_(0.0)  # eager work between replays
        g.hist.copy_(hist0)
        g.state.copy_(state0)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert int(g.status.item()) == 0
        for a, b in zip(bufs, ref):
            assert torch.equal(a, b), f"replay {rep} differs from the eager result"


# ---------------------------------------------------------------- fused plain step
FUSED_SHAPES = DECODE_SHAPES + [
    (2, 3, 2, 6, 16, 128, None),   # 3 value heads per q/k head x 4 column blocks: waves with two blocks
    (2, 3, 1, 8, 32, 128, 0),      # 32 blocks per group: one workgroup per block, with the counters
]


@pytest.mark.parametrize("C,P,Hk,Hv,dk,dv,pad", FUSED_SHAPES)
def test_fused_plain_steps_equal_separate_calls(C, P, Hk, Hv, dk, dv, pad):
    """conv_decode_step against conv_step + decode_step, GPU against GPU, over 5
    consecutive tokens: outputs, state and history bit for bit, untouched slots and padding
    lanes unchanged, and the sync counters back to zero after every call."""
    T = 5
    case = synth_case(C, T, P, Hk, Hv, dk, dv, seed=90 + C + dk + dv, tree=False)
    slots = case["slot_ids"].copy()
    if pad is not None:
        slots[pad] = -1
    log(f"[plain] fused vs separate C={C} P={P} Hk={Hk} Hv={Hv} dk={dk} dv={dv} slots={slots.tolist()}")
    a, b = PlainStep(case, Hk, slots), PlainStep(case, Hk, slots)
    for t in range(T):
        _, oa = a.decode(t)
        ob = b.fused(t)
        torch.cuda.synchronize()
        assert int(a.status.item()) == 0 and int(b.status.item()) == 0
        assert np.array_equal(oa.np(), ob.np()), f"out of token {t}"
        assert ob.guards_intact()
        assert not b.sync.any(), f"sync counters left non-zero after token {t}"
    assert torch.equal(a.state, b.state) and torch.equal(a.hist, b.hist)


def test_fused_plain_step_parity():
    """conv_decode_step at the headline head shape against the fp64 oracle over 3 tokens."""
    C, P, Hk, Hv, dk, dv, T = 4, 8, 16, 32, 128, 128, 3
    case = synth_case(C, T, P, Hk, Hv, dk, dv, seed=97, tree=False)
    slots = case["slot_ids"].copy()
    slots[2] = -1
    log(f"[plain] fused parity slots={slots.tolist()}")
    g, r = PlainStep(case, Hk, slots), OraclePlain(case, Hk, slots)
    worst = 0.0
    for t in range(T):
        go = g.fused(t)
        _, ro = r.decode(t)
        torch.cuda.synchronize()
        worst = max(worst, _compare_rows(go, ro, slots, REC_TOL, f"out token {t}"))
    assert int(g.status.item()) == 0
    e_state = _check_pools(g, r, "fused steps")
    log(f"[plain] fused: out {worst:.2e} state {e_state:.2e}")


@pytest.mark.parametrize("bad", ["slot_dup", "slot_range", "status_in"])
def test_fused_plain_step_is_all_or_nothing(bad):
    """A rejected fused step writes nothing and leaves the sync counters at zero, so the next
    call on the same counters is exact."""
    C, P, Hk, Hv, dk, dv = 3, 5, 1, 2, 32, 32
    case = synth_case(C, 2, P, Hk, Hv, dk, dv, seed=98, tree=False)
    slots = {"slot_dup": [0, 3, 3], "slot_range": [0, 5, 2], "status_in": [0, 3, 2]}[bad]
    bit = {"slot_dup": gdn.STATUS_SLOT_DUP, "slot_range": gdn.STATUS_SLOT_RANGE, "status_in": 0x100}[bad]
    log(f"[plain] fused transaction {bad}: slots={slots}")
    g = PlainStep(case, Hk, slots)
    if bad == "status_in":
        g.status.fill_(0x100)
    go = g.fused(0)
    torch.cuda.synchronize()
    assert int(g.status.item()) & bit
    assert (go.np() == np.float32(SENTINEL)).all()
    assert np.array_equal(g.hist.cpu().numpy(), case["conv_hist"])
    assert np.array_equal(g.state.cpu().numpy(), case["state"])
    assert not g.sync.any()
    # the same counters then serve a valid step exactly
    ok = [0, 3, 2]
    a, b = PlainStep(case, Hk, ok), PlainStep(case, Hk, ok)
    b.sync = g.sync
    _, oa = a.decode(1)
    ob = b.fused(1)
    torch.cuda.synchronize()
    assert int(b.status.item()) == 0 and np.array_equal(oa.np(), ob.np())
    assert torch.equal(a.state, b.state) and torch.equal(a.hist, b.hist) and not b.sync.any()
