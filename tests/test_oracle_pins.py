"""Pins of the fp64 oracle against facts that do not come from the oracle itself:
hand-derived worked examples (tests/golden), closed forms, library routines
(numpy.correlate, scipy.special), algebraic invariants and brute force over
every small draft tree."""

import itertools
import os

import numpy as np
import pytest
from scipy import special

from oracle import gdn_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _read_golden(name):
    out = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, val = line.split(":", 1)
            rows = [[float(t) for t in part.split()] for part in val.split("|")]
            out[key.strip()] = np.array(rows if len(rows) > 1 else rows[0])
    return out


def all_parent_arrays(n):
    """Every valid parent array of n nodes: parent[i] in [-1, i-1]."""
    return [np.array(p, dtype=np.int32) for p in itertools.product(*[range(-1, i) for i in range(n)])]


# ------------------------------------------------------------------ elementwise
def test_gate_closed_forms():
    beta, g = O.gates(0.0, 0.0, 0.0, -1.0)
    assert beta == 0.5 and abs(g - 0.5) < 1e-16
    beta, g = O.gates(0.0, 1.5, -1.5, -3.0)  # a + dt_bias = 0 -> g = 2^-3
    assert abs(g - 0.125) < 1e-16
    beta, g = O.gates(50.0, 0.3, 0.2, 0.0)  # A = 0 -> no decay
    assert g == 1.0 and abs(beta - 1.0) < 1e-20
    assert O.softplus(0.0) == np.log(2.0)
    assert abs(O.softplus(60.0) - 60.0) < 1e-20
    assert abs(O.softplus(-60.0) - np.exp(-60.0)) < 1e-40
    z = np.linspace(-30, 30, 601)
    np.testing.assert_allclose(O.sigmoid(z), special.expit(z), rtol=1e-14, atol=1e-300)
    np.testing.assert_allclose(O.silu(z), z * special.expit(z), rtol=1e-14, atol=1e-300)
    np.testing.assert_allclose(O.softplus(z), np.logaddexp(0.0, z), rtol=1e-14)


# ------------------------------------------------------------------ conv
def _conv_case(rng, C, N, Ch, P, parents):
    x = rng.standard_normal((C, N, Ch)).astype(np.float32)
    w = (0.5 * rng.standard_normal((Ch, 4))).astype(np.float32)
    hist = rng.standard_normal((P, Ch, 3)).astype(np.float32)
    out = np.full((C, N, Ch), np.nan)
    win = np.full((C, N, Ch, 3), np.nan)
    return x, w, hist, out, win


def test_conv_golden_worked_example():
    gd = _read_golden("conv_taps.txt")
    x = gd["tokens"].reshape(1, 5, 1)
    w = gd["weights"].reshape(1, 4)
    hist = gd["history"].reshape(1, 1, 3)
    parents = gd["parents"].astype(np.int32).reshape(1, 5)
    out = np.full((1, 5, 1), np.nan)
    win = np.full((1, 5, 1, 3), np.nan)
    assert O.conv_tree_step(x, w, hist, np.array([0]), parents, out, win) == 0
    np.testing.assert_array_equal(out[0, :, 0], gd["conv_out"])
    np.testing.assert_array_equal(win[0, :, 0, :], gd["commit_win"])


def test_conv_chain_is_textbook_depthwise_conv():
    """A chain reduces to a causal depthwise conv1d (cross-correlation) over [history; x]."""
    rng = np.random.default_rng(1)
    C, N, Ch, P = 2, 7, 24, 3
    parents = np.tile(np.arange(-1, N - 1, dtype=np.int32), (C, 1))
    x, w, hist, out, win = _conv_case(rng, C, N, Ch, P, parents)
    slots = np.array([2, 0], dtype=np.int32)
    assert O.conv_tree_step(x, w, hist, slots, parents, out, win) == 0
    for c in range(C):
        for ch in range(Ch):
            seq = np.concatenate([hist[slots[c], ch].astype(np.float64), x[c, :, ch].astype(np.float64)])
            z = np.correlate(seq, w[ch].astype(np.float64), mode="valid")
            np.testing.assert_allclose(out[c, :, ch], z * special.expit(z), rtol=1e-13, atol=1e-14)
            for i in range(N):  # commit window = last 3 columns up to token i
                np.testing.assert_array_equal(win[c, i, ch], seq[i + 1:i + 4])


@pytest.mark.parametrize("tap", range(4))
def test_conv_one_hot_tap_order(tap):
    """Weight one-hot at tap j selects window column j (tap 0 = oldest)."""
    rng = np.random.default_rng(2)
    C, N, Ch, P = 1, 5, 8, 1
    parents = np.array([[-1, 0, 1, 2, 3]], dtype=np.int32)
    x, w, hist, out, win = _conv_case(rng, C, N, Ch, P, parents)
    w[:] = 0
    w[:, tap] = 1
    O.conv_tree_step(x, w, hist, np.array([0]), parents, out, win)
    seq = np.concatenate([hist[0].T, x[0]], axis=0).astype(np.float64)  # [3+N, Ch]
    for i in range(N):
        z = seq[i + tap]
        np.testing.assert_allclose(out[0, i], z * special.expit(z), rtol=1e-14)


@pytest.mark.parametrize("n", [4, 5])
def test_conv_tree_equals_chain_on_root_path_all_trees(n):
    """Brute force over every parent array: a node's conv output and commit window
    equal the chain conv of its root path."""
    rng = np.random.default_rng(3 + n)
    Ch = 6
    x = rng.standard_normal((1, n, Ch)).astype(np.float32)
    w = (0.5 * rng.standard_normal((Ch, 4))).astype(np.float32)
    hist = rng.standard_normal((1, Ch, 3)).astype(np.float32)
    for parents in all_parent_arrays(n):
        out = np.full((1, n, Ch), np.nan)
        win = np.full((1, n, Ch, 3), np.nan)
        O.conv_tree_step(x, w, hist, np.array([0]), parents[None], out, win)
        for i in range(n):
            path = O.root_path(parents, i)
            seq = np.concatenate([hist[0].T, x[0, path]], axis=0).astype(np.float64)
            z = np.array([np.correlate(seq[:, ch], w[ch].astype(np.float64), "valid")[-1] for ch in range(Ch)])
            np.testing.assert_allclose(out[0, i], z * special.expit(z), rtol=1e-13, atol=1e-14)
            np.testing.assert_array_equal(win[0, i], seq[-3:].T)


# ------------------------------------------------------------------ recurrence
def test_delta_rule_golden_worked_example():
    gd = _read_golden("delta_rule_2x2.txt")
    S = gd["S0"].astype(np.float64)
    for t in range(2):
        S, o, g, k_hat, delta = O.token_step(S, gd["q"][t], gd["k"][t], gd["v"][t], gd["b"][t], gd["a"][t],
                                             gd["dt_bias"].item(), gd["A"].item())
        np.testing.assert_allclose(g, gd["g"][t], rtol=1e-15)
        np.testing.assert_allclose(delta, gd["delta"][t], rtol=1e-14, atol=1e-15)
        np.testing.assert_allclose(S, gd["S%d" % (t + 1)], rtol=1e-14, atol=1e-15)
        np.testing.assert_allclose(o * np.sqrt(2.0), gd["o_times_sqrt2"][t], rtol=1e-14, atol=1e-15)


def _rand_token(rng, d_k, d_v):
    return (rng.standard_normal(d_k), rng.standard_normal(d_k), rng.standard_normal(d_v),
            rng.standard_normal(), rng.standard_normal(), 0.5 * rng.standard_normal(), -np.exp(rng.uniform(-1, 1)))


def test_delta_rule_write_property():
    """beta = 1: after the step the state maps k_hat to v exactly, whatever the decay
    (the correction is taken against the decayed state)."""
    rng = np.random.default_rng(4)
    for _ in range(20):
        S = 0.1 * rng.standard_normal((16, 12))
        q, k, v, _, a, dt, A = _rand_token(rng, 16, 12)
        S1, *_ = O.token_step(S, q, k, v, 800.0, a, dt, A)
        np.testing.assert_allclose(S1.T @ (k / np.linalg.norm(k)), v, rtol=1e-12, atol=1e-12)


def test_delta_rule_partial_strength():
    """0 < beta < 1: S1^T k_hat = (1 - beta) g S^T k_hat + beta v."""
    rng = np.random.default_rng(5)
    for _ in range(20):
        S = 0.1 * rng.standard_normal((8, 8))
        q, k, v, b, a, dt, A = _rand_token(rng, 8, 8)
        beta, g = special.expit(b), np.exp(np.logaddexp(0.0, a + dt) * A)
        kh = k / np.linalg.norm(k)
        S1, *_ = O.token_step(S, q, k, v, b, a, dt, A)
        np.testing.assert_allclose(S1.T @ kh, (1 - beta) * g * (S.T @ kh) + beta * v, rtol=1e-12, atol=1e-12)


def test_output_reads_updated_state_and_scale():
    """beta = 1 and q = k: the output is v / sqrt(d_k)."""
    rng = np.random.default_rng(6)
    S = 0.1 * rng.standard_normal((32, 16))
    _, k, v, _, a, dt, A = _rand_token(rng, 32, 16)
    _, o, *_ = O.token_step(S, 3.0 * k, k, v, 800.0, a, dt, A)
    np.testing.assert_allclose(o, v / np.sqrt(32), rtol=1e-12, atol=1e-12)


def test_zero_beta_is_pure_decay():
    """beta = 0: S_t = (prod g) S0 and o_t = (prod g) S0^T q_hat / sqrt(d_k)."""
    rng = np.random.default_rng(7)
    S0 = 0.1 * rng.standard_normal((16, 16))
    S, G = S0.copy(), 1.0
    for _ in range(6):
        q, k, v, _, a, dt, A = _rand_token(rng, 16, 16)
        with np.errstate(over="ignore"):
            S, o, g, *_ = O.token_step(S, q, k, v, -1e4, a, dt, A)
        G *= np.exp(np.logaddexp(0.0, a + dt) * A)
        np.testing.assert_allclose(S, G * S0, rtol=1e-12, atol=1e-300)
        np.testing.assert_allclose(o, G * S0.T @ (q / np.linalg.norm(q)) / 4.0, rtol=1e-12, atol=1e-300)


def test_associative_memory_retrieval():
    """No decay, beta = 1, empty state, orthonormal keys: querying key j returns v_j / sqrt(d_k)."""
    rng = np.random.default_rng(8)
    d = 16
    Qm, _ = np.linalg.qr(rng.standard_normal((d, d)))
    keys = Qm[:, :6].T
    vals = rng.standard_normal((6, d))
    S = np.zeros((d, d))
    for j in range(5):
        S, *_ = O.token_step(S, keys[j], keys[j], vals[j], 800.0, 0.0, 0.0, 0.0)
    for j in range(5):  # a 6th write along an orthogonal key, queried with key j
        _, o, *_ = O.token_step(S, keys[j], keys[5], vals[5], 800.0, 0.0, 0.0, 0.0)
        np.testing.assert_allclose(o, vals[j] / 4.0, rtol=1e-12, atol=1e-12)


def test_qk_scale_invariance():
    rng = np.random.default_rng(9)
    S = 0.1 * rng.standard_normal((8, 8))
    q, k, v, b, a, dt, A = _rand_token(rng, 8, 8)
    r1 = O.token_step(S, q, k, v, b, a, dt, A)
    r2 = O.token_step(S, 7.5 * q, 0.01 * k, v, b, a, dt, A)
    for x1, x2 in zip(r1, r2):
        np.testing.assert_allclose(x1, x2, rtol=1e-12, atol=1e-14)


def _verify_inputs(rng, C, N, P, Hk, Hv, dk, dv):
    Ch = 2 * Hk * dk + Hv * dv
    return dict(
        qkv=rng.standard_normal((C, N, Ch)),
        b=rng.standard_normal((C, N, Hv)),
        a=rng.standard_normal((C, N, Hv)),
        dt=0.5 * rng.standard_normal(Hv),
        A=-np.exp(rng.uniform(-1, 1, Hv)),
        pool=0.1 * rng.standard_normal((P, Hv, dk, dv)),
    )


def _run_verify(inp, slots, parents, Hk):
    C, N, _ = inp["qkv"].shape
    P, Hv, dk, dv = inp["pool"].shape
    out = np.full((C, N, Hv, dv), np.nan)
    log = np.full((C, N, Hv, 1 + dk + dv), np.nan)
    st = O.tree_verify(inp["qkv"], inp["b"], inp["a"], inp["dt"], inp["A"], inp["pool"], np.asarray(slots),
                       parents, Hk, out, log)
    return st, out, log


def test_tree_verify_equals_chain_on_every_path_all_trees():
    """Brute force over all 120 trees of 5 nodes: node i's output and log row equal
    those of the last token of a chain made of i's root path."""
    rng = np.random.default_rng(10)
    Hk, Hv, dk, dv, N = 2, 2, 16, 16, 5
    inp = _verify_inputs(rng, 1, N, 2, Hk, Hv, dk, dv)
    for parents in all_parent_arrays(N):
        st, out, log = _run_verify(inp, [1], parents[None], Hk)
        assert st == 0
        for i in range(N):
            path = O.root_path(parents, i)
            m = len(path)
            chain = {k: (v[:, path] if k in ("qkv", "b", "a") else v) for k, v in inp.items()}
            _, cout, clog = _run_verify(chain, [1], np.arange(-1, m - 1, dtype=np.int32)[None], Hk)
            np.testing.assert_allclose(out[0, i], cout[0, m - 1], rtol=1e-12, atol=1e-13)
            np.testing.assert_allclose(log[0, i], clog[0, m - 1], rtol=1e-12, atol=1e-13)


def test_grouped_heads_equal_tiled_non_grouped():
    """H_v = 4 value heads over H_k = 2 q/k heads equals an H_k = 4 run whose q/k heads
    are tiled (0,1,0,1): value head h reads q/k head h mod H_k."""
    rng = np.random.default_rng(11)
    C, N, P, dk, dv = 2, 4, 3, 8, 8
    inp = _verify_inputs(rng, C, N, P, 2, 4, dk, dv)
    parents = np.array([[-1, 0, 0, 1], [-1, -1, 1, 2]], dtype=np.int32)
    st, out_g, log_g = _run_verify(inp, [2, 0], parents, 2)
    q, k, v = inp["qkv"][..., :2 * dk], inp["qkv"][..., 2 * dk:4 * dk], inp["qkv"][..., 4 * dk:]
    tiled = dict(inp)
    tiled["qkv"] = np.concatenate([q, q, k, k, v], axis=-1)
    st2, out_t, log_t = _run_verify(tiled, [2, 0], parents, 4)
    assert st == st2 == 0
    np.testing.assert_array_equal(out_g, out_t)
    np.testing.assert_array_equal(log_g, log_t)


def test_unrolled_closed_form_of_tree_states():
    """The state after node i equals G_i S0 + sum_{a on path(i)} (G_i / G_a) k_hat_a delta_a^T,
    with G the product of the logged decays along the path (an exact algebraic identity)."""
    rng = np.random.default_rng(12)
    Hk, Hv, dk, dv, N = 1, 1, 8, 8, 7
    inp = _verify_inputs(rng, 1, N, 1, Hk, Hv, dk, dv)
    parents = np.array([[-1, 0, 1, 0, 3, 2, -1]], dtype=np.int32)
    _, out, log = _run_verify(inp, [0], parents, Hk)
    q_all = inp["qkv"][0, :, :dk]
    for i in range(N):
        path = O.root_path(parents[0], i)
        G = np.cumprod([log[0, a, 0, 0] for a in path])
        S = G[-1] * inp["pool"][0, 0]
        for j, a in enumerate(path):
            S = S + (G[-1] / G[j]) * np.outer(log[0, a, 0, 1:1 + dk], log[0, a, 0, 1 + dk:])
        qh = q_all[i] / np.linalg.norm(q_all[i])
        np.testing.assert_allclose(out[0, i, 0], S.T @ qh / np.sqrt(dk), rtol=1e-11, atol=1e-12)


# ------------------------------------------------------------------ read-only + commit
def _full_case(rng, C, N, P, Hk, Hv, dk, dv):
    Ch = 2 * Hk * dk + Hv * dv
    return dict(
        x=rng.standard_normal((C, N, Ch)).astype(np.float32),
        ba=rng.standard_normal((C, N, 2 * Hv)).astype(np.float32),
        conv_w=(0.5 * rng.standard_normal((Ch, 4))).astype(np.float32),
        hist=rng.standard_normal((P, Ch, 3)).astype(np.float32),
        pool=(0.1 * rng.standard_normal((P, Hv, dk, dv))).astype(np.float32),
        dt=(0.5 * rng.standard_normal(Hv)).astype(np.float32),
        A=(-np.exp(rng.uniform(-1, 1, Hv))).astype(np.float32),
    )


def _round(case, slots, parents, Hk, pool=None, hist=None):
    pool = case["pool"] if pool is None else pool
    hist = case["hist"] if hist is None else hist
    return O.verify_round(case["x"], case["ba"], case["conv_w"], hist, pool, case["dt"], case["A"],
                          np.asarray(slots, np.int32), parents, Hk)


def test_verify_leaves_persistent_state_untouched():
    rng = np.random.default_rng(13)
    case = _full_case(rng, 2, 5, 4, 2, 2, 16, 16)
    pool0, hist0 = case["pool"].copy(), case["hist"].copy()
    r = _round(case, [3, 1], np.array([[-1, 0, 0, 1, 3], [-1, 0, 1, 2, 3]], np.int32), 2)
    assert r["status"] == 0
    assert pool0.tobytes() == case["pool"].tobytes() and hist0.tobytes() == case["hist"].tobytes()


def _single_token_step(case, c, t, slot, pool, hist, Hk):
    """Verify a 1-node tree made of lane c's node t on the live pools, then commit it."""
    one = {k: (v[c:c + 1, t:t + 1] if k in ("x", "ba") else v) for k, v in case.items()}
    r = O.verify_round(one["x"], one["ba"], one["conv_w"], hist, pool, one["dt"], one["A"],
                       np.array([slot], np.int32), np.array([[-1]], np.int32), Hk)
    st = O.replay_commit(r["replay_log"], r["commit_win"], np.array([slot], np.int32), np.array([[-1]], np.int32),
                         np.array([0], np.int32), pool, hist)
    assert st == 0


def test_commit_equals_sequential_single_token_steps_all_trees():
    """Brute force over all 24 trees of 4 nodes and every accept node: committing the
    accepted path from the replay log equals running the path's tokens one at a time
    (verify a 1-node tree, commit it) on the live pools."""
    rng = np.random.default_rng(14)
    Hk, Hv, dk, dv, N, P = 1, 2, 8, 8, 4, 3
    case = _full_case(rng, 1, N, P, Hk, Hv, dk, dv)
    for parents in all_parent_arrays(N):
        r = _round(case, [2], parents[None], Hk)
        for e in range(-1, N):
            pool = case["pool"].astype(np.float64)
            hist = case["hist"].astype(np.float64)
            st = O.replay_commit(r["replay_log"], r["commit_win"], np.array([2], np.int32), parents[None],
                                 np.array([e], np.int32), pool, hist)
            assert st == 0
            pool_s = case["pool"].astype(np.float64)
            hist_s = case["hist"].astype(np.float64)
            for t in (O.root_path(parents, e) if e >= 0 else []):
                _single_token_step(case, 0, t, 2, pool_s, hist_s, Hk)
            np.testing.assert_allclose(pool, pool_s, rtol=1e-11, atol=1e-12)
            np.testing.assert_array_equal(hist, hist_s)
            if e == -1:
                assert pool.tobytes() == case["pool"].astype(np.float64).tobytes()


def _commit_case():
    rng = np.random.default_rng(15)
    Hk, Hv, dk, dv, N, P = 1, 2, 8, 8, 4, 5
    case = _full_case(rng, 3, N, P, Hk, Hv, dk, dv)
    parents = np.array([[-1, 0, 1, 1], [-1, -1, 0, 2], [-1, 0, 1, 2]], np.int32)
    return case, parents, Hk


def test_commit_touches_only_accepting_slots():
    case, parents, Hk = _commit_case()
    slots = np.array([4, 0, 2], np.int32)
    r = _round(case, slots, parents, Hk)
    pool, hist = case["pool"].astype(np.float64), case["hist"].astype(np.float64)
    st = O.replay_commit(r["replay_log"], r["commit_win"], slots, parents, np.array([3, -1, 0], np.int32), pool, hist)
    assert st == 0
    for s in (0, 1, 3):  # lane 1 accepts nothing; slots 1 and 3 are unused
        assert pool[s].tobytes() == case["pool"][s].astype(np.float64).tobytes()
        assert hist[s].tobytes() == case["hist"][s].astype(np.float64).tobytes()
    assert not np.allclose(pool[4], case["pool"][4]) and not np.allclose(pool[2], case["pool"][2])


@pytest.mark.parametrize("bad,bit", [
    ("accept", O.STATUS_ACCEPT), ("slot_range", O.STATUS_SLOT_RANGE), ("slot_dup", O.STATUS_SLOT_DUP),
    ("parent", O.STATUS_PARENT), ("status_in", 0x100),
])
def test_commit_is_all_or_nothing(bad, bit):
    case, parents, Hk = _commit_case()
    slots = np.array([4, 0, 2], np.int32)
    r = _round(case, slots, parents, Hk)
    accept = np.array([3, 1, 2], np.int32)
    status_in = 0
    if bad == "accept":
        accept[1] = 4
    elif bad == "slot_range":
        slots = np.array([4, 5, 2], np.int32)
    elif bad == "slot_dup":
        slots = np.array([4, 2, 2], np.int32)
    elif bad == "parent":
        parents = parents.copy()
        parents[1, 2] = 2
    else:
        status_in = bit
    pool, hist = case["pool"].astype(np.float64), case["hist"].astype(np.float64)
    st = O.replay_commit(r["replay_log"], r["commit_win"], slots, parents, accept, pool, hist, status_in)
    assert st & bit
    assert pool.tobytes() == case["pool"].astype(np.float64).tobytes()
    assert hist.tobytes() == case["hist"].astype(np.float64).tobytes()


def test_invalid_and_padding_lanes_write_nothing():
    case, parents, Hk = _commit_case()
    bad_parents = parents.copy()
    bad_parents[0, 3] = 3  # lane 0: parent not before its child
    r = _round(case, [4, -1, 2], bad_parents, Hk)
    assert r["status"] == O.STATUS_PARENT
    for name in ("conv_out", "commit_win", "out", "replay_log"):
        assert np.isnan(r[name][0]).all() and np.isnan(r[name][1]).all()
        assert not np.isnan(r[name][2]).any()


def test_slot_permutation_equivariance():
    """Permuting the pools by pi and the slot ids through pi leaves every output unchanged."""
    case, parents, Hk = _commit_case()
    slots = np.array([4, 0, 2], np.int32)
    pi = np.array([3, 0, 4, 1, 2])  # new slot of old slot s is pi[s]
    r1 = _round(case, slots, parents, Hk)
    pool2 = np.empty_like(case["pool"])
    hist2 = np.empty_like(case["hist"])
    pool2[pi] = case["pool"]
    hist2[pi] = case["hist"]
    r2 = _round(case, pi[slots], parents, Hk, pool=pool2, hist=hist2)
    for name in ("conv_out", "commit_win", "out", "replay_log"):
        np.testing.assert_array_equal(r1[name], r2[name])


# ------------------------------------------------------------------ plain decode step
def _decode_case(rng, C, N, P, Hk, Hv, dk, dv):
    case = _full_case(rng, C, N, P, Hk, Hv, dk, dv)
    case["qkv"] = rng.standard_normal((C, case["x"].shape[2])).astype(np.float32)
    return case


@pytest.mark.parametrize("n", [1, 5])
def test_conv_step_is_textbook_conv_with_history_shift(n):
    """The chain conv step equals numpy.correlate over [history; tokens] followed by
    SiLU, and leaves the slot holding the last 3 columns of that sequence."""
    rng = np.random.default_rng(20 + n)
    C, Ch, P = 3, 12, 4
    x, w, hist, out, _ = _conv_case(rng, C, n, Ch, P, None)
    slots = np.array([3, -1, 0], np.int32)
    hist64 = hist.astype(np.float64)
    assert O.conv_step(x, w, hist64, slots, out) == 0
    for c in (0, 2):
        s = slots[c]
        for ch in range(Ch):
            seq = np.concatenate([hist[s, ch].astype(np.float64), x[c, :, ch].astype(np.float64)])
            z = np.correlate(seq, w[ch].astype(np.float64), mode="valid")
            np.testing.assert_allclose(out[c, :, ch], z * special.expit(z), rtol=1e-13, atol=1e-14)
            np.testing.assert_array_equal(hist64[s, ch], seq[-3:])
    assert np.isnan(out[1]).all()  # padding lane
    for s in (1, 2):  # unused slots keep their history
        assert hist64[s].tobytes() == hist[s].astype(np.float64).tobytes()


def test_conv_step_equals_tree_conv_of_a_chain():
    """conv_step on a chain gives the tree conv's outputs, and the history it leaves is
    the tree conv's commit window of the last token."""
    rng = np.random.default_rng(26)
    C, N, Ch, P = 2, 4, 10, 3
    parents = np.tile(np.arange(-1, N - 1, dtype=np.int32), (C, 1))
    x, w, hist, out, win = _conv_case(rng, C, N, Ch, P, parents)
    slots = np.array([2, 1], np.int32)
    assert O.conv_tree_step(x, w, hist, slots, parents, out, win) == 0
    out2 = np.full_like(out, np.nan)
    hist64 = hist.astype(np.float64)
    assert O.conv_step(x, w, hist64, slots, out2) == 0
    np.testing.assert_allclose(out2, out, rtol=1e-15, atol=0)
    for c in range(C):
        np.testing.assert_array_equal(hist64[slots[c]], win[c, N - 1])


@pytest.mark.parametrize("bad,bit", [("slot_range", O.STATUS_SLOT_RANGE), ("slot_dup", O.STATUS_SLOT_DUP),
                                     ("status_in", 0x100)])
def test_plain_step_is_all_or_nothing(bad, bit):
    rng = np.random.default_rng(27)
    C, P, Hk, Hv, dk, dv = 3, 4, 1, 2, 8, 8
    case = _decode_case(rng, C, 2, P, Hk, Hv, dk, dv)
    slots = {"slot_range": [0, 4, 2], "slot_dup": [0, 2, 2], "status_in": [0, 1, 2]}[bad]
    slots = np.array(slots, np.int32)
    status_in = bit if bad == "status_in" else 0
    hist = case["hist"].astype(np.float64)
    out = np.full(case["x"].shape, np.nan)
    assert O.conv_step(case["x"], case["conv_w"], hist, slots, out, status_in) & bit
    assert np.isnan(out).all() and hist.tobytes() == case["hist"].astype(np.float64).tobytes()
    pool = case["pool"].astype(np.float64)
    o = np.full((C, Hv, dv), np.nan)
    st = O.decode_step(case["qkv"], case["ba"][:, 0, :Hv], case["ba"][:, 0, Hv:], case["dt"], case["A"], pool, slots,
                       Hk, o, status_in)
    assert st & bit
    assert np.isnan(o).all() and pool.tobytes() == case["pool"].astype(np.float64).tobytes()


def test_decode_step_zero_beta_is_pure_decay():
    """beta = 0 (b -> -inf): the state only decays, S' = g S, and the output reads it."""
    rng = np.random.default_rng(28)
    C, P, Hk, Hv, dk, dv = 1, 2, 1, 2, 8, 4
    case = _decode_case(rng, C, 1, P, Hk, Hv, dk, dv)
    b = np.full((C, Hv), -1e4)
    a = case["ba"][:, 0, Hv:].astype(np.float64)
    pool = case["pool"].astype(np.float64)
    out = np.full((C, Hv, dv), np.nan)
    with np.errstate(over="ignore"):  # sigmoid(-1e4) = 1 / (1 + inf) = 0 exactly
        assert O.decode_step(case["qkv"], b, a, case["dt"], case["A"], pool, np.array([1], np.int32), Hk, out) == 0
    for h in range(Hv):
        g = np.exp(np.log1p(np.exp(a[0, h] + np.float64(case["dt"][h]))) * np.float64(case["A"][h]))
        S0 = case["pool"][1, h].astype(np.float64)
        np.testing.assert_allclose(pool[1, h], g * S0, rtol=1e-14)
        q = case["qkv"][0, :dk].astype(np.float64)
        np.testing.assert_allclose(out[0, h], g * S0.T @ (q / np.linalg.norm(q)) / np.sqrt(dk), rtol=1e-12)
    assert pool[0].tobytes() == case["pool"][0].astype(np.float64).tobytes()


def test_decode_step_stores_and_retrieves_one_association():
    """Empty state, beta = 1 (b -> +inf) and q = k: the step writes k^ v^T and reads
    back exactly v / sqrt(d_k), whatever the decay."""
    rng = np.random.default_rng(29)
    Hk, Hv, dk, dv = 1, 1, 16, 8
    case = _decode_case(rng, 1, 1, 1, Hk, Hv, dk, dv)
    qkv = case["qkv"].astype(np.float64)
    qkv[0, :dk] = qkv[0, dk:2 * dk]  # q = k
    pool = np.zeros((1, Hv, dk, dv))
    out = np.full((1, Hv, dv), np.nan)
    assert O.decode_step(qkv, np.full((1, Hv), 1e4), case["ba"][:, 0, Hv:], case["dt"], case["A"], pool,
                         np.array([0], np.int32), Hk, out) == 0
    k = qkv[0, dk:2 * dk]
    v = qkv[0, 2 * dk:]
    np.testing.assert_allclose(pool[0, 0], np.outer(k / np.linalg.norm(k), v), rtol=1e-14, atol=1e-15)
    np.testing.assert_allclose(out[0, 0], v / np.sqrt(dk), rtol=1e-13)


def test_decode_steps_equal_chain_verify_then_commit():
    """k plain steps (conv step + decode step, one token at a time) leave the pools and
    produce the outputs of a k-token chain verify followed by the commit of all k tokens."""
    rng = np.random.default_rng(30)
    C, N, P, Hk, Hv, dk, dv = 3, 4, 4, 2, 4, 8, 8
    case = _full_case(rng, C, N, P, Hk, Hv, dk, dv)
    slots = np.array([3, -1, 0], np.int32)
    parents = np.tile(np.arange(-1, N - 1, dtype=np.int32), (C, 1))
    r = _round(case, slots, parents, Hk)
    assert r["status"] == 0
    pool_v, hist_v = case["pool"].astype(np.float64), case["hist"].astype(np.float64)
    assert O.replay_commit(r["replay_log"], r["commit_win"], slots, parents, np.array([N - 1, -1, N - 1], np.int32),
                           pool_v, hist_v) == 0
    pool_d, hist_d = case["pool"].astype(np.float64), case["hist"].astype(np.float64)
    for t in range(N):
        qkv = np.full((C, 1, case["x"].shape[2]), np.nan)
        assert O.conv_step(case["x"][:, t:t + 1], case["conv_w"], hist_d, slots, qkv) == 0
        out = np.full((C, Hv, dv), np.nan)
        assert O.decode_step(qkv[:, 0], case["ba"][:, t, :Hv], case["ba"][:, t, Hv:], case["dt"], case["A"], pool_d,
                             slots, Hk, out) == 0
        for c in (0, 2):
            np.testing.assert_allclose(qkv[c, 0], r["conv_out"][c, t], rtol=1e-14, atol=1e-15)
            np.testing.assert_allclose(out[c], r["out"][c, t], rtol=1e-11, atol=1e-12)
        assert np.isnan(out[1]).all()
    np.testing.assert_allclose(pool_d, pool_v, rtol=1e-11, atol=1e-12)
    np.testing.assert_array_equal(hist_d, hist_v)


# ------------------------------------------------------------------ ragged lanes
def _ragged_case():
    rng = np.random.default_rng(90)
    C, N, P, Hk, Hv, dk, dv = 4, 6, 6, 1, 2, 8, 8
    case = _full_case(rng, C, N, P, Hk, Hv, dk, dv)
    parents = np.array([[-1, 0, 1, 1, 3, 0], [-1, -1, 0, 2, 2, 4], [-1, 0, 0, 1, 2, 3], [-1, 0, 1, 2, 3, 4]],
                       np.int32)
    return case, parents, np.array([5, 0, 3, 2], np.int32), np.array([6, 2, 0, 3], np.int32), Hk


def test_ragged_lane_equals_a_batch_of_its_own_length():
    """A lane with v present nodes gives exactly the outputs of that lane run alone as a
    v-node batch; absent nodes are never written, and garbage in their parents is ignored."""
    case, parents, slots, counts, Hk = _ragged_case()
    garbage = parents.copy()
    for c in range(len(slots)):
        garbage[c, counts[c]:] = 99  # absent nodes: not validated
    r = O.verify_round(case["x"], case["ba"], case["conv_w"], case["hist"], case["pool"], case["dt"], case["A"],
                       slots, garbage, Hk, lane_nodes=counts)
    assert r["status"] == 0
    for c in range(len(slots)):
        v = int(counts[c])
        for name in ("conv_out", "commit_win", "out", "replay_log"):
            assert np.isnan(r[name][c, v:]).all()
        if v == 0:
            continue
        alone = O.verify_round(case["x"][c:c + 1, :v], case["ba"][c:c + 1, :v], case["conv_w"], case["hist"],
                               case["pool"], case["dt"], case["A"], slots[c:c + 1], parents[c:c + 1, :v], Hk)
        assert alone["status"] == 0
        for name in ("conv_out", "commit_win", "out", "replay_log"):
            np.testing.assert_array_equal(r[name][c, :v], alone[name][0])


@pytest.mark.parametrize("bad", [-1, 7])
def test_ragged_lane_count_out_of_range(bad):
    case, parents, slots, counts, Hk = _ragged_case()
    counts = counts.copy()
    counts[2] = bad
    r = O.verify_round(case["x"], case["ba"], case["conv_w"], case["hist"], case["pool"], case["dt"], case["A"],
                       slots, parents, Hk, lane_nodes=counts)
    assert r["status"] == O.STATUS_NODES
    assert np.isnan(r["out"][2]).all() and not np.isnan(r["out"][0]).any()


def test_ragged_commit_accepts_only_present_nodes():
    case, parents, slots, counts, Hk = _ragged_case()
    r = O.verify_round(case["x"], case["ba"], case["conv_w"], case["hist"], case["pool"], case["dt"], case["A"],
                       slots, parents, Hk, lane_nodes=counts)
    pool, hist = case["pool"].astype(np.float64), case["hist"].astype(np.float64)
    accept = np.array([5, 1, -1, 2], np.int32)  # the last present node of lanes 0, 1, 3; lane 2 has none
    assert O.replay_commit(r["replay_log"], r["commit_win"], slots, parents, accept, pool, hist,
                           lane_nodes=counts) == 0
    for c, e in ((0, 5), (1, 1), (3, 2)):
        S = case["pool"][slots[c]].astype(np.float64)
        for t in O.root_path(parents[c], e):
            for h in range(S.shape[0]):
                row = r["replay_log"][c, t, h]
                S[h] = row[0] * S[h] + np.outer(row[1:9], row[9:])
        np.testing.assert_allclose(pool[slots[c]], S, rtol=1e-13)
    assert pool[slots[2]].tobytes() == case["pool"][slots[2]].astype(np.float64).tobytes()
    pool2, hist2 = case["pool"].astype(np.float64), case["hist"].astype(np.float64)
    st = O.replay_commit(r["replay_log"], r["commit_win"], slots, parents, np.array([5, 2, -1, 2], np.int32), pool2,
                         hist2, lane_nodes=counts)  # node 2 of lane 1 is absent
    assert st == O.STATUS_ACCEPT
    assert pool2.tobytes() == case["pool"].astype(np.float64).tobytes()


# ------------------------------------------------------------------ prefill
def _prefill_case(seed=110, C=3, T=9, P=4, Hk=2, Hv=4, dk=8, dv=8):
    rng = np.random.default_rng(seed)
    case = _full_case(rng, C, T, P, Hk, Hv, dk, dv)
    case["qkv"] = rng.standard_normal((C, T, case["x"].shape[2])).astype(np.float32)
    case["z"] = rng.standard_normal((C, T, Hv, dv)).astype(np.float32)
    return case, Hk


def _run_prefill(case, Hk, slots, gate=None, mode=0):
    Hv = case["pool"].shape[1]
    pool = case["pool"].astype(np.float64)
    out = np.full(case["z"].shape, np.nan)
    st = O.prefill(case["qkv"], case["ba"][..., :Hv], case["ba"][..., Hv:], case["dt"], case["A"], pool, slots, Hk,
                   out, gate, mode)
    return st, pool, out


def test_prefill_equals_single_token_steps():
    """The prefill over T tokens leaves the state and gives the outputs of T successive
    plain decode steps."""
    case, Hk = _prefill_case()
    slots = np.array([2, -1, 0], np.int32)
    st, pool, out = _run_prefill(case, Hk, slots)
    assert st == 0
    Hv = case["pool"].shape[1]
    pool_d = case["pool"].astype(np.float64)
    for t in range(case["qkv"].shape[1]):
        o = np.full((3, Hv, case["z"].shape[3]), np.nan)
        assert O.decode_step(case["qkv"][:, t], case["ba"][:, t, :Hv], case["ba"][:, t, Hv:], case["dt"], case["A"],
                             pool_d, slots, Hk, o) == 0
        np.testing.assert_allclose(out[:, t], o, rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(pool, pool_d, rtol=1e-13, atol=1e-15)
    assert np.isnan(out[1]).all()
    for s in (1, 3):
        assert pool[s].tobytes() == case["pool"][s].astype(np.float64).tobytes()


def test_prefill_output_gates():
    """gate_mode 1 multiplies by the logistic function (scipy's expit); gate_mode 0 by
    silu(z) = z * expit(z), so the SiLU-gated output is the sigmoid-gated one times z."""
    case, Hk = _prefill_case(seed=111)
    slots = np.array([0, 1, 3], np.int32)
    _, _, plain = _run_prefill(case, Hk, slots)
    _, _, sig = _run_prefill(case, Hk, slots, case["z"], 1)
    _, _, sil = _run_prefill(case, Hk, slots, case["z"], 0)
    z = case["z"].astype(np.float64)
    np.testing.assert_allclose(sig, plain * special.expit(z), rtol=1e-14, atol=1e-16)
    np.testing.assert_allclose(sil, sig * z, rtol=1e-13, atol=1e-16)
    zero = np.zeros_like(case["z"])
    _, _, s0 = _run_prefill(case, Hk, slots, zero, 1)
    _, _, l0 = _run_prefill(case, Hk, slots, zero, 0)
    np.testing.assert_array_equal(s0, plain / 2)
    assert (l0 == 0).all()


@pytest.mark.parametrize("bad,bit", [("slot_dup", O.STATUS_SLOT_DUP), ("status_in", 0x100)])
def test_prefill_is_all_or_nothing(bad, bit):
    case, Hk = _prefill_case(seed=112)
    slots = np.array([0, 2, 2] if bad == "slot_dup" else [0, 1, 2], np.int32)
    Hv = case["pool"].shape[1]
    pool = case["pool"].astype(np.float64)
    out = np.full(case["z"].shape, np.nan)
    st = O.prefill(case["qkv"], case["ba"][..., :Hv], case["ba"][..., Hv:], case["dt"], case["A"], pool, slots, Hk,
                   out, status_in=bit if bad == "status_in" else 0)
    assert st & bit
    assert np.isnan(out).all() and pool.tobytes() == case["pool"].astype(np.float64).tobytes()
