"""The seeded generator: determinism, shapes, and valid tree / slot / acceptance structure."""

import numpy as np
import pytest

from workloads import WORKLOADS, layer_params, path_to_root, round_inputs, round_structure


@pytest.mark.parametrize("name", list(WORKLOADS))
def test_structure_is_valid(name):
    wl = WORKLOADS[name]
    for rnd in range(min(wl.n_rounds, 3)):
        st = round_structure(wl, rnd)
        slots, parents, acc = st["slot_ids"], st["parents"], st["accept_node"]
        assert slots.shape == (wl.n_seqs,) and len(set(slots.tolist())) == wl.n_seqs
        assert ((slots >= 0) & (slots < wl.n_slots)).all()
        assert parents.shape == (wl.n_seqs, wl.n_nodes) and parents.dtype == np.int32
        for c in range(wl.n_seqs):
            for i in range(wl.n_nodes):
                assert -1 <= parents[c, i] < i
            if not wl.tree:
                assert (parents[c] == np.arange(-1, wl.n_nodes - 1)).all()
            assert -1 <= acc[c] < wl.n_nodes
            if wl.accept == "leaf":  # a whole root-to-leaf path
                assert acc[c] not in parents[c]
        assert (round_structure(wl, rnd)["slot_ids"] == round_structure(wl, 0)["slot_ids"]).all()


def test_fixed_prefix_and_shapes():
    wl = WORKLOADS["tiny-chain"]
    assert wl.channels == 96 and wl.log_row == 33
    assert round_structure(wl, 0)["accept_node"].tolist() == [1]
    lp = layer_params(wl, 0)
    assert lp["conv_w"].shape == (96, 4) and lp["conv_hist"].shape == (2, 96, 3)
    assert lp["state"].shape == (2, 2, 16, 16) and (lp["A"] < 0).all()
    ri = round_inputs(wl, 0, 0)
    assert ri["x"].shape == (1, 4, 96) and ri["ba"].shape == (1, 4, 4)
    assert WORKLOADS["tree-c4-n16"].channels == 8192 and WORKLOADS["chains-c5-n8-l48"].channels == 12288
    assert WORKLOADS["tree-c4-n16"].log_row == 257


def test_determinism_and_independence():
    wl = WORKLOADS["tree-c4-n16"]
    a, b = round_inputs(wl, 0, 0, seed=0), round_inputs(wl, 0, 0, seed=0)
    assert a["x"].tobytes() == b["x"].tobytes()
    c = round_inputs(wl, 1, 0, seed=0)
    assert not np.array_equal(a["x"], c["x"])
    lp = layer_params(WORKLOADS["tiny-chain"], 0)
    assert abs(float(lp["state"].std()) - 0.1) < 0.02


def test_leaf_prefix_acceptance_on_path():
    wl = WORKLOADS["stress-c64-n32-l48"]
    st = round_structure(wl, 1)
    depths = [len(path_to_root(st["parents"][c], int(e))) if e >= 0 else 0 for c, e in enumerate(st["accept_node"])]
    assert min(depths) >= 0 and max(depths) <= wl.n_nodes


def test_edge_inputs_reach_their_extremes():
    """The edge inputs do what they are for, checked on the oracle's float64 values: keys
    within a few degrees of each other, decays of exactly exp(-480) and of 1 - 1e-12 or
    closer, beta saturated, q|k channels scaled and nothing else touched."""
    from oracle import gdn_oracle as O
    from workloads import EDGE_KINDS, edge_case, synth_case

    C, N, P, Hk, Hv, d = 2, 32, 3, 2, 4, 128
    base = synth_case(C, N, P, Hk, Hv, d, d, seed=332, tree=False)

    def run(kind):
        case = edge_case(base, kind, Hk, d, seed=1)
        with np.errstate(over="ignore"):
            ref = O.verify_round(case["x"], case["ba"], case["conv_w"], case["conv_hist"], case["state"],
                                 case["dt_bias"], case["A"], case["slot_ids"], case["parents"], Hk)
        assert ref["status"] == 0
        return case, ref

    case, ref = run("parallel_keys")
    k = ref["conv_out"][..., Hk * d:2 * Hk * d].reshape(C, N, Hk, d)
    kn = k / np.linalg.norm(k, axis=-1, keepdims=True)
    cos = np.einsum("cihd,cjhd->chij", kn, kn)
    assert cos.min() >= 0.95, f"keys not near-parallel: min cos {cos.min():.3f}"
    assert (ref["replay_log"][..., 0] > 1 - 1e-9).all()
    _, ref = run("decay_zero")
    assert (ref["replay_log"][..., 0] < 1e-200).all()
    _, ref = run("decay_one")
    assert (ref["replay_log"][..., 0] > 1 - 1e-9).all()
    case, _ = run("beta_zero")
    assert (case["ba"][..., :Hv] == -30).all() and np.array_equal(case["ba"][..., Hv:], base["ba"][..., Hv:])
    case, _ = run("gates_mixed")
    b = case["ba"][..., :Hv]
    assert (b == 30).any() and (b == -30).any() and (np.abs(b) < 30).any()
    assert (case["A"] <= -1).all() and (case["A"] >= -np.exp(3.0) - 1e-3).all()
    for kind, s in (("qk_small", 1e-3), ("qk_large", 1e3)):
        case, _ = run(kind)
        qk = 2 * Hk * d
        assert np.allclose(case["x"][..., :qk], base["x"][..., :qk] * np.float32(s), rtol=1e-6)
        assert np.array_equal(case["x"][..., qk:], base["x"][..., qk:])
        assert np.allclose(case["conv_hist"][:, :qk], base["conv_hist"][:, :qk] * np.float32(s), rtol=1e-6)
    assert set(EDGE_KINDS) >= {"beta_one", "beta_zero", "decay_zero", "decay_one", "gates_mixed", "parallel_keys",
                               "qk_small", "qk_large"}
