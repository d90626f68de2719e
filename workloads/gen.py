"""Workload table and seeded generators.

Shapes follow the pages' deployment: Qwen3.5/3.8-style GDN layers with state
size 128 ("perf(qwen38): various DFlash2 optimizations concurrency C1-C5",
Summary, mechanism 3), concurrent lanes C1-C5 (same page, C1-C4 mechanisms),
width-8 draft chains and tree budgets of 16-32 nodes ("qwen35: DSpark
speculative decoding", DDTree budgets), 48 GDN layers per model (C1-C5 page,
launch accounting).  Channel count = 2*H_k*d_k + H_v*d_v
("llama-cpp-bonsai-gdn-conv.patch", qwen35.cpp hunk).

Value distributions (all drawn in float64 with numpy's PCG64 and rounded to
float32; the second parameter of N(.,.) is the standard deviation):
  projected tokens x ~ N(0,1), conv weights ~ N(0,0.5), conv history ~ N(0,1),
  recurrent state ~ N(0,0.1), beta/alpha logits ~ N(0,1), dt_bias ~ N(0,0.5),
  A = -exp(U(-1,1)).

Random streams: every draw comes from
  Generator(PCG64(SeedSequence([seed, workload_id, layer, round, tag])))
with tag 0 = per-layer persistent parameters (round fixed at 0), tag 1 = the
round's tree/slot/acceptance structure (layer fixed at 0), tag 2 = the round's
per-layer activations.  Within a stream the draw order is fixed (see each
function), so any array can be regenerated alone.
"""

from __future__ import annotations

from dataclasses import dataclass

import numpy as np

TAG_LAYER, TAG_STRUCT, TAG_ACT = 0, 1, 2


@dataclass(frozen=True)
class Workload:
    name: str
    wid: int  # stable id used in the seed key
    n_seqs: int  # C lanes
    n_slots: int  # P pool slots
    n_layers: int
    n_k_heads: int  # H_k
    n_v_heads: int  # H_v
    d_k: int
    d_v: int
    n_nodes: int  # N draft nodes per lane
    tree: bool  # random trees (else linear chains parent[i] = i-1)
    accept: str  # "fixed:<k>", "prefix", "leaf", "leaf-prefix"
    n_rounds: int = 1
    d_conv: int = 4

    @property
    def channels(self) -> int:
        return 2 * self.n_k_heads * self.d_k + self.n_v_heads * self.d_v

    @property
    def log_row(self) -> int:
        return 1 + self.d_k + self.d_v

    def shape_dict(self) -> dict:
        return dict(
            n_seqs=self.n_seqs, n_nodes=self.n_nodes, n_slots=self.n_slots,
            n_k_heads=self.n_k_heads, n_v_heads=self.n_v_heads,
            d_k=self.d_k, d_v=self.d_v, d_conv=self.d_conv,
        )


WORKLOADS = {
    w.name: w
    for w in [
        # 1 lane in a 2-slot pool, 2 heads of width 16, 4-token chain, accepted prefix 2
        Workload("tiny-chain", 0, 1, 2, 1, 2, 2, 16, 16, 4, False, "fixed:2"),
        # 1 lane, grouped heads (2 value heads per q/k head), d=128, 8-token chain
        Workload("grouped-chain-n8", 1, 1, 1, 1, 16, 32, 128, 128, 8, False, "prefix"),
        # 4 lanes in an 8-slot pool, 16-node random trees, one layer (the headline shape)
        Workload("tree-c4-n16", 2, 4, 8, 1, 16, 32, 128, 128, 16, True, "leaf"),
        # 5 lanes in a 16-slot pool, non-grouped 32 heads, 8-token chains, 48 layers
        Workload("chains-c5-n8-l48", 3, 5, 16, 48, 32, 32, 128, 128, 8, False, "prefix"),
        # 64 lanes in a 128-slot pool, 32-node trees, 48 layers, 20 verify/commit rounds
        Workload("stress-c64-n32-l48", 4, 64, 128, 48, 16, 32, 128, 128, 32, True,
                 "leaf-prefix", n_rounds=20),
    ]
}


def _rng(seed: int, wid: int, layer: int, rnd: int, tag: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, wid, layer, rnd, tag])))


def _normal(rng: np.random.Generator, std: float, shape) -> np.ndarray:
    return (rng.standard_normal(shape) * std).astype(np.float32)


def layer_params(wl: Workload, layer: int, seed: int = 0) -> dict:
    """Per-layer persistent tensors, in draw order: conv_w, conv_hist, state, dt_bias, A."""
    rng = _rng(seed, wl.wid, layer, 0, TAG_LAYER)
    ch, w = wl.channels, wl.d_conv - 1
    conv_w = _normal(rng, 0.5, (ch, wl.d_conv))
    conv_hist = _normal(rng, 1.0, (wl.n_slots, ch, w))
    state = _normal(rng, 0.1, (wl.n_slots, wl.n_v_heads, wl.d_k, wl.d_v))
    dt_bias = _normal(rng, 0.5, (wl.n_v_heads,))
    A = (-np.exp(rng.uniform(-1.0, 1.0, wl.n_v_heads))).astype(np.float32)
    return dict(conv_w=conv_w, conv_hist=conv_hist, state=state, dt_bias=dt_bias, A=A)


def path_to_root(parents_row: np.ndarray, node: int) -> list:
    """Nodes from the root's child down to `node` (structure only)."""
    out = []
    while node >= 0:
        out.append(int(node))
        node = int(parents_row[node])
    return out[::-1]


def _random_parents(rng: np.random.Generator, n: int) -> np.ndarray:
    p = np.empty(n, dtype=np.int32)
    p[0] = -1
    for i in range(1, n):
        p[i] = rng.integers(-1, i)  # uniform over [-1, i-1]
    return p


def round_structure(wl: Workload, rnd: int, seed: int = 0) -> dict:
    """Slots (fixed over rounds), draft-tree parents and accepted node per lane.

    Draw order: slot permutation (from the round-0 stream), then per lane the
    parents, then per lane the acceptance draw(s).
    """
    slot_rng = _rng(seed, wl.wid, 0, 0, TAG_STRUCT)
    slot_ids = slot_rng.permutation(wl.n_slots)[: wl.n_seqs].astype(np.int32)
    rng = _rng(seed, wl.wid, 0, rnd, TAG_STRUCT) if rnd else slot_rng
    C, N = wl.n_seqs, wl.n_nodes
    if wl.tree:
        parents = np.stack([_random_parents(rng, N) for _ in range(C)])
    else:
        parents = np.tile(np.arange(-1, N - 1, dtype=np.int32), (C, 1))
    accept = np.empty(C, dtype=np.int32)
    for c in range(C):
        if wl.accept.startswith("fixed:"):
            accept[c] = int(wl.accept.split(":")[1]) - 1
        elif wl.accept == "prefix":  # chain: accepted prefix length k ~ U{0..N}
            accept[c] = int(rng.integers(0, N + 1)) - 1
        else:
            has_child = np.zeros(N, dtype=bool)
            for i in range(N):
                if parents[c, i] >= 0:
                    has_child[parents[c, i]] = True
            leaves = np.flatnonzero(~has_child)
            leaf = int(leaves[rng.integers(0, len(leaves))])
            if wl.accept == "leaf":
                accept[c] = leaf
            else:  # leaf-prefix: accepted depth ~ U{0..depth(leaf)} along that path
                path = path_to_root(parents[c], leaf)
                depth = int(rng.integers(0, len(path) + 1))
                accept[c] = path[depth - 1] if depth > 0 else -1
    return dict(slot_ids=slot_ids, parents=parents.astype(np.int32), accept_node=accept)


def round_inputs(wl: Workload, layer: int, rnd: int, seed: int = 0) -> dict:
    """Per-round per-layer activations, in draw order: x, then the stacked beta|alpha logits.

    `ba[c, i, :H_v]` are the beta logits and `ba[c, i, H_v:]` the alpha logits of
    node i (the stacked projection layout).
    """
    rng = _rng(seed, wl.wid, layer, rnd, TAG_ACT)
    x = _normal(rng, 1.0, (wl.n_seqs, wl.n_nodes, wl.channels))
    ba = _normal(rng, 1.0, (wl.n_seqs, wl.n_nodes, 2 * wl.n_v_heads))
    return dict(x=x, ba=ba)


def synth_case(C: int, N: int, P: int, Hk: int, Hv: int, dk: int, dv: int, seed: int, tree: bool = True,
               slots=None) -> dict:
    """One layer and one round at an arbitrary shape, with the workload distributions.

    Draw order: conv_w, conv_hist, state, dt_bias, A, slot permutation, parents
    (random trees or chains), x, ba.  `slots` overrides the drawn slot ids.
    """
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, 1000, C, N, P, Hk, Hv, dk, dv])))
    ch = 2 * Hk * dk + Hv * dv
    out = dict(
        conv_w=_normal(rng, 0.5, (ch, 4)),
        conv_hist=_normal(rng, 1.0, (P, ch, 3)),
        state=_normal(rng, 0.1, (P, Hv, dk, dv)),
        dt_bias=_normal(rng, 0.5, (Hv,)),
        A=(-np.exp(rng.uniform(-1.0, 1.0, Hv))).astype(np.float32),
    )
    perm = rng.permutation(P)[:C].astype(np.int32)
    out["slot_ids"] = perm if slots is None else np.asarray(slots, np.int32)
    if tree:
        out["parents"] = np.stack([_random_parents(rng, N) for _ in range(C)]).astype(np.int32)
    else:
        out["parents"] = np.tile(np.arange(-1, N - 1, dtype=np.int32), (C, 1))
    out["x"] = _normal(rng, 1.0, (C, N, ch))
    out["ba"] = _normal(rng, 1.0, (C, N, 2 * Hv))
    return out


# Inputs at the extremes the gate formula and the q/k normalisation reach.  The gates are
# beta = sigmoid(b) and g = exp(softplus(a + dt_bias) * A) ("qwen35: DSpark speculative
# decoding", raw-gate commit message); real layers carry A = -exp(A_log) over a wide range.
EDGE_KINDS = (
    "beta_one",       # b = +30: beta -> 1 (the write replaces what the state held along k)
    "beta_zero",      # b = -30: beta -> 0 (pure decay)
    "decay_zero",     # a + dt_bias = +30 with A = -16: g = exp(-480), zero in float32
    "decay_one",      # a + dt_bias = -30: g -> 1
    "gates_mixed",    # per token and head one of the four above or the normal draw; A = -exp(U(0, 3))
    "parallel_keys",  # beta -> 1, g -> 1, and k rows of every token within a few degrees of each other
    "qk_small",       # the q|k channels of tokens and history scaled by 1e-3
    "qk_large",       # ... and by 1e3
)


def edge_case(case: dict, kind: str, n_k_heads: int, d_k: int, seed: int = 0) -> dict:
    """A copy of a `synth_case`-style dict with its inputs pushed to one extreme (EDGE_KINDS).

    Touches `ba` (beta logits in the first H_v columns of a token's row, alpha logits in the
    next H_v), `A`, and the q|k channels (the first 2 * n_k_heads * d_k) of `x`, `conv_hist`
    and, when present, `qkv` (a chain's conv output rows).  Draw order for the kinds that
    draw: the beta picks, the alpha picks, A (gates_mixed); the shared key direction, then
    the per-row perturbations of x, conv_hist and qkv in that order (parallel_keys).
    """
    if kind not in EDGE_KINDS:
        raise ValueError(f"unknown edge kind {kind!r}")
    out = {k: (v.copy() if isinstance(v, np.ndarray) else v) for k, v in case.items()}
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, 2000, EDGE_KINDS.index(kind)])))
    Hv = out["dt_bias"].shape[0]
    b, a = out["ba"][..., :Hv], out["ba"][..., Hv:]  # views: writes land in out["ba"]
    dt = out["dt_bias"].astype(np.float32)
    a_hi, a_lo = np.float32(30.0) - dt, np.float32(-30.0) - dt  # a + dt_bias = +30 / -30
    qk = 2 * n_k_heads * d_k
    slabs = [k for k in ("x", "conv_hist", "qkv") if k in out]
    if kind == "beta_one":
        b[...] = 30.0
    elif kind == "beta_zero":
        b[...] = -30.0
    elif kind == "decay_zero":
        a[...] = np.broadcast_to(a_hi, a.shape)
        out["A"][...] = -16.0
    elif kind == "decay_one":
        a[...] = np.broadcast_to(a_lo, a.shape)
    elif kind == "gates_mixed":
        pb = rng.integers(0, 3, size=b.shape)
        b[...] = np.where(pb == 0, 30.0, np.where(pb == 1, -30.0, b))
        pa = rng.integers(0, 3, size=a.shape)
        a[...] = np.where(pa == 0, np.broadcast_to(a_hi, a.shape), np.where(pa == 1, np.broadcast_to(a_lo, a.shape), a))
        out["A"][...] = (-np.exp(rng.uniform(0.0, 3.0, Hv))).astype(np.float32)
    elif kind == "parallel_keys":
        b[...] = 30.0
        a[...] = np.broadcast_to(a_lo, a.shape)
        base = rng.standard_normal(n_k_heads * d_k)  # one direction per key channel
        for k in slabs:
            arr = out[k]
            kslab = (slice(None),) * (arr.ndim - 1) + (slice(n_k_heads * d_k, qk),)
            if k == "conv_hist":  # [P][Ch][3]: the key channels of every history column
                kslab = (slice(None), slice(n_k_heads * d_k, qk), slice(None))
                shape = arr[kslab].shape
                arr[kslab] = (base[None, :, None] + 0.1 * rng.standard_normal(shape)).astype(np.float32)
            else:
                shape = arr[kslab].shape
                arr[kslab] = (base + 0.1 * rng.standard_normal(shape)).astype(np.float32)
    else:
        s = np.float32(1e-3 if kind == "qk_small" else 1e3)
        for k in slabs:
            arr = out[k]
            if k == "conv_hist":
                arr[:, :qk, :] *= s
            else:
                arr[..., :qk] *= s
    return out
