"""Plain, slow fp64 CPU oracle of the speculative-verify Gated DeltaNet route.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import or call this
module; only the tests, the smoke check and the bench's CPU-baseline leg do.
It shares no code, table or helper with the HIP library: it reads the same
float32 input arrays, upcasts them to float64 and evaluates the plain
definitions below, one lane / head / node at a time.

Sources (page title, then section):
  [P1] "perf(qwen35): fuse the DFlash2 concurrent verify Gated DeltaNet route"
       - Optimizations (tree conv step + commit window; read-only mapped
         recurrence writing output + replay log; gates applied in-kernel),
         closing paragraph (tap/accumulation order kept; persistent state
         read-only during verification; replay-log commit advances it).
  [P2] "Feature/support dflash2"
       - deferred-state commit message: a step the drafter did not draft for commits
         its post-step state to the slot immediately (the plain decode step);
       - first-version commit message: the recurrence of prefill runs on a chunked GDN
         kernel that closes with a SiLU or, by gate_mode, a sigmoid output gate.
  [P3] "qwen35: DSpark speculative decoding (Qwen3.8-27B drafters)"
       - raw-gate commit message: beta = sigmoid(b), gate = softplus(a + dt_bias) * A;
       - v_len commit message: verify and accept run over each lane's drafted length,
         not the buffer-sizing length;
       - DeltaNet-block commit message: one causal-conv step kernel (history window,
         silu(conv), in-place history write-back) and the gated delta rule in place;
       - stacked-projection commit message: ssm_beta|ssm_alpha back to back,
         one l2_norm over the q|k slab, q/k heads broadcast (no repeat).
  [P4] "perf(qwen38): various DFlash2 optimizations concurrency C1-C5"
       - Summary, mechanism 3: replay width 257 for state size 128;
       - Correctness and verification: padded and permuted slots, transaction preflight.
  [P5] "llama-cpp-bonsai-gdn-conv.patch"
       - ssm-conv.cu hunk: conv column p < d_conv-1 is history, else a token;
         sum over taps ascending from the oldest column, then SiLU;
       - ssm-conv.cuh hunk: history stored as [d_conv-1, channels] per sequence;
       - models.h / qwen35.cpp hunks: channel count 2*H_k*d_k + H_v*d_v.
  The per-token recurrence is the gated delta rule (Yang, Kautz, Hatamizadeh,
  "Gated Delta Networks", 2024) in the form the pages' kernels use: decay the
  state, correct it toward v along k with strength beta, read the output from
  the updated state with scale 1/sqrt(d_k).

Readings where the pages are silent (each listed in the design notes):
  * tap 0 multiplies the oldest column; no conv bias (the fused launcher passes none);
  * one 3-column commit window per node: the last 3 columns of the node's
    extended sequence (history followed by the tokens on its root path);
  * value head h uses q/k head (h mod H_k): the broadcast reproduces a tiled repeat;
  * q and k are divided by their exact L2 norm;
  * replay-log row = (g, k_hat[d_k], delta[d_v]): 1 + d_k + d_v floats (257 at 128);
  * accept_node[c] = deepest accepted node (-1 = nothing); the accepted path is
    that node's root path; a lane with slot -1 is padding and is never touched;
  * ragged lanes: lane c may draft fewer than N nodes (lane_nodes[c], default
    N); nodes i >= lane_nodes[c] are absent: never read, written or validated.
    Parents precede children, so an absent node is never an ancestor of a
    present one and the present nodes compute exactly what a lane_nodes[c]-node
    batch would;
  * lane validity: slot outside [-1, P), a slot used by two lanes, a node count
    outside [0, N], a present node's parent outside [-1, i-1] or (commit only)
    an accept node outside [-1, lane_nodes[c]) sets a status bit; conv and verify then write nothing for that lane, and the
    commit mutates nothing at all (all-or-nothing transaction);
  * the plain decode step (conv_step + decode_step) and the prefill mutate the
    pools directly, so they are transactions like the commit: a bad slot
    anywhere, or a non-zero incoming status, and nothing is written;
  * prefill: a chain of T tokens per lane, equal to T single-token steps (the
    chunking is the kernel's business); its optional output gate is
    o * silu(z) (gate_mode 0) or o * sigmoid(z) (gate_mode 1).

Every function below is pinned by tests/test_oracle_pins.py against closed
forms, library routines and brute force.
"""

from __future__ import annotations

import numpy as np

STATUS_SLOT_RANGE = 1
STATUS_SLOT_DUP = 2
STATUS_PARENT = 4
STATUS_ACCEPT = 8
STATUS_NODES = 16

D_CONV = 4


# ---------------------------------------------------------------- elementwise pieces
def silu(z):
    """z * sigmoid(z)."""
    z = np.asarray(z, dtype=np.float64)
    return z / (1.0 + np.exp(-z))


def sigmoid(z):
    z = np.asarray(z, dtype=np.float64)
    return 1.0 / (1.0 + np.exp(-z))


def softplus(z):
    """log(1 + exp(z)), evaluated as max(z,0) + log1p(exp(-|z|)) to avoid overflow."""
    z = np.asarray(z, dtype=np.float64)
    return np.maximum(z, 0.0) + np.log1p(np.exp(-np.abs(z)))


def gates(b, a, dt_bias, A):
    """[P3] raw gates: beta = sigmoid(b); decay g = exp(softplus(a + dt_bias) * A)."""
    beta = sigmoid(b)
    g = np.exp(softplus(np.asarray(a, np.float64) + np.float64(dt_bias)) * np.float64(A))
    return beta, g


def l2_normalize(v):
    v = np.asarray(v, dtype=np.float64)
    return v / np.sqrt(np.sum(v * v))


# ---------------------------------------------------------------- tree structure
def root_path(parents_row, node):
    """Nodes from the root's child down to `node`, following parent links."""
    path = []
    while node >= 0:
        path.append(int(node))
        node = int(parents_row[node])
    return path[::-1]


def lane_counts(lane_nodes, C, N):
    """Nodes present in each lane: lane_nodes[c] (the lane's own draft length), or all N."""
    return [N] * C if lane_nodes is None else [int(v) for v in lane_nodes]


def lane_status(slot_ids, parents, n_slots, lane_nodes=None):
    """Per-lane status bits for conv and verify (padding lanes get 0 and are skipped).
    Only the present nodes' parents are checked; a node count outside [0, N] is an error."""
    slot_ids = np.asarray(slot_ids)
    C, N = np.asarray(parents).shape
    counts = lane_counts(lane_nodes, C, N)
    bits = np.zeros(C, dtype=np.int64)
    for c in range(C):
        s = int(slot_ids[c])
        if s == -1:
            continue
        if s < -1 or s >= n_slots:
            bits[c] |= STATUS_SLOT_RANGE
        if any(int(slot_ids[o]) == s for o in range(C) if o != c):
            bits[c] |= STATUS_SLOT_DUP
        if not 0 <= counts[c] <= N:
            bits[c] |= STATUS_NODES
            continue
        for i in range(counts[c]):
            p = int(parents[c][i])
            if p < -1 or p >= i:
                bits[c] |= STATUS_PARENT
    return bits


# ---------------------------------------------------------------- conv tree step
def conv_tree_step(x, conv_w, conv_hist, slot_ids, parents, conv_out, commit_win, lane_nodes=None):
    """[P1] Optimizations, first bullet; [P5] ssm-conv.cu hunk.

    For lane c with slot s and node i, the extended sequence is the slot's
    history columns (oldest first) followed by the tokens on i's root path.
    conv_out[c,i,ch] = silu(sum_{j=0..3} w[ch,j] * E[-4+j][ch]) and
    commit_win[c,i,ch,:] = E[-3:][ch] (the history the slot would hold if i
    were the last accepted node).  Writes only valid, non-padding lanes and,
    with lane_nodes, only their present nodes i < lane_nodes[c] ([P3] v_len
    commit message: verify runs over the drafted length, not the buffer size);
    returns the OR of the lane status bits.
    """
    x = np.asarray(x)
    C, N, Ch = x.shape
    P = conv_hist.shape[0]
    W = D_CONV - 1
    bits = lane_status(slot_ids, parents, P, lane_nodes)
    counts = lane_counts(lane_nodes, C, N)
    for c in range(C):
        s = int(slot_ids[c])
        if s == -1 or bits[c]:
            continue
        hist_cols = [conv_hist[s][:, j].astype(np.float64) for j in range(W)]
        for i in range(counts[c]):
            ext = hist_cols + [x[c, a].astype(np.float64) for a in root_path(parents[c], i)]
            win = ext[-D_CONV:]
            acc = np.zeros(Ch, dtype=np.float64)
            for j in range(D_CONV):
                acc = acc + conv_w[:, j].astype(np.float64) * win[j]
            conv_out[c, i] = silu(acc)
            commit_win[c, i] = np.stack(ext[-W:], axis=-1)
    return int(np.bitwise_or.reduce(bits)) if C else 0


# ---------------------------------------------------------------- recurrence
def token_step(S, q_raw, k_raw, v, b, a, dt_bias, A):
    """One token of the gated delta rule on a [d_k, d_v] state (float64).

    Returns (S_new, o, g, k_hat, delta):
      q_hat, k_hat = q/|q|, k/|k|; beta, g from the raw gates;
      S' = g*S;  u = S'^T k_hat;  delta = beta*(v - u);  S_new = S' + k_hat delta^T;
      o = S_new^T q_hat / sqrt(d_k).
    """
    d_k = S.shape[0]
    q_hat = l2_normalize(q_raw)
    k_hat = l2_normalize(k_raw)
    beta, g = gates(b, a, dt_bias, A)
    S_dec = g * S
    u = S_dec.T @ k_hat
    delta = beta * (np.asarray(v, np.float64) - u)
    S_new = S_dec + np.outer(k_hat, delta)
    o = (S_new.T @ q_hat) / np.sqrt(d_k)
    return S_new, o, g, k_hat, delta


def split_qkv(row, n_k_heads, n_v_heads, d_k, d_v, h):
    """Channel order q | k | v, each head a contiguous block; value head h reads q/k head h mod H_k."""
    kh = h % n_k_heads
    q = row[kh * d_k:(kh + 1) * d_k]
    k = row[n_k_heads * d_k + kh * d_k: n_k_heads * d_k + (kh + 1) * d_k]
    v0 = 2 * n_k_heads * d_k + h * d_v
    return q, k, row[v0:v0 + d_v]


def tree_verify(qkv, beta_logits, alpha_logits, dt_bias, A, state_pool, slot_ids, parents,
                n_k_heads, out, replay_log, lane_nodes=None):
    """[P1] Optimizations, second and third bullets.

    Per valid lane c (slot s) and value head h, nodes in index order: the
    parent state is the pool state of slot s for root children, else the
    parent node's state; apply token_step.  out[c,i,h] = o,
    replay_log[c,i,h] = (g, k_hat, delta).  state_pool is only read.
    beta_logits / alpha_logits are [C, N, H_v] arrays (the stacked projection's
    two halves).  With lane_nodes only the present nodes i < lane_nodes[c] are
    run and written.  Returns the OR of the lane status bits.
    """
    C, N, _ = qkv.shape
    P, H_v, d_k, d_v = state_pool.shape
    bits = lane_status(slot_ids, parents, P, lane_nodes)
    counts = lane_counts(lane_nodes, C, N)
    for c in range(C):
        s = int(slot_ids[c])
        if s == -1 or bits[c]:
            continue
        for h in range(H_v):
            states = {}
            for i in range(counts[c]):
                p = int(parents[c][i])
                S_par = state_pool[s, h].astype(np.float64) if p == -1 else states[p]
                q, k, v = split_qkv(qkv[c, i].astype(np.float64), n_k_heads, H_v, d_k, d_v, h)
                S_i, o, g, k_hat, delta = token_step(S_par, q, k, v, beta_logits[c, i, h],
                                                     alpha_logits[c, i, h], dt_bias[h], A[h])
                states[i] = S_i
                out[c, i, h] = o
                replay_log[c, i, h, 0] = g
                replay_log[c, i, h, 1:1 + d_k] = k_hat
                replay_log[c, i, h, 1 + d_k:] = delta
    return int(np.bitwise_or.reduce(bits)) if C else 0


# ---------------------------------------------------------------- commit
def commit_preflight(slot_ids, parents, accept_node, n_slots, status_in=0, lane_nodes=None):
    """[P4] transaction preflight: status bits over all non-padding lanes, OR-ed with status_in.
    The accept node must be a present node of its lane (or -1)."""
    C, N = np.asarray(parents).shape
    bits = int(status_in)
    lb = lane_status(slot_ids, parents, n_slots, lane_nodes)
    counts = lane_counts(lane_nodes, C, N)
    for c in range(C):
        if int(slot_ids[c]) == -1:
            continue
        bits |= int(lb[c])
        e = int(accept_node[c])
        if e < -1 or e >= min(max(counts[c], 0), N):
            bits |= STATUS_ACCEPT
    return bits


def replay_commit(replay_log, commit_win, slot_ids, parents, accept_node, state_pool, conv_hist,
                  status_in=0, lane_nodes=None):
    """[P1] closing paragraph; [P4] mechanism 3 and transaction preflight.

    If the preflight (including any bit already in status_in) is clean, every
    non-padding lane with accept node e >= 0 replays the logged transitions of
    e's root path into its slot, S <- g*S + k_hat delta^T (float64), and sets
    the slot's conv history to commit_win[c, e].  Otherwise nothing changes.
    Mutates state_pool / conv_hist in place; returns the status word.
    """
    P, H_v, d_k, d_v = state_pool.shape
    bits = commit_preflight(slot_ids, parents, accept_node, P, status_in, lane_nodes)
    if bits:
        return bits
    for c in range(len(slot_ids)):
        s, e = int(slot_ids[c]), int(accept_node[c])
        if s == -1 or e < 0:
            continue
        path = root_path(parents[c], e)
        for h in range(H_v):
            S = state_pool[s, h].astype(np.float64)
            for t in path:
                row = replay_log[c, t, h].astype(np.float64)
                S = row[0] * S + np.outer(row[1:1 + d_k], row[1 + d_k:])
            state_pool[s, h] = S
        conv_hist[s] = commit_win[c, e]
    return 0


# ---------------------------------------------------------------- plain decode step
def slot_preflight(slot_ids, n_slots, status_in=0):
    """Status bits of a call that mutates the pools directly: slot range and duplicate
    slots over every non-padding lane, OR-ed with status_in."""
    bits = int(status_in)
    C = len(slot_ids)
    for c in range(C):
        s = int(slot_ids[c])
        if s == -1:
            continue
        if s < -1 or s >= n_slots:
            bits |= STATUS_SLOT_RANGE
        if any(int(slot_ids[o]) == s for o in range(C) if o != c):
            bits |= STATUS_SLOT_DUP
    return bits


def conv_step(x, conv_w, conv_hist, slot_ids, conv_out, status_in=0):
    """[P3] DeltaNet-block commit message: the causal-conv step of a decode or chain
    verify (history window, silu(conv), in-place history write-back); [P5] ssm-conv.cu hunk.

    x[c] holds a chain of N tokens for lane c (slot s).  With E the slot's history
    columns followed by x[c, 0..N-1], conv_out[c, t] = silu(sum_j w[:, j] * E[t + j])
    (the window ending at token t), and afterwards conv_hist[s] holds the last 3
    columns of E.  If the preflight (slot range, duplicate slots, status_in) is not
    clean nothing is written at all.  Mutates conv_hist / conv_out in place; returns
    the status word.
    """
    x = np.asarray(x)
    C, N, Ch = x.shape
    W = D_CONV - 1
    bits = slot_preflight(slot_ids, conv_hist.shape[0], status_in)
    if bits:
        return bits
    for c in range(C):
        s = int(slot_ids[c])
        if s == -1:
            continue
        cols = [conv_hist[s][:, j].astype(np.float64) for j in range(W)]
        cols += [x[c, t].astype(np.float64) for t in range(N)]
        for t in range(N):
            acc = np.zeros(Ch, dtype=np.float64)
            for j in range(D_CONV):
                acc = acc + conv_w[:, j].astype(np.float64) * cols[t + j]
            conv_out[c, t] = silu(acc)
        conv_hist[s] = np.stack(cols[-W:], axis=-1)
    return 0


def decode_step(qkv, beta_logits, alpha_logits, dt_bias, A, state_pool, slot_ids, n_k_heads, out, status_in=0):
    """[P2] deferred-state commit message (a step without a draft commits its state at
    once); [P3] raw-gate gated delta rule applied in place, no state copy.

    One token per lane: qkv[c] is lane c's conv output row, beta_logits / alpha_logits
    are [C, H_v].  For every non-padding lane (slot s) and value head h, token_step on
    state_pool[s, h] replaces it in place and out[c, h] = o.  If the preflight (slot
    range, duplicate slots, status_in) is not clean nothing is written at all.
    Returns the status word.
    """
    P, H_v, d_k, d_v = state_pool.shape
    bits = slot_preflight(slot_ids, P, status_in)
    if bits:
        return bits
    for c in range(len(slot_ids)):
        s = int(slot_ids[c])
        if s == -1:
            continue
        for h in range(H_v):
            q, k, v = split_qkv(np.asarray(qkv[c], np.float64), n_k_heads, H_v, d_k, d_v, h)
            S_new, o, _, _, _ = token_step(state_pool[s, h].astype(np.float64), q, k, v, beta_logits[c, h],
                                           alpha_logits[c, h], dt_bias[h], A[h])
            state_pool[s, h] = S_new
            out[c, h] = o
    return 0


# ---------------------------------------------------------------- prefill
def output_gate(o, z, gate_mode):
    """[P2] chunked-GDN commit message: the kernel closes with a SiLU (gate_mode 0) or a
    sigmoid (gate_mode 1) gate on the output: o * silu(z) or o * sigmoid(z)."""
    z = np.asarray(z, np.float64)
    return o * (silu(z) if gate_mode == 0 else sigmoid(z))


def prefill(qkv, beta_logits, alpha_logits, dt_bias, A, state_pool, slot_ids, n_k_heads, out, gate_z=None,
            gate_mode=0, status_in=0):
    """[P2] chunked-GDN commit message (the recurrence over a prompt's tokens, with an
    optional closing output gate); [P3] raw-gate commit message.

    qkv[c] holds the conv output rows of a chain of T tokens for lane c (slot s);
    beta_logits / alpha_logits are [C, T, H_v].  For every non-padding lane and value
    head h, token_step over the tokens in order, starting from and replacing
    state_pool[s, h] in place; out[c, t, h] = o, times act(gate_z[c, t, h]) when a gate
    is given (output_gate).  A transaction like decode_step: nothing is written unless
    the slot preflight and status_in are clean.  Returns the status word.
    """
    P, H_v, d_k, d_v = state_pool.shape
    bits = slot_preflight(slot_ids, P, status_in)
    if bits:
        return bits
    C, T, _ = qkv.shape
    for c in range(C):
        s = int(slot_ids[c])
        if s == -1:
            continue
        for h in range(H_v):
            S = state_pool[s, h].astype(np.float64)
            for t in range(T):
                q, k, v = split_qkv(np.asarray(qkv[c, t], np.float64), n_k_heads, H_v, d_k, d_v, h)
                S, o, _, _, _ = token_step(S, q, k, v, beta_logits[c, t, h], alpha_logits[c, t, h], dt_bias[h], A[h])
                out[c, t, h] = o if gate_z is None else output_gate(o, gate_z[c, t, h], gate_mode)
            state_pool[s, h] = S
    return 0


def new_outputs(C, N, Ch, H_v, d_k, d_v, fill=np.nan):
    """float64 output arrays pre-filled with `fill` (untouched lanes keep it)."""
    W = D_CONV - 1
    return dict(
        conv_out=np.full((C, N, Ch), fill),
        commit_win=np.full((C, N, Ch, W), fill),
        out=np.full((C, N, H_v, d_v), fill),
        replay_log=np.full((C, N, H_v, 1 + d_k + d_v), fill),
    )


def verify_round(x, ba, conv_w, conv_hist, state_pool, dt_bias, A, slot_ids, parents, n_k_heads,
                 lane_nodes=None):
    """Conv then verify for one layer of one round; returns the float64 outputs and status."""
    C, N, Ch = x.shape
    P, H_v, d_k, d_v = state_pool.shape
    o = new_outputs(C, N, Ch, H_v, d_k, d_v)
    st = conv_tree_step(x, conv_w, conv_hist, slot_ids, parents, o["conv_out"], o["commit_win"], lane_nodes)
    st |= tree_verify(o["conv_out"], ba[:, :, :H_v], ba[:, :, H_v:], dt_bias, A, state_pool,
                      slot_ids, parents, n_k_heads, o["out"], o["replay_log"], lane_nodes)
    o["status"] = st
    return o
