"""Helpers for the GPU parity tests: move seeded inputs to the device, run the HIP
route through the C ABI, run the oracle on the same float32 inputs, compare."""

from __future__ import annotations

import sys

import numpy as np
import torch

import gated_deltanet_speculative_amd as gdn
from oracle import gdn_oracle as O

SENTINEL = -7.25e33  # fill of untouched outputs and guard bands
GUARD = 4096  # floats of guard band on each side of every output buffer


def log(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def err_metric(gpu: np.ndarray, ref: np.ndarray) -> float:
    """max |g - r| / max(1, |r|), the tolerance metric for float outputs."""
    gpu = np.asarray(gpu, np.float64)
    ref = np.asarray(ref, np.float64)
    assert gpu.shape == ref.shape
    if gpu.size == 0:
        return 0.0
    assert np.isfinite(gpu).all(), "non-finite GPU output"
    return float(np.max(np.abs(gpu - ref) / np.maximum(1.0, np.abs(ref))))


class Guarded:
    """A device buffer with sentinel guard bands on both sides; .t is the payload view."""

    def __init__(self, shape, dtype=torch.float32, fill=SENTINEL):
        n = int(np.prod(shape))
        self.base = torch.full((n + 2 * GUARD,), fill, dtype=dtype, device="cuda")
        self.t = self.base[GUARD:GUARD + n].view(*shape)
        self.fill = fill

    def guards_intact(self) -> bool:
        b = self.base.cpu()
        ref = torch.full((GUARD,), self.fill, dtype=b.dtype)
        return bool(torch.equal(b[:GUARD], ref) and torch.equal(b[-GUARD:], ref))

    def np(self) -> np.ndarray:
        return self.t.cpu().numpy()


def dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda")


def shape_of(C, N, P, Hk, Hv, dk, dv) -> gdn.Shape:
    return gdn.Shape(C, N, P, Hk, Hv, dk, dv)


class GpuRound:
    """Device copies of one layer's inputs plus guarded outputs; runs conv, verify, commit."""

    def __init__(self, sh: gdn.Shape, x, ba, conv_w, conv_hist, state, dt_bias, A, slot_ids, parents, fused=False,
                 lane_nodes=None):
        self.sh = sh
        self.fused = fused  # verify() runs the fused conv + verify call instead of the two separate calls
        self.lane_nodes = None if lane_nodes is None else dev(np.asarray(lane_nodes, np.int32))
        C, N, Ch, Hv = sh.n_seqs, sh.n_nodes, sh.channels, sh.n_v_heads
        self.x, self.ba, self.conv_w = dev(x), dev(ba), dev(conv_w)
        self.conv_hist, self.state = dev(conv_hist), dev(state)
        self.dt_bias, self.A = dev(dt_bias), dev(A)
        self.slot_ids, self.parents = dev(slot_ids.astype(np.int32)), dev(parents.astype(np.int32))
        self.conv_out = Guarded((C, N, Ch))
        self.commit_win = Guarded((C, N, Ch, 3))
        self.out = Guarded((C, N, Hv, sh.d_v))
        self.replay_log = Guarded((C, N, Hv, sh.log_row))
        self.status = torch.zeros(1, dtype=torch.int32, device="cuda")

    def verify(self):
        sh = self.sh
        Hv = sh.n_v_heads
        if self.fused:
            gdn.conv_tree_verify(sh, self.x, self.conv_w, self.conv_hist, self.ba[..., :Hv], self.ba[..., Hv:],
                                 self.dt_bias, self.A, self.state, self.slot_ids, self.parents, out=self.out.t,
                                 replay_log=self.replay_log.t, commit_win=self.commit_win.t, status=self.status,
                                 lane_nodes=self.lane_nodes)
            return self
        gdn.conv_tree_step(sh, self.x, self.conv_w, self.conv_hist, self.slot_ids, self.parents,
                           conv_out=self.conv_out.t, commit_win=self.commit_win.t, status=self.status,
                           lane_nodes=self.lane_nodes)
        gdn.tree_verify(sh, self.conv_out.t, self.ba[..., :Hv], self.ba[..., Hv:], self.dt_bias, self.A,
                        self.state, self.slot_ids, self.parents, out=self.out.t, replay_log=self.replay_log.t,
                        status=self.status, lane_nodes=self.lane_nodes)
        return self

    def commit(self, accept_node):
        gdn.replay_commit(self.sh, self.replay_log.t, self.commit_win.t, self.slot_ids, self.parents,
                          dev(np.asarray(accept_node, np.int32)), self.state, self.conv_hist, self.status,
                          lane_nodes=self.lane_nodes)
        return self

    def guards_intact(self) -> bool:
        return all(b.guards_intact() for b in (self.conv_out, self.commit_win, self.out, self.replay_log))


def oracle_round(sh, x, ba, conv_w, conv_hist, state, dt_bias, A, slot_ids, parents, lane_nodes=None):
    return O.verify_round(x, ba, conv_w, conv_hist, state, dt_bias, A, np.asarray(slot_ids, np.int32),
                          np.asarray(parents, np.int32), sh.n_k_heads, lane_nodes)


def oracle_commit(sh, ref, slot_ids, parents, accept, state, conv_hist, status_in=0, lane_nodes=None):
    pool = state.astype(np.float64)
    hist = conv_hist.astype(np.float64)
    st = O.replay_commit(ref["replay_log"], ref["commit_win"], np.asarray(slot_ids, np.int32),
                         np.asarray(parents, np.int32), np.asarray(accept, np.int32), pool, hist, status_in,
                         lane_nodes)
    return st, pool, hist


def compare_verify(g: GpuRound, ref: dict, lanes=None, ref_is_subset=False, conv_tol=1e-5, rec_tol=2e-4) -> dict:
    """Element-wise comparison of the GPU lanes `lanes` (all if None) with the oracle's;
    `ref_is_subset` means the oracle ran on exactly those lanes."""
    sel = lanes if isinstance(lanes, slice) else (slice(None) if lanes is None else np.asarray(lanes))
    rsel = slice(None) if ref_is_subset else sel
    co, cw = g.conv_out.np()[sel], g.commit_win.np()[sel]
    out, lg = g.out.np()[sel], g.replay_log.np()[sel]
    ref = {k: (v[rsel] if isinstance(v, np.ndarray) else v) for k, v in ref.items()}
    sel = slice(None)
    if g.fused:  # the fused call keeps the conv output on chip: its buffer stays untouched
        assert (co == np.float32(SENTINEL)).all(), "fused route wrote conv_out"
        e_conv = 0.0
    else:
        e_conv = err_metric(co, ref["conv_out"][sel])
        assert e_conv <= conv_tol, f"conv_out error {e_conv}"
    ref_win = ref["commit_win"][sel].astype(np.float32)
    assert np.array_equal(cw, ref_win), "commit windows differ (must be bit-exact copies)"
    e_out = err_metric(out, ref["out"][sel])
    e_log = err_metric(lg, ref["replay_log"][sel])
    assert e_out <= rec_tol, f"out error {e_out}"
    assert e_log <= rec_tol, f"replay_log error {e_log}"
    return dict(conv=e_conv, out=e_out, log=e_log)
