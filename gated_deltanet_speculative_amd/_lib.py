"""ctypes binding of libgdnverify.so: argument marshalling only.

Every step of the route runs in the library's HIP kernels.  torch provides the
device memory (tensors) and the stream (torch's current stream); this module
checks tensor shapes, dtypes, devices and layouts, allocates missing outputs,
and passes raw pointers and the stream to the C ABI.  There is no fallback: if
the library is missing or a call fails, an exception is raised.
"""

from __future__ import annotations

import ctypes
import os
from typing import NamedTuple, Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libgdnverify.so")

(GDN_OK, GDN_ERR_NULL, GDN_ERR_SHAPE, GDN_ERR_UNSUPPORTED, GDN_ERR_ALIAS, GDN_ERR_HIP, GDN_ERR_ALIGN,
 GDN_ERR_WORKSPACE, GDN_ERR_SCRATCH) = range(9)
STATUS_SLOT_RANGE, STATUS_SLOT_DUP, STATUS_PARENT, STATUS_ACCEPT, STATUS_NODES = 1, 2, 4, 8, 16
EXPORTED = ("gdn_conv_tree_step", "gdn_tree_verify", "gdn_conv_tree_verify", "gdn_replay_commit",
            "gdn_replay_commit_layers", "gdn_conv_step", "gdn_decode_step", "gdn_conv_decode_step", "gdn_prefill",
            "gdn_prefill_workspace_size", "gdn_prefill_noalloc", "gdn_strerror")
MAX_CHAIN = 65536
MAX_LAYERS = 64
SYNC_STRIDE = 32  # int32 per counter of conv_decode_step (one 128-byte line)


class GdnError(RuntimeError):
    def __init__(self, code: int, where: str):
        self.code = code
        super().__init__(f"{where}: {strerror(code)} (code {code})")


class _CShape(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in
                ("n_seqs", "n_nodes", "n_slots", "n_k_heads", "n_v_heads", "d_k", "d_v", "d_conv")]


class Shape(NamedTuple):
    n_seqs: int
    n_nodes: int
    n_slots: int
    n_k_heads: int
    n_v_heads: int
    d_k: int
    d_v: int
    d_conv: int = 4

    @property
    def channels(self) -> int:
        return 2 * self.n_k_heads * self.d_k + self.n_v_heads * self.d_v

    @property
    def log_row(self) -> int:
        return 1 + self.d_k + self.d_v

    def c_struct(self) -> _CShape:
        return _CShape(*[int(v) for v in self])


_lib = None


def load_library(path: Optional[str] = None) -> ctypes.CDLL:
    """Load (once) and return the C-ABI library; raises if it has not been built."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise RuntimeError(f"{p} is missing: build it with `python -m gated_deltanet_speculative_amd.build`")
    lib = ctypes.CDLL(p)
    vp, i32, i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
    sp = ctypes.POINTER(_CShape)
    lib.gdn_conv_tree_step.argtypes = [sp] + [vp] * 10
    lib.gdn_tree_verify.argtypes = [sp, vp, vp, vp, i64] + [vp] * 10
    lib.gdn_conv_tree_verify.argtypes = [sp, vp, vp, vp, vp, vp, i64] + [vp] * 11
    lib.gdn_replay_commit.argtypes = [sp] + [vp] * 10
    lib.gdn_replay_commit_layers.argtypes = [sp, i32] + [vp] * 10
    lib.gdn_conv_step.argtypes = [sp] + [vp] * 7
    lib.gdn_decode_step.argtypes = [sp, vp, vp, vp, i64] + [vp] * 7
    lib.gdn_conv_decode_step.argtypes = [sp, vp, vp, vp, vp, vp, i64] + [vp] * 8
    lib.gdn_prefill.argtypes = [sp, vp, vp, vp, i64, vp, vp, vp, vp, vp, i32, vp, vp, ctypes.c_size_t, vp, vp]
    lib.gdn_prefill_noalloc.argtypes = [sp, vp, vp, vp, i64, vp, vp, vp, vp, vp, i32, vp, vp, vp]
    lib.gdn_prefill_workspace_size.argtypes = [sp]
    lib.gdn_prefill_workspace_size.restype = ctypes.c_size_t
    for f in ("gdn_conv_tree_step", "gdn_tree_verify", "gdn_conv_tree_verify", "gdn_replay_commit",
              "gdn_replay_commit_layers", "gdn_conv_step", "gdn_decode_step", "gdn_conv_decode_step", "gdn_prefill",
              "gdn_prefill_noalloc"):
        getattr(lib, f).restype = i32
    lib.gdn_strerror.argtypes = [ctypes.c_int]
    lib.gdn_strerror.restype = ctypes.c_char_p
    if path is None:
        _lib = lib
    return lib


def strerror(code: int) -> str:
    return load_library().gdn_strerror(int(code)).decode()


# ---------------------------------------------------------------- marshalling helpers
def _dev(t: torch.Tensor, name: str, dtype: torch.dtype, shape: tuple) -> int:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name}: expected {dtype}, got {t.dtype}")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a device tensor")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: expected shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.data_ptr()


def _gate_view(t: torch.Tensor, name: str, sh: Shape) -> tuple:
    """A [C, N, H_v] float32 view whose rows are `gate_stride` floats apart (e.g. one half
    of the stacked beta|alpha projection).  Returns (pointer, gate_stride)."""
    if t.dtype != torch.float32 or t.device.type != "cuda":
        raise TypeError(f"{name} must be a float32 device tensor")
    C, N, Hv = sh.n_seqs, sh.n_nodes, sh.n_v_heads
    if tuple(t.shape) != (C, N, Hv):
        raise ValueError(f"{name}: expected shape {(C, N, Hv)}, got {tuple(t.shape)}")
    s0, s1, s2 = t.stride()
    if s2 != 1:
        raise ValueError(f"{name}: heads of one token must be contiguous")
    if N > 1:
        stride = s1
        if C > 1 and s0 != N * s1:
            raise ValueError(f"{name}: token rows must be evenly strided across lanes")
    elif C > 1:
        stride = s0
    else:
        stride = Hv
    return t.data_ptr(), int(stride)


def _counts(lane_nodes, sh: Shape):
    """Pointer to the per-lane node counts ([C] int32 device tensor), or None (every lane has N nodes)."""
    return None if lane_nodes is None else _dev(lane_nodes, "lane_nodes", torch.int32, (sh.n_seqs,))


def _stream(t: torch.Tensor) -> int:
    return torch.cuda.current_stream(t.device).cuda_stream


def _check(code: int, where: str) -> None:
    if code != GDN_OK:
        raise GdnError(code, where)


def _status(status: Optional[torch.Tensor], like: torch.Tensor) -> torch.Tensor:
    if status is None:
        return torch.zeros(1, dtype=torch.int32, device=like.device)
    _dev(status, "status", torch.int32, (1,))
    return status


# ---------------------------------------------------------------- the three calls
def conv_tree_step(sh: Shape, x, conv_w, conv_hist, slot_ids, parents, conv_out=None, commit_win=None,
                   status=None, lane_nodes=None):
    """Tree conv + SiLU and commit windows; returns (conv_out, commit_win, status).
    lane_nodes ([C] int32, optional): nodes present per lane (ragged lanes)."""
    C, N, P, Ch = sh.n_seqs, sh.n_nodes, sh.n_slots, sh.channels
    if conv_out is None:
        conv_out = torch.empty((C, N, Ch), dtype=torch.float32, device=x.device)
    if commit_win is None:
        commit_win = torch.empty((C, N, Ch, 3), dtype=torch.float32, device=x.device)
    status = _status(status, x)
    args = [
        _dev(x, "x", torch.float32, (C, N, Ch)),
        _dev(conv_w, "conv_w", torch.float32, (Ch, sh.d_conv)),
        _dev(conv_hist, "conv_hist", torch.float32, (P, Ch, sh.d_conv - 1)),
        _dev(slot_ids, "slot_ids", torch.int32, (C,)),
        _dev(parents, "parents", torch.int32, (C, N)),
        _counts(lane_nodes, sh),
        _dev(conv_out, "conv_out", torch.float32, (C, N, Ch)),
        _dev(commit_win, "commit_win", torch.float32, (C, N, Ch, sh.d_conv - 1)),
        status.data_ptr(),
        _stream(x),
    ]
    cs = sh.c_struct()
    _check(load_library().gdn_conv_tree_step(ctypes.byref(cs), *args), "gdn_conv_tree_step")
    return conv_out, commit_win, status


def tree_verify(sh: Shape, qkv, beta_logits, alpha_logits, dt_bias, A, state_pool, slot_ids, parents, out=None,
                replay_log=None, status=None, lane_nodes=None):
    """Read-only tree verify; beta/alpha logits are [C, N, H_v] views sharing one row stride
    (e.g. ba[..., :H_v] and ba[..., H_v:] of the stacked projection).  Returns (out, replay_log, status)."""
    C, N, P, Hv, dk, dv = sh.n_seqs, sh.n_nodes, sh.n_slots, sh.n_v_heads, sh.d_k, sh.d_v
    if out is None:
        out = torch.empty((C, N, Hv, dv), dtype=torch.float32, device=qkv.device)
    if replay_log is None:
        replay_log = torch.empty((C, N, Hv, sh.log_row), dtype=torch.float32, device=qkv.device)
    status = _status(status, qkv)
    bp, bs = _gate_view(beta_logits, "beta_logits", sh)
    ap, as_ = _gate_view(alpha_logits, "alpha_logits", sh)
    if bs != as_:
        raise ValueError("beta_logits and alpha_logits must share one row stride")
    args = [
        _dev(qkv, "qkv", torch.float32, (C, N, sh.channels)), bp, ap, bs,
        _dev(dt_bias, "dt_bias", torch.float32, (Hv,)),
        _dev(A, "A", torch.float32, (Hv,)),
        _dev(state_pool, "state_pool", torch.float32, (P, Hv, dk, dv)),
        _dev(slot_ids, "slot_ids", torch.int32, (C,)),
        _dev(parents, "parents", torch.int32, (C, N)),
        _counts(lane_nodes, sh),
        _dev(out, "out", torch.float32, (C, N, Hv, dv)),
        _dev(replay_log, "replay_log", torch.float32, (C, N, Hv, sh.log_row)),
        status.data_ptr(),
        _stream(qkv),
    ]
    cs = sh.c_struct()
    _check(load_library().gdn_tree_verify(ctypes.byref(cs), *args), "gdn_tree_verify")
    return out, replay_log, status


def conv_tree_verify(sh: Shape, x, conv_w, conv_hist, beta_logits, alpha_logits, dt_bias, A, state_pool, slot_ids,
                     parents, out=None, replay_log=None, commit_win=None, status=None, lane_nodes=None):
    """Fused tree conv + verify (the conv output stays on chip).  Returns
    (out, replay_log, commit_win, status)."""
    C, N, P, Hv, dk, dv, Ch = sh.n_seqs, sh.n_nodes, sh.n_slots, sh.n_v_heads, sh.d_k, sh.d_v, sh.channels
    if out is None:
        out = torch.empty((C, N, Hv, dv), dtype=torch.float32, device=x.device)
    if replay_log is None:
        replay_log = torch.empty((C, N, Hv, sh.log_row), dtype=torch.float32, device=x.device)
    if commit_win is None:
        commit_win = torch.empty((C, N, Ch, sh.d_conv - 1), dtype=torch.float32, device=x.device)
    status = _status(status, x)
    bp, bs = _gate_view(beta_logits, "beta_logits", sh)
    ap, as_ = _gate_view(alpha_logits, "alpha_logits", sh)
    if bs != as_:
        raise ValueError("beta_logits and alpha_logits must share one row stride")
    args = [
        _dev(x, "x", torch.float32, (C, N, Ch)),
        _dev(conv_w, "conv_w", torch.float32, (Ch, sh.d_conv)),
        _dev(conv_hist, "conv_hist", torch.float32, (P, Ch, sh.d_conv - 1)),
        bp, ap, bs,
        _dev(dt_bias, "dt_bias", torch.float32, (Hv,)),
        _dev(A, "A", torch.float32, (Hv,)),
        _dev(state_pool, "state_pool", torch.float32, (P, Hv, dk, dv)),
        _dev(slot_ids, "slot_ids", torch.int32, (C,)),
        _dev(parents, "parents", torch.int32, (C, N)),
        _counts(lane_nodes, sh),
        _dev(out, "out", torch.float32, (C, N, Hv, dv)),
        _dev(replay_log, "replay_log", torch.float32, (C, N, Hv, sh.log_row)),
        _dev(commit_win, "commit_win", torch.float32, (C, N, Ch, sh.d_conv - 1)),
        status.data_ptr(),
        _stream(x),
    ]
    cs = sh.c_struct()
    _check(load_library().gdn_conv_tree_verify(ctypes.byref(cs), *args), "gdn_conv_tree_verify")
    return out, replay_log, commit_win, status


def replay_commit(sh: Shape, replay_log, commit_win, slot_ids, parents, accept_node, state_pool, conv_hist,
                  status, lane_nodes=None):
    """Preflight + replay commit in place on state_pool / conv_hist; returns status."""
    C, N, P, Hv, dk, dv, Ch = sh.n_seqs, sh.n_nodes, sh.n_slots, sh.n_v_heads, sh.d_k, sh.d_v, sh.channels
    if status is None:
        raise ValueError("replay_commit needs a status word (the round's transaction flag)")
    args = [
        _dev(replay_log, "replay_log", torch.float32, (C, N, Hv, sh.log_row)),
        _dev(commit_win, "commit_win", torch.float32, (C, N, Ch, sh.d_conv - 1)),
        _dev(slot_ids, "slot_ids", torch.int32, (C,)),
        _dev(parents, "parents", torch.int32, (C, N)),
        _counts(lane_nodes, sh),
        _dev(accept_node, "accept_node", torch.int32, (C,)),
        _dev(state_pool, "state_pool", torch.float32, (P, Hv, dk, dv)),
        _dev(conv_hist, "conv_hist", torch.float32, (P, Ch, sh.d_conv - 1)),
        _dev(status, "status", torch.int32, (1,)),
        _stream(state_pool),
    ]
    cs = sh.c_struct()
    _check(load_library().gdn_replay_commit(ctypes.byref(cs), *args), "gdn_replay_commit")
    return status


def replay_commit_layers(sh: Shape, replay_logs, commit_wins, slot_ids, parents, accept_node, state_pools,
                         conv_hists, status, lane_nodes=None):
    """Preflight + replay commit of every layer of the round in one launch.

    replay_logs, commit_wins, state_pools and conv_hists are equal-length sequences
    (one entry per layer) of tensors laid out as for replay_commit; slot_ids,
    parents, accept_node and the status word are shared.  All layers commit or none.
    """
    C, N, P, Hv, dk, dv, Ch = sh.n_seqs, sh.n_nodes, sh.n_slots, sh.n_v_heads, sh.d_k, sh.d_v, sh.channels
    if status is None:
        raise ValueError("replay_commit_layers needs a status word (the round's transaction flag)")
    L = len(replay_logs)
    if not (len(commit_wins) == len(state_pools) == len(conv_hists) == L):
        raise ValueError("replay_commit_layers: per-layer sequences differ in length")
    if not 1 <= L <= MAX_LAYERS:
        raise ValueError(f"replay_commit_layers: {L} layers, expected 1..{MAX_LAYERS}")
    arr = ctypes.c_void_p * L
    logs = arr(*[_dev(t, f"replay_logs[{l}]", torch.float32, (C, N, Hv, sh.log_row)) for l, t in enumerate(replay_logs)])
    wins = arr(*[_dev(t, f"commit_wins[{l}]", torch.float32, (C, N, Ch, sh.d_conv - 1))
                 for l, t in enumerate(commit_wins)])
    pools = arr(*[_dev(t, f"state_pools[{l}]", torch.float32, (P, Hv, dk, dv)) for l, t in enumerate(state_pools)])
    hists = arr(*[_dev(t, f"conv_hists[{l}]", torch.float32, (P, Ch, sh.d_conv - 1)) for l, t in enumerate(conv_hists)])
    args = [
        ctypes.cast(logs, ctypes.c_void_p), ctypes.cast(wins, ctypes.c_void_p),
        _dev(slot_ids, "slot_ids", torch.int32, (C,)),
        _dev(parents, "parents", torch.int32, (C, N)),
        _counts(lane_nodes, sh),
        _dev(accept_node, "accept_node", torch.int32, (C,)),
        ctypes.cast(pools, ctypes.c_void_p), ctypes.cast(hists, ctypes.c_void_p),
        _dev(status, "status", torch.int32, (1,)),
        _stream(state_pools[0]),
    ]
    cs = sh.c_struct()
    _check(load_library().gdn_replay_commit_layers(ctypes.byref(cs), ctypes.c_int32(L), *args),
           "gdn_replay_commit_layers")
    return status


# ---------------------------------------------------------------- plain decode step
def _row_gate_view(t: torch.Tensor, name: str, sh: Shape) -> tuple:
    """A [C, H_v] float32 view whose lane rows are `gate_stride` floats apart (e.g. one half
    of the stacked beta|alpha projection of a one-token step).  Returns (pointer, stride)."""
    if t.dtype != torch.float32 or t.device.type != "cuda":
        raise TypeError(f"{name} must be a float32 device tensor")
    C, Hv = sh.n_seqs, sh.n_v_heads
    if tuple(t.shape) != (C, Hv):
        raise ValueError(f"{name}: expected shape {(C, Hv)}, got {tuple(t.shape)}")
    s0, s1 = t.stride()
    if s1 != 1:
        raise ValueError(f"{name}: heads of one lane must be contiguous")
    return t.data_ptr(), int(s0 if C > 1 else Hv)


def conv_step(sh: Shape, x, conv_w, conv_hist, slot_ids, status, conv_out=None):
    """Causal conv + SiLU over a chain of n_nodes tokens per lane, writing each slot's new
    history into conv_hist in place (a transaction on the status word).  Returns conv_out."""
    C, N, P, Ch = sh.n_seqs, sh.n_nodes, sh.n_slots, sh.channels
    if status is None:
        raise ValueError("conv_step needs a status word (it mutates the history pool)")
    if conv_out is None:
        conv_out = torch.empty((C, N, Ch), dtype=torch.float32, device=x.device)
    args = [
        _dev(x, "x", torch.float32, (C, N, Ch)),
        _dev(conv_w, "conv_w", torch.float32, (Ch, sh.d_conv)),
        _dev(conv_hist, "conv_hist", torch.float32, (P, Ch, sh.d_conv - 1)),
        _dev(slot_ids, "slot_ids", torch.int32, (C,)),
        _dev(conv_out, "conv_out", torch.float32, (C, N, Ch)),
        _dev(status, "status", torch.int32, (1,)),
        _stream(x),
    ]
    cs = sh.c_struct()
    _check(load_library().gdn_conv_step(ctypes.byref(cs), *args), "gdn_conv_step")
    return conv_out


def decode_step(sh: Shape, qkv, beta_logits, alpha_logits, dt_bias, A, state_pool, slot_ids, status, out=None):
    """One token of the recurrence per lane applied to the slots' states in place (n_nodes
    must be 1).  qkv is [C, Ch]; beta/alpha logits are [C, H_v] views sharing one row
    stride.  A transaction on the status word.  Returns out [C, H_v, d_v]."""
    C, P, Hv, dk, dv = sh.n_seqs, sh.n_slots, sh.n_v_heads, sh.d_k, sh.d_v
    if status is None:
        raise ValueError("decode_step needs a status word (it mutates the state pool)")
    if out is None:
        out = torch.empty((C, Hv, dv), dtype=torch.float32, device=qkv.device)
    bp, bs = _row_gate_view(beta_logits, "beta_logits", sh)
    ap, as_ = _row_gate_view(alpha_logits, "alpha_logits", sh)
    if bs != as_:
        raise ValueError("beta_logits and alpha_logits must share one row stride")
    args = [
        _dev(qkv, "qkv", torch.float32, (C, sh.channels)), bp, ap, bs,
        _dev(dt_bias, "dt_bias", torch.float32, (Hv,)),
        _dev(A, "A", torch.float32, (Hv,)),
        _dev(state_pool, "state_pool", torch.float32, (P, Hv, dk, dv)),
        _dev(slot_ids, "slot_ids", torch.int32, (C,)),
        _dev(out, "out", torch.float32, (C, Hv, dv)),
        _dev(status, "status", torch.int32, (1,)),
        _stream(qkv),
    ]
    cs = sh.c_struct()
    _check(load_library().gdn_decode_step(ctypes.byref(cs), *args), "gdn_decode_step")
    return out


def conv_decode_step(sh: Shape, x, conv_w, conv_hist, beta_logits, alpha_logits, dt_bias, A, state_pool, slot_ids,
                     sync, status, out=None):
    """conv_step over one token per lane and decode_step on its output, in one launch (the
    same results; n_nodes must be 1).  x is [C, Ch]; sync is a [C, H_k, SYNC_STRIDE] int32
    array that is zero on entry and left zero (not shared by calls that overlap).  A transaction on the
    status word.  Returns out [C, H_v, d_v]."""
    C, P, Hk, Hv, dk, dv, Ch = sh.n_seqs, sh.n_slots, sh.n_k_heads, sh.n_v_heads, sh.d_k, sh.d_v, sh.channels
    if status is None:
        raise ValueError("conv_decode_step needs a status word (it mutates the pools)")
    if out is None:
        out = torch.empty((C, Hv, dv), dtype=torch.float32, device=x.device)
    bp, bs = _row_gate_view(beta_logits, "beta_logits", sh)
    ap, as_ = _row_gate_view(alpha_logits, "alpha_logits", sh)
    if bs != as_:
        raise ValueError("beta_logits and alpha_logits must share one row stride")
    args = [
        _dev(x, "x", torch.float32, (C, Ch)),
        _dev(conv_w, "conv_w", torch.float32, (Ch, sh.d_conv)),
        _dev(conv_hist, "conv_hist", torch.float32, (P, Ch, sh.d_conv - 1)),
        bp, ap, bs,
        _dev(dt_bias, "dt_bias", torch.float32, (Hv,)),
        _dev(A, "A", torch.float32, (Hv,)),
        _dev(state_pool, "state_pool", torch.float32, (P, Hv, dk, dv)),
        _dev(slot_ids, "slot_ids", torch.int32, (C,)),
        _dev(sync, "sync", torch.int32, (C, Hk, SYNC_STRIDE)),
        _dev(out, "out", torch.float32, (C, Hv, dv)),
        _dev(status, "status", torch.int32, (1,)),
        _stream(x),
    ]
    cs = sh.c_struct()
    _check(load_library().gdn_conv_decode_step(ctypes.byref(cs), *args), "gdn_conv_decode_step")
    return out


# ---------------------------------------------------------------- prefill
def prefill_workspace_size(sh: Shape) -> int:
    """Bytes of device workspace prefill needs for this shape (0 for an invalid shape)."""
    cs = sh.c_struct()
    return int(load_library().gdn_prefill_workspace_size(ctypes.byref(cs)))


def prefill(sh: Shape, qkv, beta_logits, alpha_logits, dt_bias, A, state_pool, slot_ids, status, gate_z=None,
            gate_mode=0, out=None, workspace=None):
    """The recurrence over a chain of n_nodes tokens per lane (qkv [C, T, Ch] = the conv
    output of the prompt), updating the slots' states in place; beta/alpha logits are
    [C, T, H_v] views sharing one row stride.  With gate_z ([C, T, H_v, d_v]) the output is
    gated by silu(z) (gate_mode 0) or sigmoid(z) (gate_mode 1).  A transaction on the
    status word.  `workspace` is a float32 device tensor of at least
    prefill_workspace_size(sh) bytes (allocated per call when omitted).
    Returns out [C, T, H_v, d_v]."""
    C, T, P, Hv, dk, dv = sh.n_seqs, sh.n_nodes, sh.n_slots, sh.n_v_heads, sh.d_k, sh.d_v
    if status is None:
        raise ValueError("prefill needs a status word (it mutates the state pool)")
    if out is None:
        out = torch.empty((C, T, Hv, dv), dtype=torch.float32, device=qkv.device)
    ws_bytes = prefill_workspace_size(sh)
    if workspace is None:
        workspace = torch.empty(max(ws_bytes // 4, 1), dtype=torch.float32, device=qkv.device)
    if not (isinstance(workspace, torch.Tensor) and workspace.dtype == torch.float32 and workspace.is_cuda
            and workspace.is_contiguous()):
        raise ValueError("workspace must be a contiguous float32 device tensor")
    bp, bs = _gate_view(beta_logits, "beta_logits", sh)
    ap, as_ = _gate_view(alpha_logits, "alpha_logits", sh)
    if bs != as_:
        raise ValueError("beta_logits and alpha_logits must share one row stride")
    args = [
        _dev(qkv, "qkv", torch.float32, (C, T, sh.channels)), bp, ap, bs,
        _dev(dt_bias, "dt_bias", torch.float32, (Hv,)),
        _dev(A, "A", torch.float32, (Hv,)),
        _dev(state_pool, "state_pool", torch.float32, (P, Hv, dk, dv)),
        _dev(slot_ids, "slot_ids", torch.int32, (C,)),
        None if gate_z is None else _dev(gate_z, "gate_z", torch.float32, (C, T, Hv, dv)),
        ctypes.c_int32(int(gate_mode)),
        _dev(out, "out", torch.float32, (C, T, Hv, dv)),
        workspace.data_ptr(), ctypes.c_size_t(workspace.numel() * 4),
        _dev(status, "status", torch.int32, (1,)),
        _stream(qkv),
    ]
    cs = sh.c_struct()
    _check(load_library().gdn_prefill(ctypes.byref(cs), *args), "gdn_prefill")
    return out


STATIC_SCRATCH_BYTES = 32 << 20


def prefill_noalloc(sh: Shape, qkv, beta_logits, alpha_logits, dt_bias, A, state_pool, slot_ids, status, out,
                    gate_z=None, gate_mode=0):
    """prefill with its workspace in the library's static device array (for callers that
    cannot allocate): nothing is allocated, here or in the library; `out` must be given.
    Shapes whose workspace exceeds STATIC_SCRATCH_BYTES raise (GDN_ERR_SCRATCH).  Calls that
    overlap on one GPU share that array and race.  Returns out."""
    C, T, P, Hv, dk, dv = sh.n_seqs, sh.n_nodes, sh.n_slots, sh.n_v_heads, sh.d_k, sh.d_v
    if status is None or out is None:
        raise ValueError("prefill_noalloc needs a status word and an output tensor")
    bp, bs = _gate_view(beta_logits, "beta_logits", sh)
    ap, as_ = _gate_view(alpha_logits, "alpha_logits", sh)
    if bs != as_:
        raise ValueError("beta_logits and alpha_logits must share one row stride")
    args = [
        _dev(qkv, "qkv", torch.float32, (C, T, sh.channels)), bp, ap, bs,
        _dev(dt_bias, "dt_bias", torch.float32, (Hv,)),
        _dev(A, "A", torch.float32, (Hv,)),
        _dev(state_pool, "state_pool", torch.float32, (P, Hv, dk, dv)),
        _dev(slot_ids, "slot_ids", torch.int32, (C,)),
        None if gate_z is None else _dev(gate_z, "gate_z", torch.float32, (C, T, Hv, dv)),
        ctypes.c_int32(int(gate_mode)),
        _dev(out, "out", torch.float32, (C, T, Hv, dv)),
        _dev(status, "status", torch.int32, (1,)),
        _stream(qkv),
    ]
    cs = sh.c_struct()
    _check(load_library().gdn_prefill_noalloc(ctypes.byref(cs), *args), "gdn_prefill_noalloc")
    return out
