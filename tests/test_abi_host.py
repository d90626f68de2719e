"""The C-ABI library without a GPU: it loads, exports every function the header
declares, and its host-side validation returns the documented error codes
before anything is enqueued (fake, never-dereferenced pointer values)."""

import ctypes
import os
import re

import pytest

import gated_deltanet_speculative_amd as gdn
from gated_deltanet_speculative_amd import _lib

HEADER = os.path.join(os.path.dirname(os.path.dirname(__file__)), "include", "gdn_verify.h")

pytestmark = pytest.mark.skipif(not os.path.exists(_lib.LIB_PATH), reason="library not built")


def _declared():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^(?:int|size_t|const char \*)\s*(gdn_\w+)\s*\(", text, flags=re.M)))


def test_exports_every_declared_function():
    names = _declared()
    assert names == sorted(_lib.EXPORTED)
    lib = gdn.load_library()
    for n in names:
        assert hasattr(lib, n), n


def test_strerror_codes():
    assert gdn.strerror(0) == "success"
    assert "overlaps" in gdn.strerror(4)
    assert "unknown" in gdn.strerror(99)


FAKE = 0x7F0000000000  # never dereferenced: every call below fails validation first


def _shape(**kw):
    base = dict(n_seqs=2, n_nodes=4, n_slots=4, n_k_heads=2, n_v_heads=4, d_k=16, d_v=16, d_conv=4)
    base.update(kw)
    return gdn.Shape(**base)


def _ptrs(n, stride=1 << 28):
    return [FAKE + k * stride for k in range(n)]


# The helpers below take the pointers of each call without its optional lane_nodes
# argument and pass lane_nodes (default NULL: every lane has N nodes) in its place.
def _conv(sh, ptrs, status=None, lane_nodes=None):
    """ptrs: x, conv_w, conv_hist, slot_ids, parents, conv_out, commit_win"""
    lib = gdn.load_library()
    cs = sh.c_struct() if sh is not None else None
    p = list(ptrs)
    return lib.gdn_conv_tree_step(ctypes.byref(cs) if cs else None, *p[:5], lane_nodes, *p[5:], status, None)


def _verify(sh, ptrs, gate_stride, status=None, lane_nodes=None):
    """ptrs: qkv, beta, alpha, dt_bias, A, state_pool, slot_ids, parents, out, replay_log"""
    lib = gdn.load_library()
    cs = sh.c_struct()
    p = list(ptrs)
    return lib.gdn_tree_verify(ctypes.byref(cs), p[0], p[1], p[2], gate_stride, *p[3:8], lane_nodes, *p[8:], status,
                               None)


def _commit(sh, ptrs, status, lane_nodes=None):
    """ptrs: replay_log, commit_win, slot_ids, parents, accept_node, state_pool, conv_hist"""
    lib = gdn.load_library()
    cs = sh.c_struct()
    p = list(ptrs)
    return lib.gdn_replay_commit(ctypes.byref(cs), *p[:4], lane_nodes, *p[4:], status, None)


def test_null_shape_and_pointers():
    assert _conv(None, _ptrs(7)) == _lib.GDN_ERR_NULL
    p = _ptrs(7)
    p[2] = None
    assert _conv(_shape(), p) == _lib.GDN_ERR_NULL
    p = _ptrs(10)
    p[0] = None
    assert _verify(_shape(), p, 8) == _lib.GDN_ERR_NULL
    assert _commit(_shape(), _ptrs(7), None) == _lib.GDN_ERR_NULL  # commit needs its status word


@pytest.mark.parametrize("kw,code", [
    (dict(n_seqs=0), _lib.GDN_ERR_SHAPE),
    (dict(n_nodes=-1), _lib.GDN_ERR_SHAPE),
    (dict(n_v_heads=3), _lib.GDN_ERR_SHAPE),
    (dict(d_conv=3), _lib.GDN_ERR_UNSUPPORTED),
    (dict(d_k=48), _lib.GDN_ERR_UNSUPPORTED),
    (dict(d_v=256), _lib.GDN_ERR_UNSUPPORTED),
    (dict(n_nodes=33), _lib.GDN_ERR_UNSUPPORTED),
    (dict(n_seqs=1025), _lib.GDN_ERR_UNSUPPORTED),
    (dict(n_k_heads=65536, n_v_heads=65536, d_k=128, d_v=16), _lib.GDN_ERR_UNSUPPORTED),  # Ch > 2^24
    (dict(n_nodes=32, n_k_heads=8192, n_v_heads=8192, d_k=128, d_v=128), _lib.GDN_ERR_UNSUPPORTED),  # windows > 1 GiB
])
def test_shape_rejections(kw, code):
    assert _conv(_shape(**kw), _ptrs(7)) == code
    assert _verify(_shape(**kw), _ptrs(10), 8) == code
    assert _commit(_shape(**kw), _ptrs(7), FAKE + (9 << 28)) == code


def test_gate_stride_below_heads_rejected():
    assert _verify(_shape(), _ptrs(10), 3) == _lib.GDN_ERR_SHAPE


def test_misaligned_rejected():
    p = _ptrs(7)
    p[0] += 4  # x not 16-byte aligned
    assert _conv(_shape(), p) == _lib.GDN_ERR_ALIGN
    p = _ptrs(10)
    p[1] += 2  # gate rows not 4-byte aligned
    assert _verify(_shape(), p, 8) == _lib.GDN_ERR_ALIGN
    p = _ptrs(10)
    p[1] += 4  # a 4-byte offset is fine for the gates (e.g. the alpha half of b|a) ...
    p[5] += 8  # ... but not for the state pool
    assert _verify(_shape(), p, 8) == _lib.GDN_ERR_ALIGN


def test_alias_rejected():
    sh = _shape()
    p = _ptrs(7)
    p[5] = p[0] + 64  # conv_out inside x
    assert _conv(sh, p) == _lib.GDN_ERR_ALIAS
    p = _ptrs(7)
    p[6] = p[5] + 16  # commit_win overlaps conv_out
    assert _conv(sh, p) == _lib.GDN_ERR_ALIAS
    p = _ptrs(7)
    assert _conv(sh, p, status=p[3]) == _lib.GDN_ERR_ALIAS  # status inside slot_ids
    p = _ptrs(10)
    p[8] = p[5] + 16  # out overlaps the state pool
    assert _verify(sh, p, 8) == _lib.GDN_ERR_ALIAS
    p = _ptrs(10)
    p[9] = p[1] + 4 * 8 * 7  # replay log inside the strided gate rows
    assert _verify(sh, p, 8) == _lib.GDN_ERR_ALIAS
    p = _ptrs(7)
    p[6] = p[5]  # conv_hist == state_pool
    assert _commit(sh, p, FAKE + (9 << 28)) == _lib.GDN_ERR_ALIAS
    p = _ptrs(7)
    p[5] = p[0]  # state pool over the replay log
    assert _commit(sh, p, FAKE + (9 << 28)) == _lib.GDN_ERR_ALIAS


def _commit_layers(sh, L, per_layer, shared, status, n_layers=None):
    """per_layer: 4 lists (logs, wins, pools, hists) of L fake pointers; shared: 3 pointers."""
    lib = gdn.load_library()
    cs = sh.c_struct()
    arrs = [(ctypes.c_void_p * L)(*v) for v in per_layer]
    cast = [ctypes.cast(a, ctypes.c_void_p) for a in arrs]
    return lib.gdn_replay_commit_layers(ctypes.byref(cs), ctypes.c_int32(L if n_layers is None else n_layers),
                                        cast[0], cast[1], shared[0], shared[1], None, shared[2], cast[2], cast[3],
                                        status, None)


def _layer_ptrs(L):
    base = _ptrs(4 * L + 3)
    return [base[0:L], base[L:2 * L], base[2 * L:3 * L], base[3 * L:4 * L]], base[4 * L:]


def test_commit_layers_rejections():
    sh, st = _shape(), FAKE + (1 << 40)
    per, shared = _layer_ptrs(3)
    assert _commit_layers(sh, 3, per, shared, None) == _lib.GDN_ERR_NULL
    assert _commit_layers(sh, 3, per, shared, st, n_layers=0) == _lib.GDN_ERR_UNSUPPORTED
    assert _commit_layers(sh, 3, per, shared, st, n_layers=65) == _lib.GDN_ERR_UNSUPPORTED
    per, shared = _layer_ptrs(3)
    per[1][2] = None  # one layer's commit windows missing
    assert _commit_layers(sh, 3, per, shared, st) == _lib.GDN_ERR_NULL
    per, shared = _layer_ptrs(3)
    per[2][1] += 8  # one layer's state pool misaligned
    assert _commit_layers(sh, 3, per, shared, st) == _lib.GDN_ERR_ALIGN
    per, shared = _layer_ptrs(3)
    per[3][2] = per[2][0] + 16  # layer 2's history inside layer 0's state pool
    assert _commit_layers(sh, 3, per, shared, st) == _lib.GDN_ERR_ALIAS
    per, shared = _layer_ptrs(3)
    per[2][1] = per[0][2] + 16  # layer 1's state pool inside layer 2's replay log
    assert _commit_layers(sh, 3, per, shared, st) == _lib.GDN_ERR_ALIAS
    per, shared = _layer_ptrs(3)
    assert _commit_layers(sh, 3, per, shared, per[3][1]) == _lib.GDN_ERR_ALIAS  # status in a history pool
    per, shared = _layer_ptrs(3)
    assert _commit_layers(_shape(d_conv=5), 3, per, shared, st) == _lib.GDN_ERR_UNSUPPORTED


def _fused(sh, ptrs, gate_stride, status=None):
    """ptrs: x, conv_w, conv_hist, beta, alpha, dt_bias, A, state_pool, slot_ids, parents, out, replay_log, commit_win"""
    lib = gdn.load_library()
    cs = sh.c_struct()
    p = list(ptrs)
    return lib.gdn_conv_tree_verify(ctypes.byref(cs), *p[:5], gate_stride, *p[5:10], None, *p[10:], status, None)


def test_fused_rejections():
    sh = _shape()
    p = _ptrs(13)
    p[12] = None  # commit windows missing
    assert _fused(sh, p, 8) == _lib.GDN_ERR_NULL
    assert _fused(sh, _ptrs(13), 3) == _lib.GDN_ERR_SHAPE  # gate stride below H_v
    assert _fused(_shape(d_conv=3), _ptrs(13), 8) == _lib.GDN_ERR_UNSUPPORTED
    assert _fused(_shape(n_nodes=33), _ptrs(13), 8) == _lib.GDN_ERR_UNSUPPORTED
    p = _ptrs(13)
    p[2] += 4  # conv history not 16-byte aligned
    assert _fused(sh, p, 8) == _lib.GDN_ERR_ALIGN
    p = _ptrs(13)
    p[12] += 8  # commit windows not 16-byte aligned
    assert _fused(sh, p, 8) == _lib.GDN_ERR_ALIGN
    p = _ptrs(13)
    p[12] = p[0] + 64  # commit windows inside x
    assert _fused(sh, p, 8) == _lib.GDN_ERR_ALIAS
    p = _ptrs(13)
    p[10] = p[12] + 16  # out inside the commit windows
    assert _fused(sh, p, 8) == _lib.GDN_ERR_ALIAS
    p = _ptrs(13)
    p[11] = p[7] + 16  # replay log inside the state pool
    assert _fused(sh, p, 8) == _lib.GDN_ERR_ALIAS
    p = _ptrs(13)
    assert _fused(sh, p, 8, status=p[2] + 4) == _lib.GDN_ERR_ALIAS  # status inside the history pool


def _conv_step(sh, ptrs, status):
    """ptrs: x, conv_w, conv_hist, slot_ids, conv_out"""
    lib = gdn.load_library()
    cs = sh.c_struct()
    return lib.gdn_conv_step(ctypes.byref(cs), *ptrs, status, None)


def _decode_step(sh, ptrs, gate_stride, status):
    """ptrs: qkv, beta, alpha, dt_bias, A, state_pool, slot_ids, out"""
    lib = gdn.load_library()
    cs = sh.c_struct()
    p = list(ptrs)
    return lib.gdn_decode_step(ctypes.byref(cs), p[0], p[1], p[2], gate_stride, *p[3:], status, None)


def test_plain_step_rejections():
    st = FAKE + (1 << 40)
    one = _shape(n_nodes=1)
    assert _conv_step(_shape(), _ptrs(5), None) == _lib.GDN_ERR_NULL  # status is required
    assert _decode_step(one, _ptrs(8), 8, None) == _lib.GDN_ERR_NULL
    assert _decode_step(_shape(n_nodes=2), _ptrs(8), 8, st) == _lib.GDN_ERR_UNSUPPORTED  # one token only
    assert _decode_step(one, _ptrs(8), 3, st) == _lib.GDN_ERR_SHAPE  # gate stride below H_v
    assert _conv_step(_shape(d_conv=5), _ptrs(5), st) == _lib.GDN_ERR_UNSUPPORTED
    p = _ptrs(5)
    p[2] += 8  # history pool not 16-byte aligned
    assert _conv_step(_shape(), p, st) == _lib.GDN_ERR_ALIGN
    p = _ptrs(8)
    p[5] += 4  # state pool not 16-byte aligned
    assert _decode_step(one, p, 8, st) == _lib.GDN_ERR_ALIGN
    p = _ptrs(5)
    p[2] = p[0] + 64  # history pool (written in place) inside x
    assert _conv_step(_shape(), p, st) == _lib.GDN_ERR_ALIAS
    p = _ptrs(8)
    p[5] = p[0] + 16  # state pool (written in place) over qkv
    assert _decode_step(one, p, 8, st) == _lib.GDN_ERR_ALIAS
    p = _ptrs(8)
    assert _decode_step(one, p, 8, p[7] + 4) == _lib.GDN_ERR_ALIAS  # status inside out


def test_lane_nodes_checked_like_any_input():
    sh = _shape()
    nodes = FAKE + (1 << 41)
    assert _conv(sh, _ptrs(7), lane_nodes=nodes + 2) == _lib.GDN_ERR_ALIGN  # int32 counts need 4-byte alignment
    p = _ptrs(7)
    assert _conv(sh, p, lane_nodes=p[5] + 4) == _lib.GDN_ERR_ALIAS  # counts inside conv_out
    p = _ptrs(10)
    assert _verify(sh, p, 8, lane_nodes=p[9] + 8) == _lib.GDN_ERR_ALIAS  # counts inside the replay log
    p = _ptrs(7)
    assert _commit(sh, p, FAKE + (9 << 28), lane_nodes=p[5] + 16) == _lib.GDN_ERR_ALIAS  # counts inside the pool


def test_prefill_rejections():
    lib = gdn.load_library()
    st = FAKE + (1 << 40)

    def call(sh, p, gate_stride=8, gate_mode=0, status=st, ws_bytes=None):
        cs = sh.c_struct()
        if ws_bytes is None:
            ws_bytes = lib.gdn_prefill_workspace_size(ctypes.byref(cs))
        return lib.gdn_prefill(ctypes.byref(cs), p[0], p[1], p[2], gate_stride, p[3], p[4], p[5], p[6], p[7],
                               ctypes.c_int32(gate_mode), p[8], p[9], ctypes.c_size_t(ws_bytes), status, None)

    p = _ptrs(10)  # qkv, beta, alpha, dt_bias, A, state_pool, slot_ids, gate_z, out, workspace
    assert call(_shape(n_nodes=1000), p, status=None) == _lib.GDN_ERR_NULL
    q = list(p)
    q[9] = None  # no workspace
    assert call(_shape(n_nodes=1000), q) == _lib.GDN_ERR_NULL
    need = gdn.prefill_workspace_size(_shape(n_nodes=1000))
    assert call(_shape(n_nodes=1000), p, ws_bytes=need - 1) == _lib.GDN_ERR_WORKSPACE
    q = list(p)
    q[9] = q[8] + 64  # workspace inside the output
    assert call(_shape(n_nodes=1000), q) == _lib.GDN_ERR_ALIAS
    q = list(p)
    q[9] += 4  # workspace not 16-byte aligned
    assert call(_shape(n_nodes=1000), q) == _lib.GDN_ERR_ALIGN
    assert call(_shape(n_nodes=65537), p) == _lib.GDN_ERR_UNSUPPORTED  # longer than GDN_MAX_CHAIN
    assert call(_shape(n_nodes=1000), p, gate_mode=2) == _lib.GDN_ERR_SHAPE
    assert call(_shape(n_nodes=1000), p, gate_stride=3) == _lib.GDN_ERR_SHAPE
    q = list(p)
    q[7] += 4  # gate values not 16-byte aligned
    assert call(_shape(n_nodes=1000), q) == _lib.GDN_ERR_ALIGN
    q = list(p)
    q[5] = q[0] + 64  # state pool (written in place) inside qkv
    assert call(_shape(n_nodes=1000), q) == _lib.GDN_ERR_ALIAS
    q = list(p)
    q[8] = q[7] + 16  # out overlapping the gate values
    assert call(_shape(n_nodes=1000), q) == _lib.GDN_ERR_ALIAS


def test_prefill_workspace_size():
    """One package of 372 floats per (lane, value head, chunk of 16 tokens); 0 for shapes the
    prefill rejects."""
    sh = _shape(n_nodes=37)
    assert gdn.prefill_workspace_size(sh) == sh.n_seqs * sh.n_v_heads * 3 * 372 * 4
    assert gdn.prefill_workspace_size(_shape(n_nodes=16)) == _shape().n_seqs * _shape().n_v_heads * 372 * 4
    assert gdn.prefill_workspace_size(_shape(n_nodes=65537)) == 0
    assert gdn.prefill_workspace_size(_shape(d_k=24)) == 0


def test_conv_step_chain_limit():
    """The chain conv step takes up to GDN_MAX_CHAIN tokens (it feeds the prefill); longer
    chains are rejected before anything is enqueued."""
    assert gdn.MAX_CHAIN == 65536
    assert _conv_step(_shape(n_nodes=65537), _ptrs(5), FAKE + (1 << 40)) == _lib.GDN_ERR_UNSUPPORTED


def test_prefill_noalloc_rejections():
    """The prefill variant with the library's static workspace: the prefill's own checks,
    and GDN_ERR_SCRATCH, before any device call, when the shape's workspace exceeds the
    static array."""
    lib = gdn.load_library()
    st = FAKE + (1 << 40)

    def call(sh, p, gate_stride=8, gate_mode=0, status=st):
        cs = sh.c_struct()
        return lib.gdn_prefill_noalloc(ctypes.byref(cs), p[0], p[1], p[2], gate_stride, p[3], p[4], p[5], p[6], p[7],
                                       ctypes.c_int32(gate_mode), p[8], status, None)

    p = _ptrs(9)  # qkv, beta, alpha, dt_bias, A, state_pool, slot_ids, gate_z, out
    assert call(_shape(n_nodes=1000), p, status=None) == _lib.GDN_ERR_NULL
    assert call(_shape(n_nodes=1000), p, gate_mode=2) == _lib.GDN_ERR_SHAPE
    q = list(p)
    q[8] += 4
    assert call(_shape(n_nodes=1000), q) == _lib.GDN_ERR_ALIGN
    q = list(p)
    q[8] = q[7] + 16  # out overlapping the gate values
    assert call(_shape(n_nodes=1000), q) == _lib.GDN_ERR_ALIAS
    assert call(_shape(n_nodes=65537), p) == _lib.GDN_ERR_UNSUPPORTED
    big = gdn.Shape(4, 4096, 8, 16, 32, 128, 128)  # 4 x 32 x 256 packages of 1488 bytes: 49 MB
    assert gdn.prefill_workspace_size(big) > gdn.STATIC_SCRATCH_BYTES
    assert call(big, p, gate_stride=64) == _lib.GDN_ERR_SCRATCH
    assert "static scratch" in gdn.strerror(_lib.GDN_ERR_SCRATCH)
    fits = gdn.Shape(4, 1024, 8, 16, 32, 128, 128)  # the prefill bench shape: 12.2 MB
    assert gdn.prefill_workspace_size(fits) <= gdn.STATIC_SCRATCH_BYTES
