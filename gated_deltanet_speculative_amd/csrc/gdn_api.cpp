// Host entry points of the C ABI: argument validation, byte-range alias checks and
// kernel dispatch on the caller's stream.  Every check runs before anything is
// enqueued; no entry point allocates, synchronises or keeps state between calls.
#include <cstdint>
#include <initializer_list>

#include "gdn_internal.h"

namespace {

struct Range {
    const void *p;
    size_t bytes;
};

bool overlap(const Range &a, const Range &b) {
    if (!a.p || !b.p || !a.bytes || !b.bytes) return false;
    const char *a0 = static_cast<const char *>(a.p), *b0 = static_cast<const char *>(b.p);
    return a0 < b0 + b.bytes && b0 < a0 + a.bytes;
}

// every output range against every input and every other output
bool any_alias(std::initializer_list<Range> outs, std::initializer_list<Range> ins) {
    for (auto o = outs.begin(); o != outs.end(); ++o) {
        for (const Range &i : ins)
            if (overlap(*o, i)) return true;
        for (auto o2 = o + 1; o2 != outs.end(); ++o2)
            if (overlap(*o, *o2)) return true;
    }
    return false;
}

bool aligned(std::initializer_list<const void *> ps, uintptr_t a) {
    for (const void *p : ps)
        if (reinterpret_cast<uintptr_t>(p) % a) return false;
    return true;
}

bool pow2_width(int v) { return v == 16 || v == 32 || v == 64 || v == 128; }

// chain = false: a draft tree (n_nodes <= GDN_MAX_NODES, commit windows of one lane below
// 1 GiB); chain = true: a chain of up to GDN_MAX_CHAIN tokens (conv step, prefill)
int check_shape(const gdn_shape *sh, gdn::Dims *d, bool chain = false) {
    if (!sh) return GDN_ERR_NULL;
    if (sh->n_seqs <= 0 || sh->n_nodes <= 0 || sh->n_slots <= 0 || sh->n_k_heads <= 0 || sh->n_v_heads <= 0 ||
        sh->d_k <= 0 || sh->d_v <= 0 || sh->d_conv <= 0)
        return GDN_ERR_SHAPE;
    if (sh->n_v_heads % sh->n_k_heads != 0) return GDN_ERR_SHAPE;
    if (sh->d_conv != 4 || !pow2_width(sh->d_k) || !pow2_width(sh->d_v) ||
        sh->n_nodes > (chain ? GDN_MAX_CHAIN : GDN_MAX_NODES) || sh->n_seqs > GDN_MAX_SEQS)
        return GDN_ERR_UNSUPPORTED;
    const int64_t ch = 2ll * sh->n_k_heads * sh->d_k + (int64_t)sh->n_v_heads * sh->d_v;
    if (ch > (1 << 24) || (int64_t)sh->n_slots * sh->n_v_heads > (1 << 24) ||
        (!chain && (int64_t)sh->n_nodes * ch * 12 > (1 << 30)))
        return GDN_ERR_UNSUPPORTED;
    *d = gdn::Dims{sh->n_seqs, sh->n_nodes, sh->n_slots, sh->n_k_heads, sh->n_v_heads, sh->d_k, sh->d_v, (int)ch};
    return GDN_OK;
}

constexpr size_t F = sizeof(float), I = sizeof(int32_t);

}  // namespace

extern "C" {

int gdn_conv_tree_step(const gdn_shape *sh, const float *x, const float *conv_w, const float *conv_hist,
                       const int32_t *slot_ids, const int32_t *parents, const int32_t *lane_nodes, float *conv_out,
                       float *commit_win, int32_t *status, hipStream_t stream) {
    gdn::Dims d;
    if (int r = check_shape(sh, &d)) return r;
    if (!x || !conv_w || !conv_hist || !slot_ids || !parents || !conv_out || !commit_win) return GDN_ERR_NULL;
    if (!aligned({x, conv_w, conv_hist, conv_out, commit_win}, 16) || !aligned({slot_ids, parents, lane_nodes, status}, 4))
        return GDN_ERR_ALIGN;
    const size_t cnc = (size_t)d.C * d.N * d.Ch;
    if (any_alias({{conv_out, cnc * F}, {commit_win, cnc * 3 * F}, {status, I}},
                  {{x, cnc * F}, {conv_w, (size_t)d.Ch * 4 * F}, {conv_hist, (size_t)d.P * d.Ch * 3 * F},
                   {slot_ids, (size_t)d.C * I}, {parents, (size_t)d.C * d.N * I}, {lane_nodes, (size_t)d.C * I}}))
        return GDN_ERR_ALIAS;
    return gdn::launch_conv_tree_step(d, x, conv_w, conv_hist, slot_ids, parents, lane_nodes, conv_out, commit_win,
                                      status, stream) == hipSuccess
               ? GDN_OK
               : GDN_ERR_HIP;
}

int gdn_tree_verify(const gdn_shape *sh, const float *qkv, const float *beta_logits, const float *alpha_logits,
                    int64_t gate_stride, const float *dt_bias, const float *A, const float *state_pool,
                    const int32_t *slot_ids, const int32_t *parents, const int32_t *lane_nodes, float *out,
                    float *replay_log, int32_t *status, hipStream_t stream) {
    gdn::Dims d;
    if (int r = check_shape(sh, &d)) return r;
    if (!qkv || !beta_logits || !alpha_logits || !dt_bias || !A || !state_pool || !slot_ids || !parents || !out ||
        !replay_log)
        return GDN_ERR_NULL;
    if (gate_stride < d.Hv) return GDN_ERR_SHAPE;
    if (!aligned({qkv, state_pool, out}, 16) ||
        !aligned({beta_logits, alpha_logits, dt_bias, A, slot_ids, parents, lane_nodes, replay_log, status}, 4))
        return GDN_ERR_ALIGN;
    const size_t rows = (size_t)d.C * d.N;
    const size_t gate_bytes = ((rows - 1) * (size_t)gate_stride + d.Hv) * F;
    const size_t R = 1 + (size_t)d.dk + d.dv;
    if (any_alias({{out, rows * d.Hv * d.dv * F}, {replay_log, rows * d.Hv * R * F}, {status, I}},
                  {{qkv, rows * d.Ch * F}, {beta_logits, gate_bytes}, {alpha_logits, gate_bytes},
                   {dt_bias, (size_t)d.Hv * F}, {A, (size_t)d.Hv * F},
                   {state_pool, (size_t)d.P * d.Hv * d.dk * d.dv * F}, {slot_ids, (size_t)d.C * I},
                   {parents, rows * I}, {lane_nodes, (size_t)d.C * I}}))
        return GDN_ERR_ALIAS;
    gdn::VerifyArgs a{};
    a.d = d;
    a.qkv = qkv;
    a.beta_logits = beta_logits;
    a.alpha_logits = alpha_logits;
    a.gate_stride = gate_stride;
    a.dt_bias = dt_bias;
    a.A = A;
    a.state_pool = state_pool;
    a.slot_ids = slot_ids;
    a.parents = parents;
    a.lane_nodes = lane_nodes;
    a.out = out;
    a.replay_log = replay_log;
    a.status = status;
    return gdn::launch_tree_verify(a, stream) == hipSuccess ? GDN_OK : GDN_ERR_HIP;
}

int gdn_conv_tree_verify(const gdn_shape *sh, const float *x, const float *conv_w, const float *conv_hist,
                         const float *beta_logits, const float *alpha_logits, int64_t gate_stride,
                         const float *dt_bias, const float *A, const float *state_pool, const int32_t *slot_ids,
                         const int32_t *parents, const int32_t *lane_nodes, float *out, float *replay_log,
                         float *commit_win, int32_t *status, hipStream_t stream) {
    gdn::Dims d;
    if (int r = check_shape(sh, &d)) return r;
    if (!x || !conv_w || !conv_hist || !beta_logits || !alpha_logits || !dt_bias || !A || !state_pool ||
        !slot_ids || !parents || !out || !replay_log || !commit_win)
        return GDN_ERR_NULL;
    if (gate_stride < d.Hv) return GDN_ERR_SHAPE;
    if (!aligned({x, conv_w, conv_hist, state_pool, out, commit_win}, 16) ||
        !aligned({beta_logits, alpha_logits, dt_bias, A, slot_ids, parents, lane_nodes, replay_log, status}, 4))
        return GDN_ERR_ALIGN;
    const size_t rows = (size_t)d.C * d.N;
    const size_t gate_bytes = ((rows - 1) * (size_t)gate_stride + d.Hv) * F;
    const size_t R = 1 + (size_t)d.dk + d.dv;
    if (any_alias({{out, rows * d.Hv * d.dv * F}, {replay_log, rows * d.Hv * R * F},
                   {commit_win, rows * d.Ch * 3 * F}, {status, I}},
                  {{x, rows * d.Ch * F}, {conv_w, (size_t)d.Ch * 4 * F}, {conv_hist, (size_t)d.P * d.Ch * 3 * F},
                   {beta_logits, gate_bytes}, {alpha_logits, gate_bytes}, {dt_bias, (size_t)d.Hv * F},
                   {A, (size_t)d.Hv * F}, {state_pool, (size_t)d.P * d.Hv * d.dk * d.dv * F},
                   {slot_ids, (size_t)d.C * I}, {parents, rows * I}, {lane_nodes, (size_t)d.C * I}}))
        return GDN_ERR_ALIAS;
    gdn::VerifyArgs a{};
    a.d = d;
    a.x = x;
    a.conv_w = conv_w;
    a.conv_hist = conv_hist;
    a.commit_win = commit_win;
    a.beta_logits = beta_logits;
    a.alpha_logits = alpha_logits;
    a.gate_stride = gate_stride;
    a.dt_bias = dt_bias;
    a.A = A;
    a.state_pool = state_pool;
    a.slot_ids = slot_ids;
    a.parents = parents;
    a.lane_nodes = lane_nodes;
    a.out = out;
    a.replay_log = replay_log;
    a.status = status;
    return gdn::launch_tree_verify(a, stream) == hipSuccess ? GDN_OK : GDN_ERR_HIP;
}

int gdn_replay_commit_layers(const gdn_shape *sh, int32_t n_layers, const float *const *replay_logs,
                             const float *const *commit_wins, const int32_t *slot_ids, const int32_t *parents,
                             const int32_t *lane_nodes, const int32_t *accept_node, float *const *state_pools,
                             float *const *conv_hists, int32_t *status, hipStream_t stream) {
    gdn::Dims d;
    if (int r = check_shape(sh, &d)) return r;
    if (n_layers < 1 || n_layers > GDN_MAX_LAYERS) return GDN_ERR_UNSUPPORTED;
    if (!replay_logs || !commit_wins || !state_pools || !conv_hists || !slot_ids || !parents || !accept_node ||
        !status)
        return GDN_ERR_NULL;
    const size_t rows = (size_t)d.C * d.N;
    const size_t R = 1 + (size_t)d.dk + d.dv;
    const size_t pool_b = (size_t)d.P * d.Hv * d.dk * d.dv * F, hist_b = (size_t)d.P * d.Ch * 3 * F;
    const size_t log_b = rows * d.Hv * R * F, win_b = rows * d.Ch * 3 * F;
    gdn::LayerPtrs lp{};
    for (int l = 0; l < n_layers; ++l) {
        if (!replay_logs[l] || !commit_wins[l] || !state_pools[l] || !conv_hists[l]) return GDN_ERR_NULL;
        if (!aligned({commit_wins[l], state_pools[l], conv_hists[l]}, 16) || !aligned({replay_logs[l]}, 4))
            return GDN_ERR_ALIGN;
        lp.replay_log[l] = replay_logs[l];
        lp.commit_win[l] = commit_wins[l];
        lp.state_pool[l] = state_pools[l];
        lp.conv_hist[l] = conv_hists[l];
    }
    if (!aligned({slot_ids, parents, lane_nodes, accept_node, status}, 4)) return GDN_ERR_ALIGN;
    // every layer's pools against every input, the status word and every other layer's pools
    for (int l = 0; l < n_layers; ++l) {
        const Range outs[2] = {{state_pools[l], pool_b}, {conv_hists[l], hist_b}};
        for (const Range &o : outs) {
            if (any_alias({o, {status, I}}, {{slot_ids, (size_t)d.C * I}, {parents, rows * I},
                                              {lane_nodes, (size_t)d.C * I}, {accept_node, (size_t)d.C * I}}))
                return GDN_ERR_ALIAS;
            for (int m = 0; m < n_layers; ++m) {
                if (overlap(o, {replay_logs[m], log_b}) || overlap(o, {commit_wins[m], win_b})) return GDN_ERR_ALIAS;
                if (m == l) {
                    if (overlap(outs[0], outs[1])) return GDN_ERR_ALIAS;
                    continue;
                }
                if (overlap(o, {state_pools[m], pool_b}) || overlap(o, {conv_hists[m], hist_b})) return GDN_ERR_ALIAS;
            }
        }
    }
    return gdn::launch_replay_commit(d, n_layers, lp, slot_ids, parents, lane_nodes, accept_node, status, stream) ==
                   hipSuccess
               ? GDN_OK
               : GDN_ERR_HIP;
}

int gdn_replay_commit(const gdn_shape *sh, const float *replay_log, const float *commit_win,
                      const int32_t *slot_ids, const int32_t *parents, const int32_t *lane_nodes,
                      const int32_t *accept_node, float *state_pool, float *conv_hist, int32_t *status,
                      hipStream_t stream) {
    if (!replay_log || !commit_win || !state_pool || !conv_hist) {
        gdn::Dims d;
        if (int r = check_shape(sh, &d)) return r;
        return GDN_ERR_NULL;
    }
    return gdn_replay_commit_layers(sh, 1, &replay_log, &commit_win, slot_ids, parents, lane_nodes, accept_node,
                                    &state_pool, &conv_hist, status, stream);
}

int gdn_conv_step(const gdn_shape *sh, const float *x, const float *conv_w, float *conv_hist,
                  const int32_t *slot_ids, float *conv_out, int32_t *status, hipStream_t stream) {
    gdn::Dims d;
    if (int r = check_shape(sh, &d, true)) return r;
    if (!x || !conv_w || !conv_hist || !slot_ids || !conv_out || !status) return GDN_ERR_NULL;
    if (!aligned({x, conv_w, conv_hist, conv_out}, 16) || !aligned({slot_ids, status}, 4)) return GDN_ERR_ALIGN;
    const size_t cnc = (size_t)d.C * d.N * d.Ch;
    if (any_alias({{conv_hist, (size_t)d.P * d.Ch * 3 * F}, {conv_out, cnc * F}, {status, I}},
                  {{x, cnc * F}, {conv_w, (size_t)d.Ch * 4 * F}, {slot_ids, (size_t)d.C * I}}))
        return GDN_ERR_ALIAS;
    return gdn::launch_conv_step(d, x, conv_w, conv_hist, slot_ids, conv_out, status, stream) == hipSuccess
               ? GDN_OK
               : GDN_ERR_HIP;
}

int gdn_decode_step(const gdn_shape *sh, const float *qkv, const float *beta_logits, const float *alpha_logits,
                    int64_t gate_stride, const float *dt_bias, const float *A, float *state_pool,
                    const int32_t *slot_ids, float *out, int32_t *status, hipStream_t stream) {
    gdn::Dims d;
    if (int r = check_shape(sh, &d)) return r;
    if (d.N != 1) return GDN_ERR_UNSUPPORTED;
    if (!qkv || !beta_logits || !alpha_logits || !dt_bias || !A || !state_pool || !slot_ids || !out || !status)
        return GDN_ERR_NULL;
    if (gate_stride < d.Hv) return GDN_ERR_SHAPE;
    if (!aligned({qkv, state_pool, out}, 16) || !aligned({beta_logits, alpha_logits, dt_bias, A, slot_ids, status}, 4))
        return GDN_ERR_ALIGN;
    const size_t gate_bytes = ((size_t)(d.C - 1) * (size_t)gate_stride + d.Hv) * F;
    if (any_alias({{state_pool, (size_t)d.P * d.Hv * d.dk * d.dv * F}, {out, (size_t)d.C * d.Hv * d.dv * F},
                   {status, I}},
                  {{qkv, (size_t)d.C * d.Ch * F}, {beta_logits, gate_bytes}, {alpha_logits, gate_bytes},
                   {dt_bias, (size_t)d.Hv * F}, {A, (size_t)d.Hv * F}, {slot_ids, (size_t)d.C * I}}))
        return GDN_ERR_ALIAS;
    return gdn::launch_decode_step(d, qkv, beta_logits, alpha_logits, gate_stride, dt_bias, A, state_pool, slot_ids,
                                   out, status, stream) == hipSuccess
               ? GDN_OK
               : GDN_ERR_HIP;
}

int gdn_conv_decode_step(const gdn_shape *sh, const float *x, const float *conv_w, float *conv_hist,
                         const float *beta_logits, const float *alpha_logits, int64_t gate_stride,
                         const float *dt_bias, const float *A, float *state_pool, const int32_t *slot_ids,
                         int32_t *sync, float *out, int32_t *status, hipStream_t stream) {
    gdn::Dims d;
    if (int r = check_shape(sh, &d)) return r;
    if (d.N != 1) return GDN_ERR_UNSUPPORTED;
    if (!x || !conv_w || !conv_hist || !beta_logits || !alpha_logits || !dt_bias || !A || !state_pool || !slot_ids ||
        !sync || !out || !status)
        return GDN_ERR_NULL;
    if (gate_stride < d.Hv) return GDN_ERR_SHAPE;
    if (!aligned({x, conv_w, conv_hist, state_pool, out}, 16) ||
        !aligned({beta_logits, alpha_logits, dt_bias, A, slot_ids, sync, status}, 4))
        return GDN_ERR_ALIGN;
    const size_t gate_bytes = ((size_t)(d.C - 1) * (size_t)gate_stride + d.Hv) * F;
    if (any_alias({{conv_hist, (size_t)d.P * d.Ch * 3 * F}, {state_pool, (size_t)d.P * d.Hv * d.dk * d.dv * F},
                   {out, (size_t)d.C * d.Hv * d.dv * F}, {sync, (size_t)d.C * d.Hk * GDN_SYNC_STRIDE * I}, {status, I}},
                  {{x, (size_t)d.C * d.Ch * F}, {conv_w, (size_t)d.Ch * 4 * F}, {beta_logits, gate_bytes},
                   {alpha_logits, gate_bytes}, {dt_bias, (size_t)d.Hv * F}, {A, (size_t)d.Hv * F},
                   {slot_ids, (size_t)d.C * I}}))
        return GDN_ERR_ALIAS;
    return gdn::launch_conv_decode_step(d, x, conv_w, conv_hist, beta_logits, alpha_logits, gate_stride, dt_bias, A,
                                        state_pool, slot_ids, sync, out, status, stream) == hipSuccess
               ? GDN_OK
               : GDN_ERR_HIP;
}

size_t gdn_prefill_workspace_size(const gdn_shape *sh) {
    gdn::Dims d;
    if (check_shape(sh, &d, true)) return 0;
    return gdn::prefill_workspace_floats(d) * F;
}

// Argument checks shared by gdn_prefill and gdn_prefill_noalloc (whose workspace is the
// library's own array: no caller buffer can overlap it).
static int prefill_args(const gdn_shape *sh, gdn::Dims *dp, const float *qkv, const float *beta_logits,
                        const float *alpha_logits, int64_t gate_stride, const float *dt_bias, const float *A,
                        float *state_pool, const int32_t *slot_ids, const float *gate_z, int32_t gate_mode,
                        float *out, const float *workspace, size_t ws_b, int32_t *status) {
    gdn::Dims &d = *dp;
    if (int r = check_shape(sh, &d, true)) return r;
    if (!qkv || !beta_logits || !alpha_logits || !dt_bias || !A || !state_pool || !slot_ids || !out || !status)
        return GDN_ERR_NULL;
    if (gate_stride < d.Hv || (gate_mode != 0 && gate_mode != 1)) return GDN_ERR_SHAPE;
    if (!aligned({qkv, state_pool, out, gate_z, workspace}, 16) ||
        !aligned({beta_logits, alpha_logits, dt_bias, A, slot_ids, status}, 4))
        return GDN_ERR_ALIGN;
    const size_t rows = (size_t)d.C * d.N;
    const size_t gate_bytes = ((rows - 1) * (size_t)gate_stride + d.Hv) * F;
    const size_t out_b = rows * d.Hv * d.dv * F;
    if (any_alias({{state_pool, (size_t)d.P * d.Hv * d.dk * d.dv * F}, {out, out_b}, {workspace, ws_b}, {status, I}},
                  {{qkv, rows * d.Ch * F}, {beta_logits, gate_bytes}, {alpha_logits, gate_bytes},
                   {dt_bias, (size_t)d.Hv * F}, {A, (size_t)d.Hv * F}, {slot_ids, (size_t)d.C * I},
                   {gate_z, out_b}}))
        return GDN_ERR_ALIAS;
    return GDN_OK;
}

int gdn_prefill(const gdn_shape *sh, const float *qkv, const float *beta_logits, const float *alpha_logits,
                int64_t gate_stride, const float *dt_bias, const float *A, float *state_pool, const int32_t *slot_ids,
                const float *gate_z, int32_t gate_mode, float *out, float *workspace, size_t workspace_bytes,
                int32_t *status, hipStream_t stream) {
    gdn::Dims d;
    if (int r = check_shape(sh, &d, true)) return r;
    if (!qkv || !beta_logits || !alpha_logits || !dt_bias || !A || !state_pool || !slot_ids || !out || !workspace ||
        !status)
        return GDN_ERR_NULL;
    if (gate_stride < d.Hv || (gate_mode != 0 && gate_mode != 1)) return GDN_ERR_SHAPE;
    const size_t ws_b = gdn::prefill_workspace_floats(d) * F;
    if (workspace_bytes < ws_b) return GDN_ERR_WORKSPACE;
    if (int r = prefill_args(sh, &d, qkv, beta_logits, alpha_logits, gate_stride, dt_bias, A, state_pool, slot_ids,
                             gate_z, gate_mode, out, workspace, ws_b, status))
        return r;
    return gdn::launch_prefill(d, d.N, qkv, beta_logits, alpha_logits, gate_stride, dt_bias, A, state_pool, slot_ids,
                               gate_z, gate_mode, out, workspace, status, stream) == hipSuccess
               ? GDN_OK
               : GDN_ERR_HIP;
}

int gdn_prefill_noalloc(const gdn_shape *sh, const float *qkv, const float *beta_logits, const float *alpha_logits,
                        int64_t gate_stride, const float *dt_bias, const float *A, float *state_pool,
                        const int32_t *slot_ids, const float *gate_z, int32_t gate_mode, float *out, int32_t *status,
                        hipStream_t stream) {
    gdn::Dims d;
    if (int r = prefill_args(sh, &d, qkv, beta_logits, alpha_logits, gate_stride, dt_bias, A, state_pool, slot_ids,
                             gate_z, gate_mode, out, nullptr, 0, status))
        return r;
    if (gdn::prefill_workspace_floats(d) > gdn::kStaticScratchFloats) return GDN_ERR_SCRATCH;
    float *ws = nullptr;
    if (gdn::static_scratch(stream, &ws) != hipSuccess) return GDN_ERR_HIP;
    return gdn::launch_prefill(d, d.N, qkv, beta_logits, alpha_logits, gate_stride, dt_bias, A, state_pool, slot_ids,
                               gate_z, gate_mode, out, ws, status, stream) == hipSuccess
               ? GDN_OK
               : GDN_ERR_HIP;
}

const char *gdn_strerror(int code) {
    switch (code) {
        case GDN_OK: return "success";
        case GDN_ERR_NULL: return "a required pointer is NULL";
        case GDN_ERR_SHAPE: return "invalid shape (non-positive dimension, H_v not a multiple of H_k, or gate_stride < H_v)";
        case GDN_ERR_UNSUPPORTED: return "unsupported shape (d_conv != 4, head width not in {16,32,64,128}, more than 32 nodes or 1024 lanes)";
        case GDN_ERR_ALIAS: return "an output buffer overlaps an input or another output";
        case GDN_ERR_HIP: return "HIP kernel launch failed";
        case GDN_ERR_ALIGN: return "a buffer is misaligned (dense float buffers need 16 bytes, others 4)";
        case GDN_ERR_WORKSPACE: return "the workspace is smaller than the size query returns for this shape";
        case GDN_ERR_SCRATCH: return "the shape needs more workspace than the static scratch of gdn_prefill_noalloc (32 MiB)";
        default: return "unknown error code";
    }
}

}  // extern "C"
