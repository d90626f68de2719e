// Internal declarations shared by the host entry points and the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gdn_verify.h"

namespace gdn {

struct Dims {
    int C, N, P, Hk, Hv, dk, dv, Ch;
};

// Nodes present in lane c: lane_nodes[c] (the lane's drafted length) or all N when the
// caller passes no counts.  A count outside [0, N] is reported as GDN_STATUS_NODES.
__device__ inline int lane_node_count(const int32_t *__restrict__ lane_nodes, const Dims &d, int c) {
    return lane_nodes ? lane_nodes[c] : d.N;
}

hipError_t launch_conv_tree_step(const Dims &d, const float *x, const float *conv_w, const float *conv_hist,
                                 const int32_t *slot_ids, const int32_t *parents, const int32_t *lane_nodes,
                                 float *conv_out, float *commit_win, int32_t *status, hipStream_t stream);

// Arguments of the tree verify kernels, passed by value.  The separate route reads the
// conv output `qkv`; the fused route reads x, conv_w and conv_hist, computes the conv
// in-kernel and writes commit_win (the unused pointers are null).
struct VerifyArgs {
    Dims d;
    const float *qkv;
    const float *x, *conv_w, *conv_hist;
    float *commit_win;
    const float *beta_logits, *alpha_logits;
    int64_t gate_stride;
    const float *dt_bias, *A;
    const float *state_pool;
    const int32_t *slot_ids, *parents;
    const int32_t *lane_nodes;  // may be null: every lane has N nodes
    float *out, *replay_log;
    int32_t *status;
};

hipError_t launch_tree_verify(const VerifyArgs &a, hipStream_t stream);

// Per-layer buffers of a multi-layer commit, passed by value as a kernel argument.
struct LayerPtrs {
    const float *replay_log[GDN_MAX_LAYERS];
    const float *commit_win[GDN_MAX_LAYERS];
    float *state_pool[GDN_MAX_LAYERS];
    float *conv_hist[GDN_MAX_LAYERS];
};

hipError_t launch_replay_commit(const Dims &d, int n_layers, const LayerPtrs &lp, const int32_t *slot_ids,
                                const int32_t *parents, const int32_t *lane_nodes, const int32_t *accept_node,
                                int32_t *status, hipStream_t stream);

// Plain decode step: chain conv with in-place history write-back, then one token of the
// recurrence applied to the slot's state in place.
hipError_t launch_conv_step(const Dims &d, const float *x, const float *conv_w, float *conv_hist,
                            const int32_t *slot_ids, float *conv_out, int32_t *status, hipStream_t stream);
hipError_t launch_decode_step(const Dims &d, const float *qkv, const float *beta_logits, const float *alpha_logits,
                              int64_t gate_stride, const float *dt_bias, const float *A, float *state_pool,
                              const int32_t *slot_ids, float *out, int32_t *status, hipStream_t stream);
// Both in one launch; sync holds C * H_k zero counters GDN_SYNC_STRIDE apart, left zero.
hipError_t launch_conv_decode_step(const Dims &d, const float *x, const float *conv_w, float *conv_hist,
                                   const float *beta_logits, const float *alpha_logits, int64_t gate_stride,
                                   const float *dt_bias, const float *A, float *state_pool, const int32_t *slot_ids,
                                   int32_t *sync, float *out, int32_t *status, hipStream_t stream);

// Prefill: the recurrence over a chain of d.N tokens per lane, state updated in place,
// optional output gate (gate_z may be null).  Two launches: the chunk coefficients of
// every (lane, value head, chunk of kPrefillChunk tokens) into `workspace`
// (kPackFloats floats each), then the state recurrence over the chunks.
constexpr int kPrefillChunk = 16;
constexpr int kPackFloats = 372;
inline size_t prefill_workspace_floats(const Dims &d) {
    return (size_t)d.C * d.Hv * (size_t)((d.N + kPrefillChunk - 1) / kPrefillChunk) * kPackFloats;
}
// The static workspace of the prefill variant that allocates nothing: the device address of
// this GPU's copy (the stream's device, else the current one), looked up once per device.
constexpr size_t kStaticScratchFloats = GDN_STATIC_SCRATCH_BYTES / sizeof(float);
hipError_t static_scratch(hipStream_t stream, float **ptr);
hipError_t launch_prefill(const Dims &d, int n_tokens, const float *qkv, const float *beta_logits,
                          const float *alpha_logits, int64_t gate_stride, const float *dt_bias, const float *A,
                          float *state_pool, const int32_t *slot_ids, const float *gate_z, int gate_mode, float *out,
                          float *workspace, int32_t *status, hipStream_t stream);

}  // namespace gdn
