/*
 * gdn_verify.h -- C ABI of the speculative-verify Gated DeltaNet route on MI355X (gfx950).
 *
 * One speculative round of one GDN layer is three calls on ONE caller stream:
 *
 *   gdn_conv_tree_step  tree-parent causal conv + SiLU over slot-mapped history,
 *                       plus one commit window per draft node;
 *   gdn_tree_verify     gated delta-rule recurrence over each lane's draft tree,
 *                       reading the slot's persistent state read-only and writing
 *                       the attention output and a replay log;
 *   gdn_replay_commit   after the host has chosen the accepted node of every lane,
 *                       advances the live recurrent state and conv history of the
 *                       accepting slots (an all-or-nothing transaction).
 *
 * Two further calls cover the same route with fewer launches:
 *   gdn_conv_tree_verify      the first two calls fused (conv output kept on chip);
 *   gdn_replay_commit_layers  the commit of every layer of a round in one launch.
 *
 * A step without a draft (plain decode) skips verify and commit and advances the slots
 * directly, also on one stream:
 *   gdn_conv_step    causal conv + SiLU over a chain of tokens per lane, writing each
 *                    slot's new conv history in place;
 *   gdn_decode_step  one token of the gated delta rule applied to each slot's state in
 *                    place, with the output row
 *                    (gdn_conv_decode_step: both for one token in one launch).
 *
 * A prompt fills a slot the same way, with gdn_conv_step over its tokens and then
 *   gdn_prefill      the gated delta rule over a chain of tokens per lane, the slot's state
 *                    updated in place, with an optional closing output gate
 *                    (gdn_prefill_noalloc: the same without a caller workspace).
 *
 * Sources (page title, then section):
 *   "perf(qwen35): fuse the DFlash2 concurrent verify Gated DeltaNet route",
 *       Summary and Optimizations (the three operations and their inputs/outputs),
 *       closing paragraph of Optimizations (tap/accumulation order; persistent state
 *       read-only during verification; replay-log commit after acceptance).
 *   "qwen35: DSpark speculative decoding (Qwen3.8-27B drafters)", commit messages
 *       (raw gates sigmoid(beta), softplus(alpha + dt_bias) * A; stacked
 *       ssm_beta|ssm_alpha projection; one l2_norm over q|k; q/k heads broadcast).
 *   "perf(qwen38): various DFlash2 optimizations concurrency C1-C5", Summary item 3
 *       (state size 128, replay width 257), Correctness and verification (padded and
 *       permuted slots, transaction preflight), review of the replay-log commit
 *       (commit must be ordered after the producer on the same stream).
 *   "llama-cpp-bonsai-gdn-conv.patch", ssm-conv.cu / ssm-conv.cuh / models.h /
 *       qwen35.cpp hunks (history layout [d_conv-1, channels] per sequence, token
 *       layout channels-contiguous, weight [channels][d_conv], state and output
 *       shapes, channel count).
 *
 * Conventions common to all calls
 *   - Every tensor is float32 or int32, C order (row-major), in device memory,
 *     allocated and owned by the caller.  The library allocates nothing, keeps no
 *     pointer or device state between calls, and is re-entrant; the one exception is
 *     gdn_prefill_noalloc, whose workspace is a static device array of the library.
 *   - Every call validates its arguments on the host, enqueues its kernels on
 *     `stream` and returns without synchronising.  Verify and commit of a round
 *     must be issued on the same stream (or the caller orders them).
 *   - Output buffers must not overlap any input or each other (checked on byte
 *     ranges, GDN_ERR_ALIAS); the pools updated in place (by the commit and the plain
 *     decode step) must not overlap their inputs or each other.
 *   - Dense float buffers (x, conv_w, conv_hist, conv_out, commit_win, qkv, state_pool,
 *     out) must be 16-byte aligned; every other buffer 4-byte aligned (GDN_ERR_ALIGN).
 *   - Host errors are returned synchronously and nothing is enqueued.
 *   - Lane errors found on the device are OR-ed into *status as GDN_STATUS_* bits
 *     (caller zeroes *status before the round).  Conv and verify write nothing for
 *     an offending lane; the commit and the plain decode step mutate nothing at all
 *     if *status is non-zero after their preflight, including bits left there by an
 *     earlier call of the round.
 *   - A lane whose slot id is -1 is a padding lane: nothing is read or written for it.
 *   - Ragged lanes: the tree calls and the commit take an optional lane_nodes [C] (int32,
 *     device; NULL = every lane has N nodes).  Lane c then has N_c = lane_nodes[c] nodes
 *     0..N_c-1 (its drafted length; "qwen35: DSpark speculative decoding", v_len commit
 *     message); nodes i >= N_c are absent: their inputs are not used, their outputs are
 *     not written and their parents are not checked, and the commit accepts only present
 *     nodes.  Parents precede children, so the present nodes compute exactly what a batch
 *     of N_c nodes would.  N_c outside [0, N] sets GDN_STATUS_NODES.
 *
 * Notation: C = n_seqs lanes, N = n_nodes draft nodes per lane, P = n_slots pool
 * slots, H_k q/k heads, H_v value heads (H_v % H_k == 0; value head h uses q/k head
 * h % H_k), Ch = 2*H_k*d_k + H_v*d_v conv channels ordered q | k | v with each head a
 * contiguous block, W = d_conv - 1 = 3, R = 1 + d_k + d_v replay-log row width.
 */
#ifndef GDN_VERIFY_H
#define GDN_VERIFY_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Host return codes. */
#define GDN_OK 0
#define GDN_ERR_NULL 1        /* a required pointer is NULL                                  */
#define GDN_ERR_SHAPE 2       /* non-positive dimension, H_v % H_k != 0, gate_stride < H_v   */
#define GDN_ERR_UNSUPPORTED 3 /* d_conv != 4, d_k/d_v not in {16,32,64,128}, N > 32, C > 1024,
                                 n_layers outside 1..GDN_MAX_LAYERS, Ch > 2^24, P*H_v > 2^24,
                                 one lane's commit windows above 1 GiB (N*Ch*12 bytes),
                                 N != 1 for gdn_decode_step, or N > GDN_MAX_CHAIN for the
                                 chain calls gdn_conv_step / gdn_prefill                     */
#define GDN_ERR_ALIAS 4       /* an output byte range overlaps an input or another output    */
#define GDN_ERR_HIP 5         /* a kernel launch failed                                      */
#define GDN_ERR_ALIGN 6       /* a dense float buffer is not 16-byte aligned, or an int32 /
                                 gate buffer not 4-byte aligned                              */
#define GDN_ERR_WORKSPACE 7   /* workspace_bytes below gdn_prefill_workspace_size()          */
#define GDN_ERR_SCRATCH 8     /* gdn_prefill_noalloc: the shape needs more workspace than
                                 GDN_STATIC_SCRATCH_BYTES                                    */

/* Device status bits (OR-ed into *status). */
#define GDN_STATUS_SLOT_RANGE 1 /* slot id outside [-1, P)                                   */
#define GDN_STATUS_SLOT_DUP 2   /* the same non-negative slot id used by two lanes           */
#define GDN_STATUS_PARENT 4     /* parents[c][i] outside [-1, i-1]                           */
#define GDN_STATUS_ACCEPT 8     /* accept_node[c] outside [-1, N_c) (commit only)            */
#define GDN_STATUS_NODES 16     /* lane_nodes[c] outside [0, N]                              */

/* Draft nodes per lane (N).  The largest verify batch the pages use is a tree of 17 to 32
   nodes: "qwen35: DSpark speculative decoding (Qwen3.8-27B drafters)", the commit message on
   the quantized-GEMM tile choice, names N = 17..32 batches for the DDTree budgets; chains there
   are 8 or 16 wide.  The fused verify keeps a (2N) x (d_k + N) block per workgroup in LDS, so
   N is bounded by that largest tree (GDN_ERR_UNSUPPORTED above it). */
#define GDN_MAX_NODES 32
#define GDN_MAX_CHAIN 65536 /* tokens per lane of gdn_conv_step and gdn_prefill */
#define GDN_MAX_SEQS 1024
#define GDN_MAX_LAYERS 64

typedef struct gdn_shape {
    int32_t n_seqs;    /* C, 1..GDN_MAX_SEQS                                     */
    int32_t n_nodes;   /* N, 1..GDN_MAX_NODES; parent[i] in [-1, i-1]            */
    int32_t n_slots;   /* P >= 1                                                 */
    int32_t n_k_heads; /* H_k >= 1                                               */
    int32_t n_v_heads; /* H_v, a multiple of H_k                                 */
    int32_t d_k;       /* 16, 32, 64 or 128                                      */
    int32_t d_v;       /* 16, 32, 64 or 128                                      */
    int32_t d_conv;    /* must be 4                                              */
} gdn_shape;

/*
 * Tree conv step ("perf(qwen35): fuse the DFlash2 concurrent verify Gated DeltaNet
 * route", Optimizations, first bullet; tap order from "llama-cpp-bonsai-gdn-conv.patch",
 * ssm-conv.cu hunk).
 *
 * For lane c (slot s = slot_ids[c]) and node i, let E(i) be the slot's history
 * columns conv_hist[s][:, 0..2] (oldest first) followed by the tokens x[c][a] of the
 * nodes a on i's root path (root child first, i last).  Then
 *   conv_out[c][i][ch]      = silu( sum_{j=0..3} conv_w[ch][j] * E(i)[-4 + j][ch] )
 *   commit_win[c][i][ch][j] = E(i)[-3 + j][ch],  j = 0..2   (bit-exact copies)
 * i.e. tap 0 multiplies the oldest column, no bias.  commit_win[c][i] is exactly the
 * history slot s must hold if node i becomes the last accepted token.
 *
 *   x          [C][N][Ch]     projected tokens                       (read)
 *   conv_w     [Ch][4]        depthwise taps                         (read)
 *   conv_hist  [P][Ch][3]     persistent history pool, READ-ONLY here
 *   slot_ids   [C]            int32, -1 = padding lane               (read)
 *   parents    [C][N]         int32 draft-tree parents               (read)
 *   lane_nodes [C]            int32 nodes per lane, or NULL (= N)    (read)
 *   conv_out   [C][N][Ch]     written for valid lanes' present nodes
 *   commit_win [C][N][Ch][3]  written for valid lanes' present nodes
 *   status     int32*         may be NULL; SLOT_RANGE / SLOT_DUP / PARENT / NODES bits
 */
int gdn_conv_tree_step(const gdn_shape *sh, const float *x, const float *conv_w, const float *conv_hist,
                       const int32_t *slot_ids, const int32_t *parents, const int32_t *lane_nodes, float *conv_out,
                       float *commit_win, int32_t *status, hipStream_t stream);

/*
 * Read-only slot-mapped tree verify ("perf(qwen35): fuse the DFlash2 concurrent
 * verify Gated DeltaNet route", Optimizations, second and third bullets; gates from
 * "qwen35: DSpark speculative decoding", raw-gate commit message).
 *
 * For lane c (slot s), value head h (q/k head kh = h % H_k) and nodes i in index
 * order, with q = qkv[c][i][kh*d_k ..], k = qkv[c][i][H_k*d_k + kh*d_k ..],
 * v = qkv[c][i][2*H_k*d_k + h*d_v ..], b = beta_logits[(c*N+i)*gate_stride + h],
 * a = alpha_logits[(c*N+i)*gate_stride + h]:
 *   q^ = q/|q|, k^ = k/|k|;  beta = sigmoid(b);  g = exp(softplus(a + dt_bias[h]) * A[h])
 *   S' = g * S_parent   (S_parent = state_pool[s][h] for a root child, else the state
 *                        after the parent node; states of [d_k][d_v], value index fastest)
 *   delta = beta * (v - S'^T k^);  S_i = S' + k^ delta^T;  out[c][i][h] = S_i^T q^ / sqrt(d_k)
 *   replay_log[c][i][h] = (g, k^[0..d_k), delta[0..d_v))            (R floats)
 * state_pool is bit-identical afterwards; no per-node state is written.
 *
 *   qkv            [C][N][Ch]          conv output of the round           (read)
 *   beta_logits    strided, see above  e.g. the stacked b|a projection [C][N][2*H_v]
 *   alpha_logits   strided, see above  with alpha_logits = beta_logits + H_v
 *   gate_stride    floats between consecutive tokens' gate rows, >= H_v
 *   dt_bias, A     [H_v]               (A negative, e.g. -exp(A_log))
 *   state_pool     [P][H_v][d_k][d_v]  persistent, READ-ONLY here
 *   slot_ids, parents, lane_nodes      as above
 *   out            [C][N][H_v][d_v]    written for valid lanes' present nodes
 *   replay_log     [C][N][H_v][R]      written for valid lanes' present nodes
 *   status         int32*              may be NULL
 */
int gdn_tree_verify(const gdn_shape *sh, const float *qkv, const float *beta_logits, const float *alpha_logits,
                    int64_t gate_stride, const float *dt_bias, const float *A, const float *state_pool,
                    const int32_t *slot_ids, const int32_t *parents, const int32_t *lane_nodes, float *out,
                    float *replay_log, int32_t *status, hipStream_t stream);

/*
 * Replay-log commit ("perf(qwen35): fuse the DFlash2 concurrent verify Gated DeltaNet
 * route", closing paragraph of Optimizations; "perf(qwen38): various DFlash2
 * optimizations concurrency C1-C5", Summary item 3 and the transaction preflight).
 *
 * Preflight over every non-padding lane: slot range, duplicate slots, node counts,
 * parents and accept_node[c] in [-1, N_c).  If *status is then non-zero nothing is written.
 * Otherwise every non-padding lane with e = accept_node[c] >= 0 replays the logged
 * transitions of e's root path, in path order, into its slot:
 *   S <- g_t * S + k^_t delta_t^T    for state_pool[s][h], every h,
 * and sets conv_hist[s] = commit_win[c][e] (bit-exact copy).  Lanes with e = -1 and
 * slots used by no accepting lane are bit-identical afterwards.
 *
 *   replay_log, commit_win   outputs of this round's verify / conv    (read)
 *   slot_ids, parents        the round's mapping and trees            (read)
 *   lane_nodes [C]           int32 nodes per lane, or NULL (= N)      (read)
 *   accept_node [C]          int32 deepest accepted node, -1 = none   (read)
 *   state_pool, conv_hist    updated in place
 *   status                   int32*, REQUIRED (GDN_ERR_NULL otherwise)
 */
int gdn_replay_commit(const gdn_shape *sh, const float *replay_log, const float *commit_win,
                      const int32_t *slot_ids, const int32_t *parents, const int32_t *lane_nodes,
                      const int32_t *accept_node, float *state_pool, float *conv_hist, int32_t *status,
                      hipStream_t stream);

/*
 * Fused tree conv + verify: gdn_conv_tree_step followed by gdn_tree_verify on its
 * output, in one launch, without materialising the conv output ("perf(qwen35): fuse
 * the DFlash2 concurrent verify Gated DeltaNet route", Optimizations: conv, SiLU,
 * window emission and the read-only recurrence in one route).  out, replay_log and
 * commit_win are the values the two separate calls produce (the conv output that feeds
 * the recurrence carries the recurrence tolerance; commit windows are exact copies).
 *
 *   x, conv_w, conv_hist          as in gdn_conv_tree_step (conv_hist READ-ONLY)
 *   beta_logits .. state_pool     as in gdn_tree_verify (state_pool READ-ONLY)
 *   slot_ids, parents, lane_nodes as above
 *   out, replay_log               as in gdn_tree_verify
 *   commit_win                    as in gdn_conv_tree_step
 *   status                        may be NULL
 * Alignment: x, conv_w, conv_hist, state_pool, out, commit_win 16 bytes; the rest 4.
 * Every output must be disjoint from every input and from the other outputs.
 */
int gdn_conv_tree_verify(const gdn_shape *sh, const float *x, const float *conv_w, const float *conv_hist,
                         const float *beta_logits, const float *alpha_logits, int64_t gate_stride,
                         const float *dt_bias, const float *A, const float *state_pool, const int32_t *slot_ids,
                         const int32_t *parents, const int32_t *lane_nodes, float *out, float *replay_log,
                         float *commit_win, int32_t *status, hipStream_t stream);

/*
 * Multi-layer replay-log commit: the commit above for every GDN layer of the round in
 * one launch.  Acceptance is per token, so all layers share slot_ids, parents and
 * accept_node; each layer l has its own replay log, commit windows, state pool and
 * history pool.  One preflight and one status word cover the round: either every
 * layer commits or none does.  (The pages' route issues one commit launch per layer,
 * "perf(qwen38): various DFlash2 optimizations concurrency C1-C5", launch accounting.)
 *
 *   n_layers                 1..GDN_MAX_LAYERS
 *   replay_logs, commit_wins host arrays of n_layers device pointers (layouts as above)
 *   state_pools, conv_hists  host arrays of n_layers device pointers, updated in place
 *   slot_ids, parents, lane_nodes, accept_node, status   as in gdn_replay_commit (status REQUIRED)
 * Every layer's pools must be disjoint from every input and from each other
 * (GDN_ERR_ALIAS).
 */
int gdn_replay_commit_layers(const gdn_shape *sh, int32_t n_layers, const float *const *replay_logs,
                             const float *const *commit_wins, const int32_t *slot_ids, const int32_t *parents,
                             const int32_t *lane_nodes, const int32_t *accept_node, float *const *state_pools,
                             float *const *conv_hists, int32_t *status, hipStream_t stream);

/*
 * Plain decode step, conv part ("qwen35: DSpark speculative decoding (Qwen3.8-27B
 * drafters)", DeltaNet-block commit message: one causal-conv step kernel with history
 * window, silu(conv) and in-place history write-back; tap order from
 * "llama-cpp-bonsai-gdn-conv.patch", ssm-conv.cu hunk).
 *
 * x[c] is a chain of N = n_nodes tokens for lane c (slot s), 1..GDN_MAX_CHAIN.  With E the slot's history
 * columns conv_hist[s][:, 0..2] (oldest first) followed by x[c][0..N-1]:
 *   conv_out[c][t][ch] = silu( sum_{j=0..3} conv_w[ch][j] * E[t + j][ch] )
 * and afterwards conv_hist[s][ch][j] = E[N + j][ch], j = 0..2 (the last 3 columns,
 * bit-exact copies).  A transaction: every non-padding lane's slot must lie in [0, P)
 * and be used by no other lane, and *status must be zero on entry; otherwise the
 * offending bits are OR-ed into *status and nothing is written at all.
 *
 *   x          [C][N][Ch]     tokens                                (read)
 *   conv_w     [Ch][4]        depthwise taps                        (read)
 *   conv_hist  [P][Ch][3]     persistent history pool, updated in place
 *   slot_ids   [C]            int32, -1 = padding lane              (read)
 *   conv_out   [C][N][Ch]     written for non-padding lanes
 *   status     int32*, REQUIRED (GDN_ERR_NULL otherwise)
 */
int gdn_conv_step(const gdn_shape *sh, const float *x, const float *conv_w, float *conv_hist,
                  const int32_t *slot_ids, float *conv_out, int32_t *status, hipStream_t stream);

/*
 * Plain decode step, recurrence part ("Feature/support dflash2", deferred-state commit
 * message: a step the drafter did not draft for commits its post-step state to the slot
 * immediately; "qwen35: DSpark speculative decoding", DeltaNet-block and raw-gate commit
 * messages: the gated delta rule in place with the gates applied in-kernel).
 *
 * One token per lane (n_nodes must be 1, GDN_ERR_UNSUPPORTED otherwise).  For lane c
 * (slot s) and value head h (q/k head kh = h % H_k), with q, k, v the head's slices of
 * qkv[c], b = beta_logits[c*gate_stride + h], a = alpha_logits[c*gate_stride + h]:
 *   q^ = q/|q|, k^ = k/|k|;  beta = sigmoid(b);  g = exp(softplus(a + dt_bias[h]) * A[h])
 *   S' = g * state_pool[s][h];  delta = beta * (v - S'^T k^)
 *   state_pool[s][h] = S' + k^ delta^T           (in place)
 *   out[c][h] = state_pool[s][h]^T q^ / sqrt(d_k)
 * A transaction with the same preflight as gdn_conv_step, so a step whose conv part
 * failed leaves the state untouched too.
 *
 *   qkv            [C][Ch]             conv output row of each lane's token  (read)
 *   beta_logits    element (c,h) at beta_logits[c*gate_stride + h]          (read)
 *   alpha_logits   element (c,h) at alpha_logits[c*gate_stride + h]         (read)
 *   gate_stride    >= H_v (2*H_v for the stacked b|a projection)
 *   dt_bias, A     [H_v]                                                    (read)
 *   state_pool     [P][H_v][d_k][d_v]  updated in place
 *   slot_ids       [C]                 int32, -1 = padding lane             (read)
 *   out            [C][H_v][d_v]       written for non-padding lanes
 *   status         int32*, REQUIRED (GDN_ERR_NULL otherwise)
 */
int gdn_decode_step(const gdn_shape *sh, const float *qkv, const float *beta_logits, const float *alpha_logits,
                    int64_t gate_stride, const float *dt_bias, const float *A, float *state_pool,
                    const int32_t *slot_ids, float *out, int32_t *status, hipStream_t stream);

/*
 * Plain decode step in one launch: gdn_conv_step over one token per lane followed by
 * gdn_decode_step on its output, with the same results bit for bit (the conv output stays
 * on chip and is not written).  Same sources as those two calls.  The pages fuse only the
 * verify route ("perf(qwen35): fuse the DFlash2 concurrent verify Gated DeltaNet route",
 * Summary: fewer launches and less temporary traffic); this call applies the same fusion
 * to the plain step, as gdn_conv_tree_verify does to the verify.
 *
 * n_nodes must be 1 (GDN_ERR_UNSUPPORTED otherwise).  A transaction with the preflight of
 * gdn_conv_step: on a bad slot or a non-zero *status nothing is written at all.
 *
 *   x              [C][Ch]             the token of each lane                 (read)
 *   conv_w         [Ch][4]             depthwise taps                         (read)
 *   conv_hist      [P][Ch][3]          history pool, updated in place
 *   beta_logits, alpha_logits, gate_stride, dt_bias, A   as in gdn_decode_step
 *   state_pool     [P][H_v][d_k][d_v]  updated in place
 *   slot_ids       [C]                 int32, -1 = padding lane               (read)
 *   sync           [C][H_k][GDN_SYNC_STRIDE]  int32 counters (element [c][kh][0] of each
 *                                      128-byte line), all zero on entry; every call leaves
 *                                      them zero.  Where a q/k head has more than 16
 *                                      (value head, 32-column block) pairs (H_v / H_k value
 *                                      heads of d_v / 32 blocks each), the in-place history of a
 *                                      q/k channel is read by several workgroups, and the last
 *                                      of them to count itself here writes it.  Required in
 *                                      every call; calls that overlap in time must not share
 *                                      one sync array.
 *   out            [C][H_v][d_v]       written for non-padding lanes
 *   status         int32*, REQUIRED (GDN_ERR_NULL otherwise)
 */
#define GDN_SYNC_STRIDE 32 /* int32 per counter of gdn_conv_decode_step: one 128-byte line */
int gdn_conv_decode_step(const gdn_shape *sh, const float *x, const float *conv_w, float *conv_hist,
                         const float *beta_logits, const float *alpha_logits, int64_t gate_stride,
                         const float *dt_bias, const float *A, float *state_pool, const int32_t *slot_ids,
                         int32_t *sync, float *out, int32_t *status, hipStream_t stream);

/*
 * Prefill ("Feature/support dflash2", first-version commit message: prefill's recurrence
 * runs on a chunked GDN kernel that closes with a SiLU or, by gate_mode, a sigmoid output
 * gate; gates as in gdn_tree_verify).
 *
 * n_nodes = T is the number of tokens per lane (1..GDN_MAX_CHAIN), a chain.  For lane c
 * (slot s) and value head h, the tokens t = 0..T-1 in order apply the rule of
 * gdn_decode_step to state_pool[s][h] (in place), and
 *   out[c][t][h] = o_t                      without a gate (gate_z NULL),
 *   out[c][t][h] = o_t * silu(z)            gate_mode 0,
 *   out[c][t][h] = o_t * sigmoid(z)         gate_mode 1,   z = gate_z[c][t][h]
 * (silu(z) = z * sigmoid(z)).  A transaction with the preflight of gdn_conv_step.
 *
 *   qkv            [C][T][Ch]          conv output rows of the tokens        (read)
 *   beta_logits    element (c,t,h) at beta_logits[(c*T+t)*gate_stride + h] (read)
 *   alpha_logits   element (c,t,h) at alpha_logits[(c*T+t)*gate_stride + h](read)
 *   gate_stride    >= H_v
 *   dt_bias, A     [H_v]                                                    (read)
 *   state_pool     [P][H_v][d_k][d_v]  updated in place
 *   slot_ids       [C]                 int32, -1 = padding lane             (read)
 *   gate_z         [C][T][H_v][d_v]    output gate values, or NULL          (read)
 *   gate_mode      0 (SiLU) or 1 (sigmoid); GDN_ERR_SHAPE otherwise
 *   out            [C][T][H_v][d_v]    written for non-padding lanes
 *   workspace      device scratch of at least gdn_prefill_workspace_size(sh) bytes,
 *                  16-byte aligned, overlapping nothing else; its contents on entry do
 *                  not matter and are undefined afterwards.  It holds the per-chunk
 *                  coefficients of the chunked form (C * H_v * ceil(T / 16) * 1488 bytes)
 *                  and must not be used by another call until this one has run.
 *   workspace_bytes its size (GDN_ERR_WORKSPACE if too small)
 *   status         int32*, REQUIRED (GDN_ERR_NULL otherwise)
 */
int gdn_prefill(const gdn_shape *sh, const float *qkv, const float *beta_logits, const float *alpha_logits,
                int64_t gate_stride, const float *dt_bias, const float *A, float *state_pool, const int32_t *slot_ids,
                const float *gate_z, int32_t gate_mode, float *out, float *workspace, size_t workspace_bytes,
                int32_t *status, hipStream_t stream);

/* Bytes of workspace gdn_prefill needs for this shape (n_nodes = T tokens per lane); 0 if
   the shape is invalid for gdn_prefill.  Host only, no device call. */
size_t gdn_prefill_workspace_size(const gdn_shape *sh);

/*
 * For callers that cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc): gdn_prefill with its workspace in a
 * static device array of the library instead of a caller buffer.  Arguments, results and
 * errors are those of gdn_prefill without workspace / workspace_bytes, plus
 * GDN_ERR_SCRATCH (nothing enqueued) when gdn_prefill_workspace_size(sh) exceeds
 * GDN_STATIC_SCRATCH_BYTES (32 MiB: e.g. 4 lanes x 1024 tokens x 32 value heads need 12.2 MB).
 * The call allocates and frees nothing.  Every GPU the library runs on holds one copy of the
 * array from the library's first use on it until the process ends; its address is looked
 * up once per device (GDN_ERR_HIP if that fails).  All calls on one GPU share that copy:
 * calls whose executions overlap on one GPU (different streams, or other host threads,
 * without ordering between them) race on it and give undefined results; calls ordered on
 * one stream are safe.  The array's contents on entry do not matter.
 */
#define GDN_STATIC_SCRATCH_BYTES (32u << 20)
int gdn_prefill_noalloc(const gdn_shape *sh, const float *qkv, const float *beta_logits, const float *alpha_logits,
                        int64_t gate_stride, const float *dt_bias, const float *A, float *state_pool,
                        const int32_t *slot_ids, const float *gate_z, int32_t gate_mode, float *out, int32_t *status,
                        hipStream_t stream);

/* Static description of a GDN_OK / GDN_ERR_* code. */
const char *gdn_strerror(int code);

#ifdef __cplusplus
}
#endif

#endif /* GDN_VERIFY_H */
