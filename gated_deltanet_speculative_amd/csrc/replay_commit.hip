// Replay-log commit for gfx950: after acceptance is known, advance each accepting slot's
// recurrent state by the logged transitions of its accepted root path and copy the
// accepted node's commit window into its conv history.  A preflight kernel validates
// every lane first; the commit kernel mutates nothing if the status word is non-zero,
// which makes the round an all-or-nothing transaction.
//
// What is computed: "perf(qwen35): fuse the DFlash2 concurrent verify Gated DeltaNet
// route", closing paragraph of Optimizations (the replay-log commit advances persistent
// state after acceptance); "perf(qwen38): various DFlash2 optimizations concurrency
// C1-C5", Summary item 3 (replay transitions, width 1 + d_k + d_v) and Correctness and
// verification (transaction preflight; padded and permuted slots).
//
// Design (HBM-bound: each accepted lane reads and writes its slot's state once).  One
// workgroup per (lane, value head, 32-row block of the state); the path's g, k^ rows of
// the block and delta rows are staged in LDS, then every thread streams float4 groups of
// the state through the m transitions S <- g S + k^ delta^T in path order and writes
// them back.  Extra workgroups per lane copy the commit window into the history pool.
#include "gdn_internal.h"

namespace gdn {
namespace {

constexpr int kThreads = 256;

__global__ __launch_bounds__(kThreads) void commit_preflight_kernel(Dims d, const int32_t *__restrict__ slot_ids,
                                                                    const int32_t *__restrict__ parents,
                                                                    const int32_t *__restrict__ accept_node,
                                                                    int32_t *__restrict__ status) {
    int bits = 0;
    for (int c = blockIdx.x * kThreads + threadIdx.x; c < d.C; c += gridDim.x * kThreads) {
        const int s = slot_ids[c];
        if (s == -1) continue;
        if (s < -1 || s >= d.P) bits |= GDN_STATUS_SLOT_RANGE;
        for (int o = 0; o < d.C; ++o)
            if (o != c && slot_ids[o] == s) bits |= GDN_STATUS_SLOT_DUP;
        for (int i = 0; i < d.N; ++i) {
            const int p = parents[(int64_t)c * d.N + i];
            if (p < -1 || p >= i) bits |= GDN_STATUS_PARENT;
        }
        const int e = accept_node[c];
        if (e < -1 || e >= d.N) bits |= GDN_STATUS_ACCEPT;
    }
    if (bits) atomicOr(status, bits);
}

template <int DK, int DV>
struct CommitCfg {
    static constexpr int RB = DK < 32 ? DK : 32;  // state rows per workgroup
    static constexpr int NB = DK / RB;
};

template <int DK, int DV>
__global__ __launch_bounds__(kThreads) void replay_commit_kernel(
    Dims d, const float *__restrict__ replay_log, const float *__restrict__ commit_win,
    const int32_t *__restrict__ slot_ids, const int32_t *__restrict__ parents, const int32_t *__restrict__ accept_node,
    float *__restrict__ state_pool, float *__restrict__ conv_hist, const int32_t *__restrict__ status) {
    constexpr int RB = CommitCfg<DK, DV>::RB;
    constexpr int R = 1 + DK + DV;
    __shared__ int s_path[GDN_MAX_NODES];
    __shared__ int s_m;
    __shared__ float s_g[GDN_MAX_NODES];
    __shared__ float s_k[GDN_MAX_NODES * RB];
    __shared__ float4 s_d4[GDN_MAX_NODES * DV / 4];

    if (*status != 0) return;  // preflight or an earlier call of the round flagged it
    const int c = blockIdx.z;
    const int s = slot_ids[c];
    const int e = accept_node[c];
    if (s < 0 || e < 0) return;  // padding lane, or nothing accepted
    const int N = d.N, Hv = d.Hv, tid = threadIdx.x;

    if (blockIdx.y == Hv) {  // conv history <- commit window of the accepted node
        const int n4 = d.Ch * 3 / 4;
        const float4 *src = reinterpret_cast<const float4 *>(commit_win + ((int64_t)c * N + e) * d.Ch * 3);
        float4 *dst = reinterpret_cast<float4 *>(conv_hist + (int64_t)s * d.Ch * 3);
        for (int idx = blockIdx.x * kThreads + tid; idx < n4; idx += gridDim.x * kThreads) dst[idx] = src[idx];
        return;
    }

    const int h = blockIdx.y;
    const int r0 = blockIdx.x * RB;
    if (tid == 0) {
        int m = 0;
        for (int a = e; a >= 0; a = parents[(int64_t)c * N + a]) ++m;
        s_m = m;
        int k = m;
        for (int a = e; a >= 0; a = parents[(int64_t)c * N + a]) s_path[--k] = a;
    }
    __syncthreads();
    const int m = s_m;
    const float *logc = replay_log + ((int64_t)c * N * Hv + h) * R;
    for (int idx = tid; idx < m * RB; idx += kThreads) {
        const int t = idx / RB, r = idx - t * RB;
        const float *lrow = logc + (int64_t)s_path[t] * Hv * R;
        s_k[idx] = lrow[1 + r0 + r];
        if (r == 0) s_g[t] = lrow[0];
    }
    float *s_d = reinterpret_cast<float *>(s_d4);
    for (int idx = tid; idx < m * DV; idx += kThreads) {
        const int t = idx / DV, j = idx - t * DV;
        s_d[idx] = logc[(int64_t)s_path[t] * Hv * R + 1 + DK + j];
    }
    __syncthreads();

    float4 *S4 = reinterpret_cast<float4 *>(state_pool + (((int64_t)s * Hv + h) * DK + r0) * DV);
    for (int idx = tid; idx < RB * DV / 4; idx += kThreads) {
        const int r = idx / (DV / 4), q = idx - r * (DV / 4);
        float4 v = S4[idx];
        for (int t = 0; t < m; ++t) {
            const float g = s_g[t], kr = s_k[t * RB + r];
            const float4 dl = s_d4[t * (DV / 4) + q];
            v.x = fmaf(kr, dl.x, g * v.x);
            v.y = fmaf(kr, dl.y, g * v.y);
            v.z = fmaf(kr, dl.z, g * v.z);
            v.w = fmaf(kr, dl.w, g * v.w);
        }
        S4[idx] = v;
    }
}

template <int DK, int DV>
hipError_t launch(const Dims &d, const float *log, const float *win, const int32_t *slots, const int32_t *parents,
                  const int32_t *accept, float *pool, float *hist, int32_t *status, hipStream_t stream) {
    const int pre_blocks = (d.C + kThreads - 1) / kThreads;
    hipLaunchKernelGGL(commit_preflight_kernel, dim3(pre_blocks), dim3(kThreads), 0, stream, d, slots, parents, accept,
                       status);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((replay_commit_kernel<DK, DV>), dim3(CommitCfg<DK, DV>::NB, d.Hv + 1, d.C), dim3(kThreads), 0,
                       stream, d, log, win, slots, parents, accept, pool, hist, status);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_replay_commit(const Dims &d, const float *replay_log, const float *commit_win,
                                const int32_t *slot_ids, const int32_t *parents, const int32_t *accept_node,
                                float *state_pool, float *conv_hist, int32_t *status, hipStream_t stream) {
#define GDN_COMMIT_CASE(K, V)                                                                                      \
    if (d.dk == K && d.dv == V)                                                                                    \
        return launch<K, V>(d, replay_log, commit_win, slot_ids, parents, accept_node, state_pool, conv_hist, status, \
                            stream);
#define GDN_COMMIT_ROW(K) GDN_COMMIT_CASE(K, 16) GDN_COMMIT_CASE(K, 32) GDN_COMMIT_CASE(K, 64) GDN_COMMIT_CASE(K, 128)
    GDN_COMMIT_ROW(16) GDN_COMMIT_ROW(32) GDN_COMMIT_ROW(64) GDN_COMMIT_ROW(128)
#undef GDN_COMMIT_ROW
#undef GDN_COMMIT_CASE
    return hipErrorInvalidValue;
}

}  // namespace gdn
