// Replay-log commit for gfx950: after acceptance is known, advance each accepting slot's
// recurrent state by the logged transitions of its accepted root path and copy the
// accepted node's commit window into its conv history, as an all-or-nothing transaction.
//
// What is computed: "perf(qwen35): fuse the DFlash2 concurrent verify Gated DeltaNet
// route", closing paragraph of Optimizations (the replay-log commit advances persistent
// state after acceptance); "perf(qwen38): various DFlash2 optimizations concurrency
// C1-C5", Summary item 3 (replay transitions, width 1 + d_k + d_v) and Correctness and
// verification (transaction preflight; padded and permuted slots).
//
// Design (HBM-bound: each accepting lane reads and writes its slot's state once).  One
// launch: every workgroup runs the preflight over all lanes itself (slot range,
// duplicate slots, parents, accept node) and also honours bits already in *status, so
// all workgroups take the same commit-or-abort decision without a second kernel.  A
// workgroup owns (lane, value head, 32-row block of the state); it requests its state
// block before validating, then walks the accepted path in LDS, stages the path's g, k^
// rows and delta rows, streams the block through S <- g S + k^ delta^T in path order and
// writes it back.  One extra workgroup row per lane copies the commit window into the
// history pool.
#include "gdn_internal.h"

namespace gdn {
namespace {

constexpr int kThreads = 256;
constexpr int kBitmapSlots = 65536;  // duplicate-slot check via an LDS bitmap up to this pool size

typedef float v4f __attribute__((ext_vector_type(4)));

template <int DK, int DV>
struct CommitCfg {
    static constexpr int RB = DK < 32 ? DK : 32;  // state rows per workgroup
    static constexpr int NB = DK / RB;
    static constexpr int F4 = RB * DV / 4;        // 4-float groups per block
    static constexpr int FPT = (F4 + kThreads - 1) / kThreads;
};

// Preflight over every lane, evaluated by each workgroup; returns the status bits.
// Contains barriers: every thread of the workgroup must call it.
__device__ int preflight(const Dims &d, const int32_t *__restrict__ slot_ids, const int32_t *__restrict__ parents,
                         const int32_t *__restrict__ accept_node, unsigned int *bitmap, int *s_bits) {
    const int tid = threadIdx.x;
    const bool use_bitmap = d.P <= kBitmapSlots;
    if (use_bitmap)
        for (int w = tid; w < (d.P + 31) / 32; w += kThreads) bitmap[w] = 0u;
    if (tid == 0) *s_bits = 0;
    __syncthreads();
    int bits = 0;
    for (int t = tid; t < d.C; t += kThreads) {
        const int s = slot_ids[t];
        if (s == -1) continue;
        const int e = accept_node[t];
        if (e < -1 || e >= d.N) bits |= GDN_STATUS_ACCEPT;
        if (s < -1 || s >= d.P) {
            bits |= GDN_STATUS_SLOT_RANGE;
        } else if (use_bitmap) {
            if (atomicOr(&bitmap[s >> 5], 1u << (s & 31)) & (1u << (s & 31))) bits |= GDN_STATUS_SLOT_DUP;
        } else {
            for (int o = 0; o < d.C; ++o)
                if (o != t && slot_ids[o] == s) bits |= GDN_STATUS_SLOT_DUP;
        }
    }
    for (int idx = tid; idx < d.C * d.N; idx += kThreads) {
        const int t = idx / d.N, i = idx - t * d.N;
        const int p = parents[idx];
        if (slot_ids[t] != -1 && (p < -1 || p >= i)) bits |= GDN_STATUS_PARENT;
    }
    if (bits) atomicOr(s_bits, bits);
    __syncthreads();
    return *s_bits;
}

template <int DK, int DV>
__global__ __launch_bounds__(kThreads) void replay_commit_kernel(
    Dims d, const float *__restrict__ replay_log, const float *__restrict__ commit_win,
    const int32_t *__restrict__ slot_ids, const int32_t *__restrict__ parents, const int32_t *__restrict__ accept_node,
    float *__restrict__ state_pool, float *__restrict__ conv_hist, int32_t *__restrict__ status) {
    using Cfg = CommitCfg<DK, DV>;
    constexpr int RB = Cfg::RB, F4 = Cfg::F4, FPT = Cfg::FPT, R = 1 + DK + DV;
    __shared__ unsigned int s_bitmap[kBitmapSlots / 32];
    __shared__ int s_bits, s_m;
    __shared__ int s_par[GDN_MAX_NODES], s_path[GDN_MAX_NODES];
    __shared__ float s_g[GDN_MAX_NODES];
    __shared__ float s_k[GDN_MAX_NODES * RB];
    __shared__ v4f s_d4[GDN_MAX_NODES * DV / 4];

    const int c = blockIdx.z, tid = threadIdx.x;
    const int N = d.N, Hv = d.Hv;
    const bool hist_copy = blockIdx.y == Hv;
    const int h = hist_copy ? 0 : blockIdx.y;
    const int r0 = blockIdx.x * RB;

    // ---- requests that do not depend on validation: this lane's slot, accept node and
    //      parents, the round's status word, and the state block (slot clamped into range)
    const int s = slot_ids[c], e = accept_node[c];
    const int st_in = *status;
    const int par = parents[(int64_t)c * N + (tid < N ? tid : 0)];
    const bool s_ok = s >= 0 && s < d.P;
    v4f *S4 = reinterpret_cast<v4f *>(state_pool + (((int64_t)(s_ok ? s : 0) * Hv + h) * DK + r0) * DV);
    v4f sv[FPT];
#pragma unroll
    for (int u = 0; u < FPT; ++u) sv[u] = S4[min(tid + kThreads * u, F4 - 1)];

    const int bits = preflight(d, slot_ids, parents, accept_node, s_bitmap, &s_bits);
    if (bits) {
        if (blockIdx.x == 0 && blockIdx.y == 0 && tid == 0) atomicOr(status, bits);
        return;
    }
    if (st_in != 0 || s < 0 || e < 0) return;  // flagged round, padding lane, or nothing accepted

    if (hist_copy) {  // conv history <- commit window of the accepted node
        const int n4 = d.Ch * 3 / 4;
        const v4f *src = reinterpret_cast<const v4f *>(commit_win + ((int64_t)c * N + e) * d.Ch * 3);
        v4f *dst = reinterpret_cast<v4f *>(conv_hist + (int64_t)s * d.Ch * 3);
        for (int idx = blockIdx.x * kThreads + tid; idx < n4; idx += gridDim.x * kThreads) dst[idx] = src[idx];
        return;
    }

    // ---- accepted path (root child first), walked in LDS
    if (tid < N) s_par[tid] = par;
    __syncthreads();
    if (tid == 0) {
        int m = 0;
        for (int a = e; a >= 0; a = s_par[a]) ++m;
        s_m = m;
        for (int a = e, k = m; a >= 0; a = s_par[a]) s_path[--k] = a;
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

    // ---- S <- g S + k^ delta^T along the path, then write the block back
    // (indices clamped as at load time: surplus threads recompute the last group from
    // the same loaded value and store the identical result)
#pragma unroll
    for (int u = 0; u < FPT; ++u) {
        const int idx = min(tid + kThreads * u, F4 - 1);
        const int r = idx / (DV / 4), q = idx - r * (DV / 4);
        v4f v = sv[u];
        for (int t = 0; t < m; ++t) {
            const float g = s_g[t], kr = s_k[t * RB + r];
            const v4f dl = s_d4[t * (DV / 4) + q];
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
