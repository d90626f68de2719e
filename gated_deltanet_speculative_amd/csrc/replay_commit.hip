// Replay-log commit for gfx950: after acceptance is known, advance each accepting slot's
// recurrent state by the logged transitions of its accepted root path and copy the
// accepted node's commit window into its conv history, as an all-or-nothing transaction,
// for one layer or for every layer of the round in a single launch.
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
// workgroup owns (lane, value head, 64-row block of the state).  It issues every load
// that does not need the slot id first, then its state block; every wave finds the
// accepted path by pointer jumping over lane shuffles, and each thread loads the logged
// g, k^ and delta values of its own state elements for every path node straight into
// registers while the block streams in, accumulating the replay of the path from a zero
// state (the transitions are linear: S_final = G S0 + A).  After the preflight (barriers
// wait for LDS traffic only) it writes G S0 + A back.
// One extra workgroup row per lane copies the commit window into the history pool.
#include "gdn_device.h"
#include "gdn_internal.h"

namespace gdn {
namespace {

constexpr int kThreads = 256;

template <int DK, int DV>
struct CommitCfg {
    static constexpr int RB = DK < 64 ? DK : 64;  // state rows per workgroup
    static constexpr int NB = DK / RB;
    static constexpr int F4 = RB * DV / 4;        // 4-float groups per block
    static constexpr int FPT = (F4 + kThreads - 1) / kThreads;  // state rows per thread
};

constexpr int kPreRows = 4;  // lanes' parent entries checked per thread in the first pass

// Root path of node e as a bit mask, from the parents held by lanes 0..N-1 of the wave
// (lane i holds parents[i]): pointer jumping, log2(N) rounds of lane shuffles, so the
// cost does not grow with the depth of the path.  Out-of-range parents end the walk
// (the preflight rejects them anyway).
__device__ inline unsigned int path_mask(int par, int lane, int N, int e) {
    int jump = (lane < N && par >= 0 && par < lane) ? par : -1;
    unsigned int anc = lane < N ? 1u << lane : 0u;
#pragma unroll
    for (int r = 1; r < GDN_MAX_NODES; r <<= 1) {
        const int src = jump < 0 ? lane : jump;
        const unsigned int aj = __shfl(anc, src);
        const int jj = __shfl(jump, src);
        if (jump >= 0) {
            anc |= aj;
            jump = jj;
        }
    }
    return (e >= 0 && e < N) ? __shfl(anc, e) : 0u;
}

// Raw buffer resources: word 3 of the descriptor for the gfx9 family (32-bit data,
// unswizzled); a load past num_records reads zero and a store there is dropped.
constexpr int kRsrcWord3 = 0x00020000;
constexpr int kNonTemporal = 2;  // cache-policy operand of the buffer stores: nt
typedef int v4i __attribute__((ext_vector_type(4)));

template <int DK, int DV>
__global__ __launch_bounds__(kThreads) void replay_commit_kernel(
    Dims d, const LayerPtrs lp, const int32_t *__restrict__ slot_ids, const int32_t *__restrict__ parents,
    const int32_t *__restrict__ lane_nodes, const int32_t *__restrict__ accept_node, int32_t *__restrict__ status) {
    using Cfg = CommitCfg<DK, DV>;
    constexpr int RB = Cfg::RB, F4 = Cfg::F4, FPT = Cfg::FPT, R = 1 + DK + DV;
    constexpr int Q4 = DV / 4;
    static_assert(kThreads % Q4 == 0, "a thread keeps one 4-column group across its rows");
    // Thread (w, q) = (tid / Q4, tid % Q4) owns the 4-column group q of the FPT consecutive
    // rows w*FPT .. w*FPT+FPT-1 of the block (clamped to the last row where the block has
    // fewer: surplus threads recompute and store identical values).  One load instruction
    // u still covers whole rows, and the logged k^ values a thread needs are contiguous.
    const int q = threadIdx.x % Q4, w = threadIdx.x / Q4;
    auto row_of = [&](int u) { return min(w * FPT + u, RB - 1); };
    __shared__ unsigned int s_bitmap[kBitmapSlots / 32];
    __shared__ int s_wbits[kThreads / 64];

    const int c = blockIdx.z, tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int N = d.N, Hv = d.Hv, C = d.C;
    const bool hist_copy = blockIdx.y == Hv;
    const int h = hist_copy ? 0 : blockIdx.y;
    const int layer = blockIdx.x / Cfg::NB, rb = blockIdx.x - layer * Cfg::NB;
    const int r0 = rb * RB;
    const float *__restrict__ replay_log = lp.replay_log[layer];
    float *__restrict__ state_pool = lp.state_pool[layer];

    // ---- every load that does not need the slot id, issued first: the lane's parents
    //      (lane i of every wave holds parents[i]) and this thread's share of the
    //      preflight (one lane's slot, accept node and node count, kPreRows parent entries
    //      with the slot and node count of their lane)
    const int par = parents[(int64_t)c * N + (lane < N ? lane : 0)];
    const int tl = tid < C ? tid : 0;
    const int so = slot_ids[tl], eo = accept_node[tl], no = lane_node_count(lane_nodes, d, tl);
    int pp[kPreRows], ps[kPreRows], pn[kPreRows];
#pragma unroll
    for (int u = 0; u < kPreRows; ++u) {
        const int idx = min(tid + kThreads * u, C * N - 1);
        pp[u] = parents[idx];
        ps[u] = slot_ids[idx / N];
        pn[u] = lane_node_count(lane_nodes, d, idx / N);
    }
    const int s = slot_ids[c], e = accept_node[c];
    const int st_in = *status;
    // ---- the state block (slot clamped into range; used only if the round commits), read
    //      non-temporal like its write-back: each line is used once, and cached loads had the
    //      state displace the logged rows and windows in L2 (3.48 -> 3.15 us per layer)
    const bool s_ok = s >= 0 && s < d.P;
    v4f *S4 = reinterpret_cast<v4f *>(state_pool + (((int64_t)(s_ok ? s : 0) * Hv + h) * DK + r0) * DV);
    v4f sv[FPT];
#pragma unroll
    for (int u = 0; u < FPT; ++u) sv[u] = __builtin_nontemporal_load(S4 + row_of(u) * Q4 + q);

    // ---- accepted path (every wave computes it) and the replay of its logged rows.
    //      The transitions are linear, so S_final = G S0 + A with G the product of the
    //      path's g and A the same replay started from a zero state; A needs only the
    //      logged rows, so it is accumulated while the state block streams in.  Path nodes
    //      are taken 4 at a time with all their loads issued together (more would cost occupancy).
    const unsigned int pm = path_mask(par, lane, N, e);
    const float *logc = replay_log + ((int64_t)c * N * Hv + h) * R;
    v4f acc[FPT];
#pragma unroll
    for (int u = 0; u < FPT; ++u) acc[u] = v4f{0.f, 0.f, 0.f, 0.f};
    float G = 1.0f;
    for (unsigned int bm = hist_copy ? 0u : pm; bm;) {
        constexpr int kChunk = 4;
        float cg[kChunk], ck[kChunk][FPT];
        v4f cd[kChunk];
#pragma unroll
        for (int j = 0; j < kChunk; ++j) {
            const bool has = bm != 0u;
            const int t = has ? __builtin_ctz(bm) : 0;
            bm = has ? bm & (bm - 1u) : 0u;
            const float *lrow = logc + (int64_t)t * Hv * R;
            const float g = lrow[0];
            const v4f dv4 = *reinterpret_cast<const v4u *>(lrow + 1 + DK + 4 * q);
            cg[j] = has ? g : 1.0f;
            cd[j] = has ? dv4 : v4f{0.f, 0.f, 0.f, 0.f};
            if constexpr (FPT % 4 == 0 && (kThreads / Q4) * FPT == RB) {  // no clamped rows: k^ as float4s
#pragma unroll
                for (int u = 0; u < FPT; u += 4) {
                    const v4f kv = *reinterpret_cast<const v4u *>(lrow + 1 + r0 + w * FPT + u);
                    ck[j][u] = has ? kv.x : 0.f;
                    ck[j][u + 1] = has ? kv.y : 0.f;
                    ck[j][u + 2] = has ? kv.z : 0.f;
                    ck[j][u + 3] = has ? kv.w : 0.f;
                }
            } else {
#pragma unroll
                for (int u = 0; u < FPT; ++u) {
                    const float kv = lrow[1 + r0 + row_of(u)];
                    ck[j][u] = has ? kv : 0.f;
                }
            }
        }
#pragma unroll
        for (int j = 0; j < kChunk; ++j) {
            G *= cg[j];
#pragma unroll
            for (int u = 0; u < FPT; ++u) {
                acc[u].x = fmaf(ck[j][u], cd[j].x, cg[j] * acc[u].x);
                acc[u].y = fmaf(ck[j][u], cd[j].y, cg[j] * acc[u].y);
                acc[u].z = fmaf(ck[j][u], cd[j].z, cg[j] * acc[u].z);
                acc[u].w = fmaf(ck[j][u], cd[j].w, cg[j] * acc[u].w);
            }
        }
    }

    // ---- preflight over every lane (slot range, duplicate slots via an LDS bitmap or a
    //      scan, node count, present nodes' parents, accept node); every workgroup reaches
    //      the same verdict
    const bool use_bitmap = d.P <= kBitmapSlots;
    if (use_bitmap)
        for (int w = tid; w < (d.P + 31) / 32; w += kThreads) s_bitmap[w] = 0u;
    lds_barrier();
    int bits = 0;
    for (int t = tid; t < C; t += kThreads) {
        const int st = t == tid ? so : slot_ids[t];
        if (st == -1) continue;
        const int et = t == tid ? eo : accept_node[t];
        const int nt = t == tid ? no : lane_node_count(lane_nodes, d, t);
        if (nt < 0 || nt > N) bits |= GDN_STATUS_NODES;
        if (et < -1 || et >= min(max(nt, 0), N)) bits |= GDN_STATUS_ACCEPT;  // a present node or -1
        if (st < -1 || st >= d.P) {
            bits |= GDN_STATUS_SLOT_RANGE;
        } else if (use_bitmap) {
            if (atomicOr(&s_bitmap[st >> 5], 1u << (st & 31)) & (1u << (st & 31))) bits |= GDN_STATUS_SLOT_DUP;
        } else {
            for (int o = 0; o < C; ++o)
                if (o != t && slot_ids[o] == st) bits |= GDN_STATUS_SLOT_DUP;
        }
    }
#pragma unroll
    for (int u = 0; u < kPreRows; ++u) {
        const int idx = tid + kThreads * u;
        if (idx < C * N && ps[u] != -1 && idx % N < pn[u] && (pp[u] < -1 || pp[u] >= idx % N))
            bits |= GDN_STATUS_PARENT;
    }
    for (int idx = tid + kThreads * kPreRows; idx < C * N; idx += kThreads) {  // beyond the first pass
        const int p = parents[idx];
        if (slot_ids[idx / N] != -1 && idx % N < lane_node_count(lane_nodes, d, idx / N) && (p < -1 || p >= idx % N))
            bits |= GDN_STATUS_PARENT;
    }
    {
        int wb = 0;
#pragma unroll
        for (int b = 0; b < 5; ++b)
            if (__builtin_amdgcn_ballot_w64((bits >> b) & 1)) wb |= 1 << b;
        if (lane == 0) s_wbits[wave] = wb;
    }
    lds_barrier();
    {
        int all = 0;
#pragma unroll
        for (int w = 0; w < kThreads / 64; ++w) all |= s_wbits[w];
        if (all) {
            if (blockIdx.x == 0 && blockIdx.y == 0 && tid == 0) atomicOr(status, all);  // once per lane
            return;
        }
    }
    if (st_in != 0 || s < 0 || e < 0) return;  // flagged round, padding lane, or nothing accepted

    if (hist_copy) {  // conv history <- commit window of the accepted node
        const int n4 = d.Ch * 3 / 4;
        const v4f *src = reinterpret_cast<const v4f *>(lp.commit_win[layer] + ((int64_t)c * N + e) * d.Ch * 3);
        v4f *dst = reinterpret_cast<v4f *>(lp.conv_hist[layer] + (int64_t)s * d.Ch * 3);
        // batches of kCopy loads, then their stores (one at a time, each store waited for its
        // load: a memory round trip per element), through raw buffer resources over the
        // window and the history row, so the elements past the end need no branch (their
        // loads read zero and their stores are dropped)
        constexpr int kCopy = 8, kStride = Cfg::NB * kThreads;
        const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(const_cast<v4f *>(src), 0, n4 * 16, kRsrcWord3);
        const __amdgpu_buffer_rsrc_t rd = __builtin_amdgcn_make_buffer_rsrc(dst, 0, n4 * 16, kRsrcWord3);
        for (int i0 = rb * kThreads + tid; i0 < n4; i0 += kCopy * kStride) {
            v4i buf[kCopy];
#pragma unroll
            for (int j = 0; j < kCopy; ++j) buf[j] = __builtin_amdgcn_raw_buffer_load_b128(rs, 16 * (i0 + j * kStride), 0, 0);
#pragma unroll
            for (int j = 0; j < kCopy; ++j) __builtin_amdgcn_raw_buffer_store_b128(buf[j], rd, 16 * (i0 + j * kStride), 0, kNonTemporal);
        }
        return;
    }

    // ---- S = G S0 + A, written back (non-temporal: the slot's state is read again only by
    // a later round's verify)
#pragma unroll
    for (int u = 0; u < FPT; ++u) {
        const v4f v = sv[u];
        __builtin_nontemporal_store(
            v4f{fmaf(G, v.x, acc[u].x), fmaf(G, v.y, acc[u].y), fmaf(G, v.z, acc[u].z), fmaf(G, v.w, acc[u].w)},
            S4 + row_of(u) * Q4 + q);
    }
}

template <int DK, int DV>
hipError_t launch(const Dims &d, int n_layers, const LayerPtrs &lp, const int32_t *slots, const int32_t *parents,
                  const int32_t *lane_nodes, const int32_t *accept, int32_t *status, hipStream_t stream) {
    hipLaunchKernelGGL((replay_commit_kernel<DK, DV>), dim3(CommitCfg<DK, DV>::NB * n_layers, d.Hv + 1, d.C),
                       dim3(kThreads), 0, stream, d, lp, slots, parents, lane_nodes, accept, status);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_replay_commit(const Dims &d, int n_layers, const LayerPtrs &lp, const int32_t *slot_ids,
                                const int32_t *parents, const int32_t *lane_nodes, const int32_t *accept_node,
                                int32_t *status, hipStream_t stream) {
#define GDN_COMMIT_CASE(K, V)                                                                               \
    if (d.dk == K && d.dv == V)                                                                             \
        return launch<K, V>(d, n_layers, lp, slot_ids, parents, lane_nodes, accept_node, status, stream);
#define GDN_COMMIT_ROW(K) GDN_COMMIT_CASE(K, 16) GDN_COMMIT_CASE(K, 32) GDN_COMMIT_CASE(K, 64) GDN_COMMIT_CASE(K, 128)
    GDN_COMMIT_ROW(16) GDN_COMMIT_ROW(32) GDN_COMMIT_ROW(64) GDN_COMMIT_ROW(128)
#undef GDN_COMMIT_ROW
#undef GDN_COMMIT_CASE
    return hipErrorInvalidValue;
}

}  // namespace gdn
