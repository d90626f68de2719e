// Tree conv step for gfx950: causal depthwise conv (d_conv = 4) + SiLU over each
// lane's slot-mapped history, following draft-tree parents, plus one 3-column commit
// window per node.
//
// What is computed: "perf(qwen35): fuse the DFlash2 concurrent verify Gated DeltaNet
// route", Optimizations, first bullet.  Column and tap order: "llama-cpp-bonsai-gdn-conv
// .patch", ssm-conv.cu hunk (history columns first, then tokens; the 4-tap sum runs from
// the oldest column; no bias).
//
// Design (HBM-bound, ~0.25 flop/B): one workgroup per (lane, 64-channel block).  The
// block's 3 history columns and the lane's N token rows are staged once in LDS as
// 4-float channel groups, so every ancestor tap a tree node needs is an LDS read and each
// input byte leaves HBM once.  All global loads (parents, tokens, weights, history) are
// issued together up front; tree ancestors are found with lane shuffles.  conv_out rows go out as
// coalesced 16-byte stores; the commit window of 4 channels is 12 consecutive floats,
// written as three 16-byte stores.
#include "gdn_device.h"
#include "gdn_internal.h"

namespace gdn {
namespace {

constexpr int kThreads = 256;
constexpr int kChBlock = 64;           // channels per workgroup
constexpr int kGroups = kChBlock / 4;  // 4-float channel groups per LDS row
constexpr int kRowsPerPass = kThreads / kGroups;

__device__ inline float silu(float z) { return z / (1.0f + expf(-z)); }

__global__ __launch_bounds__(kThreads) void conv_tree_step_kernel(
    Dims d, const float *__restrict__ x, const float *__restrict__ conv_w, const float *__restrict__ conv_hist,
    const int32_t *__restrict__ slot_ids, const int32_t *__restrict__ parents, const int32_t *__restrict__ lane_nodes,
    float *__restrict__ conv_out, float *__restrict__ commit_win, int32_t *__restrict__ status) {
    extern __shared__ v4f rows4[];  // [3 + N][kGroups]: history columns 0..2, then token rows
    __shared__ int s_wbits[kThreads / 64];
    __shared__ v4f s_chunks[kThreads * 3];  // window chunks, transposed per wave

    const int c = blockIdx.y, tid = threadIdx.x;
    const int N = d.N, Ch = d.Ch;
    const int ch0 = blockIdx.x * kChBlock;
    const int ng = min(kChBlock, Ch - ch0) / 4;  // Ch is a multiple of 16
    float *rows = reinterpret_cast<float *>(rows4);

    // ---- every global load first: parents, this thread's duplicate-slot probe, token
    //      rows of the block (into LDS), the 4 taps of this thread's channel group
    const int lane = tid & 63;
    const int par = parents[(int64_t)c * N + (lane < N ? lane : 0)];  // lane i of every wave holds parent i
    const int nv = lane_node_count(lane_nodes, d, c);                   // nodes present in this lane
    const int so = slot_ids[tid < d.C ? tid : 0];
    const v4f *x4 = reinterpret_cast<const v4f *>(x + ((int64_t)c * N) * Ch + ch0);
    const int q = tid % kGroups;  // this thread's channel group (fixed: 256 % 16 == 0)
    const int qc = q < ng ? q : 0;
    const v4f *w4 = reinterpret_cast<const v4f *>(conv_w + (int64_t)(ch0 + 4 * qc) * 4);
    const v4f wa = w4[0], wb = w4[1], wc = w4[2], wd = w4[3];  // taps of channels ch..ch+3
    constexpr int XPT = (GDN_MAX_NODES + kRowsPerPass - 1) / kRowsPerPass;  // token rows per thread
    v4f xr[XPT];
#pragma unroll
    for (int u = 0; u < XPT; ++u) {
        const int i = tid / kGroups + kRowsPerPass * u;
        xr[u] = x4[(int64_t)(i < N ? i : 0) * (Ch / 4) + qc];
    }
    const int s = slot_ids[c];
    if (s == -1) return;  // padding lane
    const bool s_ok = s >= 0 && s < d.P;
    // ---- history block [ch][3] (contiguous), this thread's float of it
    const int hn = ng * 12;
    const float hv = conv_hist[((int64_t)(s_ok ? s : 0) * Ch + ch0) * 3 + (tid < hn ? tid : 0)];
    // ---- lane validity (slot range, duplicate slot, node count, present nodes' parents);
    //      nothing is written for a bad lane
    int bits = s_ok ? 0 : GDN_STATUS_SLOT_RANGE;
    if (tid < d.C && tid != c && so == s) bits |= GDN_STATUS_SLOT_DUP;
    for (int o = tid + kThreads; o < d.C; o += kThreads)
        if (o != c && slot_ids[o] == s) bits |= GDN_STATUS_SLOT_DUP;
    if (nv < 0 || nv > N) bits |= GDN_STATUS_NODES;
    if (tid < nv && tid < N && (par < -1 || par >= tid)) bits |= GDN_STATUS_PARENT;
    {
        int wb = 0;
#pragma unroll
        for (int b = 0; b < 5; ++b)
            if (__builtin_amdgcn_ballot_w64((bits >> b) & 1)) wb |= 1 << b;
        if ((tid & 63) == 0) s_wbits[tid >> 6] = wb;
    }
    // ---- stage the block: token rows, and the history transposed into rows 0..2 (a 64-channel
    // block has 192 history floats: one per thread)
#pragma unroll
    for (int u = 0; u < XPT; ++u) {
        const int i = tid / kGroups + kRowsPerPass * u;
        if (i < N && q < ng) rows4[(3 + i) * kGroups + q] = xr[u];
    }
    if (tid < hn) rows[(tid % 3) * kChBlock + tid / 3] = hv;
    lds_barrier();
    {
        int all = 0;
#pragma unroll
        for (int w = 0; w < kThreads / 64; ++w) all |= s_wbits[w];
        if (all) {
            if (blockIdx.x == 0 && tid == 0 && status) atomicOr(status, all);
            return;
        }
    }

    // ---- conv + SiLU and the commit windows, one node row per pass.  Window sources of
    //      node i, oldest first: LDS row r < 3 is history column r, row 3 + a is the token
    //      of node a; the newest source is node i itself, then its ancestors (found with
    //      lane shuffles over the parents held by lanes 0..N-1), then history columns 2, 1, 0.
    //      A node's windows in the block are 3 * kGroups consecutive 16-byte chunks, held by
    //      one row of 16 lanes; they go through a wave-private transpose in LDS so that each
    //      store instruction writes consecutive chunks from consecutive lanes (whole lines)
    //      instead of 16-byte pieces at a 48-byte lane stride.
    const int ch = ch0 + 4 * q;
    const int l16 = tid % kGroups;  // == q
    v4f *chunks = s_chunks + 3 * (tid - l16);  // this row's 3 * kGroups chunks
#pragma unroll
    for (int u = 0; u < XPT; ++u) {
        const int i = tid / kGroups + kRowsPerPass * u;
        const int n0 = i < N ? i : 0;
        const int n1 = __shfl(par, n0);
        const int n2s = __shfl(par, n1 >= 0 ? n1 : 0);
        const int n2 = n1 >= 0 ? n2s : -1;
        const int n3s = __shfl(par, n2 >= 0 ? n2 : 0);
        const int n3 = n2 >= 0 ? n3s : -1;
        if (i >= nv) continue;  // absent node (nv <= N: a bad count returned above); uniform per row
        const int cnt = 1 + (n1 >= 0) + (n2 >= 0) + (n3 >= 0);
        const int nn[4] = {n0, n1, n2, n3};
        int src[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) src[3 - k] = k < cnt ? 3 + nn[k] : 2 - (k - cnt);
        const v4f t0 = rows4[src[0] * kGroups + q];
        const v4f t1 = rows4[src[1] * kGroups + q];
        const v4f t2 = rows4[src[2] * kGroups + q];
        const v4f t3 = rows4[src[3] * kGroups + q];
        // sum over taps from the oldest column, as in the pages' kernel
        float za = 0.f, zb = 0.f, zc = 0.f, zd = 0.f;
        za = fmaf(t0.x, wa.x, za); za = fmaf(t1.x, wa.y, za); za = fmaf(t2.x, wa.z, za); za = fmaf(t3.x, wa.w, za);
        zb = fmaf(t0.y, wb.x, zb); zb = fmaf(t1.y, wb.y, zb); zb = fmaf(t2.y, wb.z, zb); zb = fmaf(t3.y, wb.w, zb);
        zc = fmaf(t0.z, wc.x, zc); zc = fmaf(t1.z, wc.y, zc); zc = fmaf(t2.z, wc.z, zc); zc = fmaf(t3.z, wc.w, zc);
        zd = fmaf(t0.w, wd.x, zd); zd = fmaf(t1.w, wd.y, zd); zd = fmaf(t2.w, wd.z, zd); zd = fmaf(t3.w, wd.w, zd);
        const int64_t row = (int64_t)c * N + i;
        if (q < ng) *reinterpret_cast<v4f *>(conv_out + row * Ch + ch) = v4f{silu(za), silu(zb), silu(zc), silu(zd)};
        // commit window = taps 1..3 of each channel, [ch][3] layout: 12 floats for 4 channels
        chunks[3 * l16] = v4f{t1.x, t2.x, t3.x, t1.y};
        chunks[3 * l16 + 1] = v4f{t2.y, t3.y, t1.z, t2.z};
        chunks[3 * l16 + 2] = v4f{t3.z, t1.w, t2.w, t3.w};
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        // (non-temporal: the windows are read again only by the commit, after the round)
        v4f *wdst = reinterpret_cast<v4f *>(commit_win + (row * Ch + ch0) * 3);
#pragma unroll
        for (int k = 0; k < 3; ++k) {
            const int j = l16 + kGroups * k;  // chunk j holds part j % 3 of channel group j / 3
            if (j < 3 * ng) __builtin_nontemporal_store(chunks[j], wdst + j);
        }
        // the row's chunks are read before the next pass overwrites them
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }
}

}  // namespace

hipError_t launch_conv_tree_step(const Dims &d, const float *x, const float *conv_w, const float *conv_hist,
                                 const int32_t *slot_ids, const int32_t *parents, const int32_t *lane_nodes,
                                 float *conv_out, float *commit_win, int32_t *status, hipStream_t stream) {
    const dim3 grid((d.Ch + kChBlock - 1) / kChBlock, d.C);
    const size_t lds = sizeof(v4f) * (3 + d.N) * kGroups;
    hipLaunchKernelGGL(conv_tree_step_kernel, grid, dim3(kThreads), lds, stream, d, x, conv_w, conv_hist, slot_ids,
                       parents, lane_nodes, conv_out, commit_win, status);
    return hipGetLastError();
}

}  // namespace gdn
