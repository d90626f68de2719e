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
// float4 channel groups, so every ancestor tap a tree node needs is an LDS read and each
// input byte leaves HBM once.  Tap sources are resolved per node once (uniform over the
// workgroup).  conv_out rows go out as coalesced float4 stores; the commit window of 4
// channels is 12 consecutive floats, written as three float4 stores.
#include "gdn_internal.h"

namespace gdn {
namespace {

constexpr int kThreads = 256;
constexpr int kChBlock = 64;              // channels per workgroup
constexpr int kGroups = kChBlock / 4;     // float4 channel groups per LDS row

__device__ inline float silu(float z) { return z / (1.0f + expf(-z)); }

__global__ __launch_bounds__(kThreads) void conv_tree_step_kernel(
    Dims d, const float *__restrict__ x, const float *__restrict__ conv_w, const float *__restrict__ conv_hist,
    const int32_t *__restrict__ slot_ids, const int32_t *__restrict__ parents, float *__restrict__ conv_out,
    float *__restrict__ commit_win, int32_t *__restrict__ status) {
    extern __shared__ float4 rows4[];  // [3 + N][kGroups]: history columns 0..2, then token rows
    __shared__ int s_bits;
    __shared__ int s_src[GDN_MAX_NODES][4];

    const int c = blockIdx.y;
    const int s = slot_ids[c];
    if (s == -1) return;  // padding lane
    const int bits = lane_status_bits(slot_ids, parents, d, c, s, &s_bits);
    if (bits) {
        if (blockIdx.x == 0 && threadIdx.x == 0 && status) atomicOr(status, bits);
        return;
    }

    const int N = d.N, Ch = d.Ch, tid = threadIdx.x;
    const int ch0 = blockIdx.x * kChBlock;
    const int ng = min(kChBlock, Ch - ch0) / 4;  // Ch is a multiple of 16
    float *rows = reinterpret_cast<float *>(rows4);

    // Window sources of node i, oldest first: LDS row r < 3 is history column r,
    // row 3 + a is the token of node a.  Newest source is node i itself, then its
    // ancestors, then history columns 2, 1, 0.
    if (tid < N) {
        const int32_t *par = parents + (int64_t)c * N;
        const int n0 = tid;
        const int n1 = par[n0];
        const int n2 = n1 >= 0 ? par[n1] : -1;
        const int n3 = n2 >= 0 ? par[n2] : -1;
        const int nn[4] = {n0, n1, n2, n3};
        const int cnt = 1 + (n1 >= 0) + (n2 >= 0) + (n3 >= 0);
#pragma unroll
        for (int k = 0; k < 4; ++k) s_src[tid][3 - k] = k < cnt ? 3 + nn[k] : 2 - (k - cnt);
    }
    // history block [ch][3] (contiguous) transposed into rows 0..2
    const float *hsrc = conv_hist + ((int64_t)s * Ch + ch0) * 3;
    for (int idx = tid; idx < ng * 12; idx += kThreads) rows[(idx % 3) * kChBlock + idx / 3] = hsrc[idx];
    // token rows
    const float4 *x4 = reinterpret_cast<const float4 *>(x + ((int64_t)c * N) * Ch + ch0);
    for (int idx = tid; idx < N * ng; idx += kThreads) {
        const int i = idx / ng, q = idx - i * ng;
        rows4[(3 + i) * kGroups + q] = x4[(int64_t)i * (Ch / 4) + q];
    }
    __syncthreads();

    for (int idx = tid; idx < N * ng; idx += kThreads) {
        const int i = idx / ng, q = idx - i * ng;
        const int ch = ch0 + 4 * q;
        const float4 *w4 = reinterpret_cast<const float4 *>(conv_w + (int64_t)ch * 4);
        const float4 wa = w4[0], wb = w4[1], wc = w4[2], wd = w4[3];  // taps of channels ch..ch+3
        const float4 t0 = rows4[s_src[i][0] * kGroups + q];
        const float4 t1 = rows4[s_src[i][1] * kGroups + q];
        const float4 t2 = rows4[s_src[i][2] * kGroups + q];
        const float4 t3 = rows4[s_src[i][3] * kGroups + q];
        // sum over taps from the oldest column, as in the pages' kernel
        float za = 0.f, zb = 0.f, zc = 0.f, zd = 0.f;
        za = fmaf(t0.x, wa.x, za); za = fmaf(t1.x, wa.y, za); za = fmaf(t2.x, wa.z, za); za = fmaf(t3.x, wa.w, za);
        zb = fmaf(t0.y, wb.x, zb); zb = fmaf(t1.y, wb.y, zb); zb = fmaf(t2.y, wb.z, zb); zb = fmaf(t3.y, wb.w, zb);
        zc = fmaf(t0.z, wc.x, zc); zc = fmaf(t1.z, wc.y, zc); zc = fmaf(t2.z, wc.z, zc); zc = fmaf(t3.z, wc.w, zc);
        zd = fmaf(t0.w, wd.x, zd); zd = fmaf(t1.w, wd.y, zd); zd = fmaf(t2.w, wd.z, zd); zd = fmaf(t3.w, wd.w, zd);
        const int64_t row = (int64_t)c * N + i;
        reinterpret_cast<float4 *>(conv_out + row * Ch + ch)[0] = make_float4(silu(za), silu(zb), silu(zc), silu(zd));
        // commit window = taps 1..3 of each channel, [ch][3] layout: 12 floats for 4 channels
        float4 *wdst = reinterpret_cast<float4 *>(commit_win + (row * Ch + ch) * 3);
        wdst[0] = make_float4(t1.x, t2.x, t3.x, t1.y);
        wdst[1] = make_float4(t2.y, t3.y, t1.z, t2.z);
        wdst[2] = make_float4(t3.z, t1.w, t2.w, t3.w);
    }
}

}  // namespace

hipError_t launch_conv_tree_step(const Dims &d, const float *x, const float *conv_w, const float *conv_hist,
                                 const int32_t *slot_ids, const int32_t *parents, float *conv_out,
                                 float *commit_win, int32_t *status, hipStream_t stream) {
    const dim3 grid((d.Ch + kChBlock - 1) / kChBlock, d.C);
    const size_t lds = sizeof(float4) * (3 + d.N) * kGroups;
    hipLaunchKernelGGL(conv_tree_step_kernel, grid, dim3(kThreads), lds, stream, d, x, conv_w, conv_hist, slot_ids,
                       parents, conv_out, commit_win, status);
    return hipGetLastError();
}

}  // namespace gdn
