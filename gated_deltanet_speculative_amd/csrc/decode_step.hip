// Plain decode step for gfx950: the step of a lane without a draft, which commits its
// post-step state to the slot at once instead of going through a verify and a commit.
// Two launches on the caller's stream:
//   conv_step_kernel    causal conv + SiLU over a chain of tokens per lane, writing the
//                       slot's new history (the last 3 columns) back in place;
//   decode_step_kernel  one token of the gated delta rule applied to the slot's state
//                       in place, with the output row;
// or, for one token, both in one:
//   conv_decode_group_kernel  one workgroup per (lane, q/k head) forms the conv output of
//                       the group's channels once, writes their new history after its
//                       barrier, and runs the recurrence of every value block of the group;
//   conv_decode_kernel  (groups of more than 16 blocks) one wave per value block, each
//                       forming the conv of the channels it needs.  A q/k channel then
//                       feeds several workgroups, so its history may be rewritten in place
//                       only once all of them have read it: the last of them to count
//                       itself on a caller-provided counter writes it.
//
// What is computed: "Feature/support dflash2", deferred-state commit message (a step the
// drafter did not draft for commits its post-step state to the slot immediately);
// "qwen35: DSpark speculative decoding (Qwen3.8-27B drafters)", DeltaNet-block commit
// message (one conv-step kernel: history window, silu(conv), in-place history
// write-back; the gated delta rule in place, no state copy) and raw-gate commit message
// (sigmoid(beta), softplus(alpha + dt_bias) * A applied in-kernel); conv tap order from
// "llama-cpp-bonsai-gdn-conv.patch", ssm-conv.cu hunk.
//
// Both kernels mutate the pools, so each is a transaction like the commit: every
// workgroup evaluates the slot preflight over all lanes (slot range, duplicate slots)
// and honours bits already in *status, and writes nothing unless the verdict is clean.
// Loads that do not depend on the verdict are issued before it.
#include "gdn_device.h"
#include "gdn_internal.h"

namespace gdn {
namespace {

constexpr int kThreads = 256;
constexpr int kTokChunk = 8;  // conv step: tokens loaded together
constexpr int kTokRun = 32;   // conv step: tokens per thread (runs of a long chain in parallel)
using LaneSlots = LaneSlotsT<kThreads>;

template <int M>
__device__ inline float row_ror(float x) {  // lane (i - M) mod 16 of each row of 16 lanes (DPP row_ror)
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x120 + M, 0xF, 0xF, false));
}

// Sum over the lanes of a wave that share lane % Q (Q = 4 or 8): rotations within each
// row of 16 lanes, then the row pairs and wave halves exchanged by permlane swaps (with
// both operands equal, the two results of a swap add up to the pairwise sum).
template <int Q>
__device__ inline float sum_lanes_sharing(float x) {
    static_assert(Q == 4 || Q == 8, "column groups per wave row");
    if constexpr (Q == 4) x += row_ror<4>(x);
    x += row_ror<8>(x);
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
    const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// ---- conv step: thread = (lane c = blockIdx.y, 4-channel group g, run r = blockIdx.z of
//      kTokRun consecutive tokens).  The window slides over the run in registers, oldest
//      column first (tap 0 multiplies it); a run's first window is the 3 tokens before it,
//      or the slot's history for run 0.  The thread of run 0 is the only one that reads the
//      slot's history, and it alone writes the new one (the last 3 columns of history +
//      chain, formed from the chain's last tokens), so the in-place update has no hazard.
__global__ __launch_bounds__(kThreads) void conv_step_kernel(Dims d, const float *__restrict__ x,
                                                             const float *__restrict__ conv_w,
                                                             float *__restrict__ conv_hist,
                                                             const int32_t *__restrict__ slot_ids,
                                                             float *__restrict__ conv_out, int32_t *__restrict__ status) {
    __shared__ unsigned int s_bitmap[kBitmapSlots / 32];
    __shared__ int s_word;
    const int c = blockIdx.y, G4 = d.Ch / 4, N = d.N;
    const int g = blockIdx.x * kThreads + threadIdx.x, gc = g < G4 ? g : G4 - 1;
    const int t0 = blockIdx.z * kTokRun, tn = min(kTokRun, N - t0);
    const bool first = blockIdx.z == 0;
    const LaneSlots lanes(slot_ids, d.C);
    const int s = slot_ids[c];
    const int st_in = *status;
    const bool s_ok = s >= 0 && s < d.P;
    // loads first: taps, the run's first window (history, or the 3 tokens before the run),
    // the run's first tokens, and (run 0) the chain's last 3 tokens for the new history
    v4f w[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) w[e] = reinterpret_cast<const v4f *>(conv_w)[4 * gc + e];
    v4f *hp = reinterpret_cast<v4f *>(conv_hist + ((int64_t)(s_ok ? s : 0) * d.Ch + 4 * gc) * 3);
    const v4f *xr = reinterpret_cast<const v4f *>(x + (int64_t)c * N * d.Ch) + gc;
    v4f a, b, cc;  // window columns, oldest first
    if (first) {
        const v4f h0 = hp[0], h1 = hp[1], h2 = hp[2];  // layout [ch][3]: 12 consecutive floats
        a = v4f{h0.x, h0.w, h1.z, h2.y};
        b = v4f{h0.y, h1.x, h1.w, h2.z};
        cc = v4f{h0.z, h1.y, h2.x, h2.w};
    } else {
        a = xr[(int64_t)(t0 - 3) * G4];
        b = xr[(int64_t)(t0 - 2) * G4];
        cc = xr[(int64_t)(t0 - 1) * G4];
    }
    v4f xt[kTokChunk];
#pragma unroll
    for (int t = 0; t < kTokChunk; ++t) xt[t] = xr[(int64_t)min(t0 + t, N - 1) * G4];
    v4f last[3];  // run 0: tokens N-3..N-1 (clamped; only those that exist are used)
    if (first)
#pragma unroll
        for (int k = 0; k < 3; ++k) last[k] = xr[(int64_t)max(N - 3 + k, 0) * G4];

    const int bits = slot_preflight<kThreads>(lanes, slot_ids, d.C, d.P, s_bitmap, &s_word);
    if (bits || st_in) {
        if (bits && blockIdx.x == 0 && blockIdx.y == 0 && blockIdx.z == 0 && threadIdx.x == 0) atomicOr(status, bits);
        return;
    }
    if (s < 0 || g >= G4) return;  // padding lane, or past the channels

    // the new history (run 0): the last 3 columns of [history; chain]
    v4f nh[3];
    if (first) {
        const v4f old[3] = {a, b, cc};
#pragma unroll
        for (int k = 0; k < 3; ++k) nh[k] = N - 3 + k >= 0 ? last[k] : old[N + k];
    }
    v4f *orow = reinterpret_cast<v4f *>(conv_out + (int64_t)c * N * d.Ch) + g;
    for (int u0 = 0; u0 < tn; u0 += kTokChunk) {
        if (u0 > 0) {
#pragma unroll
            for (int t = 0; t < kTokChunk; ++t) xt[t] = xr[(int64_t)min(t0 + u0 + t, N - 1) * G4];
        }
#pragma unroll
        for (int t = 0; t < kTokChunk; ++t) {
            if (u0 + t >= tn) break;
            v4f y;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                float z = a[e] * w[e][0];
                z = fmaf(b[e], w[e][1], z);
                z = fmaf(cc[e], w[e][2], z);
                z = fmaf(xt[t][e], w[e][3], z);
                y[e] = fast_silu(z);  // (hardware exp2 and reciprocal, about 1 ulp each)
            }
            orow[(int64_t)(t0 + u0 + t) * G4] = y;
            a = b;
            b = cc;
            cc = xt[t];
        }
    }
    if (first) {  // in place: only this thread reads or writes these 12 floats
        hp[0] = v4f{nh[0].x, nh[1].x, nh[2].x, nh[0].y};
        hp[1] = v4f{nh[1].y, nh[2].y, nh[0].z, nh[1].z};
        hp[2] = v4f{nh[2].z, nh[0].w, nh[1].w, nh[2].w};
    }
}

// ---- decode step: workgroup = one wave = (lane c = blockIdx.y, value head h, block of JB value
//      columns).  Thread (r, q) = (lane / Q4, lane % Q4) holds the 4 columns q of the RPL
//      consecutive rows r*RPL.. of the block, so one load instruction covers RG whole row
//      segments of the block.  The wave owns every row of its columns: the column sums
//      S^T k^ and S^T q^ reduce across its lanes (DPP rotations and permlane swaps), with no
//      cross-wave exchange, and the wave writes its columns back as soon as its own loads
//      have arrived.
template <int DK, int DV>
struct DecodeCfg {
    static constexpr int JB = DV < 32 ? DV : 32;  // value columns per wave
    static constexpr int NB = DV / JB;
    static constexpr int Q4 = JB / 4;             // 4-column groups (4 or 8)
    static constexpr int RG = 64 / Q4;            // row groups
    static constexpr int RPL = DK / RG;           // consecutive rows per thread
    static_assert(RPL >= 1 && RG * RPL == DK, "rows tile the wave");
};

// The recurrence of one token on a wave's block once its inputs are in registers: this
// thread's q / k rows qq, kq, value columns v, raw gates and state rows sv (loaded from S4);
// writes the rows back and, in row group 0, the output columns to *o4.
template <int DK, int DV>
__device__ __forceinline__ void decode_block(const float (&qq)[DecodeCfg<DK, DV>::RPL],
                                             const float (&kq)[DecodeCfg<DK, DV>::RPL], v4f v, float braw, float araw,
                                             float Ah, const v4f (&sv)[DecodeCfg<DK, DV>::RPL], v4f *S4, int i0, int r,
                                             v4f *o4) {
    constexpr int Q4 = DecodeCfg<DK, DV>::Q4, RPL = DecodeCfg<DK, DV>::RPL;
    // |q|^2, |k|^2, q . k and the column sums of k_i S[i][j], q_i S[i][j] over this thread's
    // rows, then over the row groups (the lanes sharing q)
    float ssq = 0.f, ssk = 0.f, sqk = 0.f;
    v4f pu = {0.f, 0.f, 0.f, 0.f}, pw = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int e = 0; e < RPL; ++e) {
        ssq = fmaf(qq[e], qq[e], ssq);
        ssk = fmaf(kq[e], kq[e], ssk);
        sqk = fmaf(qq[e], kq[e], sqk);
        pu += kq[e] * sv[e];
        pw += qq[e] * sv[e];
    }
    ssq = sum_lanes_sharing<Q4>(ssq);
    ssk = sum_lanes_sharing<Q4>(ssk);
    sqk = sum_lanes_sharing<Q4>(sqk);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        pu[e] = sum_lanes_sharing<Q4>(pu[e]);
        pw[e] = sum_lanes_sharing<Q4>(pw[e]);
    }
    const float rq = inv_norm(ssq), rk = inv_norm(ssk);
    // S' = g S;  delta = beta (v - S'^T k^);  S_new = S' + k^ delta^T;
    // o = S_new^T q^ / sqrt(d_k) = (g S^T q^ + (q^ . k^) delta) / sqrt(d_k)
    const float g = fast_exp(fast_softplus(araw) * Ah), beta = fast_sigmoid(braw);
    const v4f delta = beta * (v - (g * rk) * pu);
#pragma unroll
    for (int e = 0; e < RPL; ++e) __builtin_nontemporal_store(g * sv[e] + (kq[e] * rk) * delta, S4 + (i0 + e) * (DV / 4));
    if (r == 0) *o4 = ((g * rq) * pw + (sqk * rq * rk) * delta) * (1.0f / sqrtf((float)DK));
}


template <int DK, int DV>
__global__ __launch_bounds__(64) void decode_step_kernel(
    Dims d, const float *__restrict__ qkv, const float *__restrict__ beta_logits,
    const float *__restrict__ alpha_logits, int64_t gate_stride, const float *__restrict__ dt_bias,
    const float *__restrict__ A, float *__restrict__ state_pool, const int32_t *__restrict__ slot_ids,
    float *__restrict__ out, int32_t *__restrict__ status) {
    using Cfg = DecodeCfg<DK, DV>;
    constexpr int JB = Cfg::JB, NB = Cfg::NB, Q4 = Cfg::Q4, RPL = Cfg::RPL;
    __shared__ unsigned int s_bitmap[kBitmapSlots / 32];
    __shared__ int s_word;

    const int c = blockIdx.y, h = blockIdx.x / NB, jb = blockIdx.x - h * NB, j0 = jb * JB;
    const int kh = h % d.Hk;
    const int lane = threadIdx.x;
    const int q = lane % Q4, r = lane / Q4, i0 = r * RPL;
    // loads in the order they are needed, all issued before any is consumed: this lane's
    // slot id (a vector load, so that its wait does not hold up the loads behind it),
    // the preflight's slot ids, this thread's q / k rows, value columns and gates, then the
    // state block
    const int s_v = __builtin_bit_cast(
        int, __builtin_amdgcn_raw_buffer_load_b32(
                 __builtin_amdgcn_make_buffer_rsrc(const_cast<int32_t *>(slot_ids), 0, 4 * d.C, 0x00020000), 4 * c, 0,
                 0));
    const LaneSlotsT<64> lanes(slot_ids, d.C);
    const int st_in = *status;
    const float *row = qkv + (int64_t)c * d.Ch;
    float kq[RPL], qq[RPL];
#pragma unroll
    for (int e = 0; e < RPL; ++e) {
        qq[e] = row[kh * DK + i0 + e];
        kq[e] = row[d.Hk * DK + kh * DK + i0 + e];
    }
    const v4f v = reinterpret_cast<const v4f *>(row + 2 * d.Hk * DK + h * DV + j0)[q];
    const float braw = beta_logits[(int64_t)c * gate_stride + h];
    const float araw = alpha_logits[(int64_t)c * gate_stride + h] + dt_bias[h];
    const float Ah = A[h];
    __builtin_amdgcn_sched_barrier(0);
    const int s = __builtin_amdgcn_readfirstlane(s_v);
    const bool s_ok = s >= 0 && s < d.P;
    v4f *S4 = reinterpret_cast<v4f *>(state_pool + ((int64_t)(s_ok ? s : 0) * d.Hv + h) * DK * DV + j0) + q;
    // the state block (slot clamped into range; written back only if the step commits), read
    // non-temporal like its write-back: each line is used once (6.28 -> 4.76 us per step)
    v4f sv[RPL];
#pragma unroll
    for (int e = 0; e < RPL; ++e) sv[e] = __builtin_nontemporal_load(S4 + (i0 + e) * (DV / 4));

    const int bits = slot_preflight<64>(lanes, slot_ids, d.C, d.P, s_bitmap, &s_word);
    if (bits || st_in) {
        if (bits && blockIdx.x == 0 && blockIdx.y == 0 && lane == 0) atomicOr(status, bits);
        return;
    }
    if (s < 0) return;  // padding lane (uniform over the wave)

    decode_block<DK, DV>(qq, kq, v, braw, araw, Ah, sv, S4, i0, r, reinterpret_cast<v4f *>(out + ((int64_t)c * d.Hv + h) * DV + j0) + q);
}

// ---- fused plain step: the waves of decode_step_kernel, each first forming the conv output of
//      the channels it needs (the 2 d_k channels of its q/k head and the JB value channels of
//      its block) from the slot's history, the token and the taps, into LDS.  The history is
//      updated in place once every reader is done with it: a wave writes its value channels'
//      new history itself (no other wave reads them); the q/k channels are read by the
//      R * NB waves of their (lane, q/k head), so the wave that arrives last at
//      sync[(c * H_k + kh) * GDN_SYNC_STRIDE] -- an atomic count taken after the wave's
//      history reads are back -- writes their new history and sets the count back to zero.
//      One counter per 128-byte line: packed into two lines, the 512 counts of the bench
//      shape queued on one L2 channel (2.4 us of a 9.3 us launch).
template <int DK, int DV>
__global__ __launch_bounds__(64) void conv_decode_kernel(
    Dims d, const float *__restrict__ x, const float *__restrict__ conv_w, float *__restrict__ conv_hist,
    const float *__restrict__ beta_logits, const float *__restrict__ alpha_logits, int64_t gate_stride,
    const float *__restrict__ dt_bias, const float *__restrict__ A, float *__restrict__ state_pool,
    const int32_t *__restrict__ slot_ids, int32_t *__restrict__ sync, float *__restrict__ out,
    int32_t *__restrict__ status) {
    using Cfg = DecodeCfg<DK, DV>;
    constexpr int JB = Cfg::JB, NB = Cfg::NB, Q4 = Cfg::Q4, RPL = Cfg::RPL;
    constexpr int GQK = DK / 2, GV = JB / 4, NI = (GQK + GV + 63) / 64;  // 4-channel groups; per lane
    __shared__ unsigned int s_bitmap[kBitmapSlots / 32];
    __shared__ int s_word;
    __shared__ __align__(16) float s_y[2 * DK + JB];  // conv outputs: q rows, k rows, value columns

    const int c = blockIdx.y, h = blockIdx.x / NB, jb = blockIdx.x - h * NB, j0 = jb * JB;
    const int kh = h % d.Hk;
    const int lane = threadIdx.x;
    const int q = lane % Q4, r = lane / Q4, i0 = r * RPL;
    // loads in the order they are needed, as in decode_step_kernel: slot id, the preflight's
    // slot ids, the taps and token of this lane's channel groups (item u = group lane + 64 u
    // of the q/k slab, then of the value block), the gates; then the history and the state
    const int s_v = __builtin_bit_cast(
        int, __builtin_amdgcn_raw_buffer_load_b32(
                 __builtin_amdgcn_make_buffer_rsrc(const_cast<int32_t *>(slot_ids), 0, 4 * d.C, 0x00020000), 4 * c, 0,
                 0));
    const LaneSlotsT<64> lanes(slot_ids, d.C);
    const int st_in = *status;
    int ch[NI], at[NI];
    v4f w[NI][4], xv[NI];
#pragma unroll
    for (int u = 0; u < NI; ++u) {
        const int f = min(lane + 64 * u, GQK + GV - 1);
        ch[u] = f < DK / 4 ? kh * DK + 4 * f
                : f < GQK  ? d.Hk * DK + kh * DK + 4 * (f - DK / 4)
                           : 2 * d.Hk * DK + h * DV + j0 + 4 * (f - GQK);
        at[u] = f < GQK ? 4 * f : 2 * DK + 4 * (f - GQK);
#pragma unroll
        for (int e = 0; e < 4; ++e) w[u][e] = reinterpret_cast<const v4f *>(conv_w)[ch[u] + e];
        xv[u] = *reinterpret_cast<const v4f *>(x + (int64_t)c * d.Ch + ch[u]);
    }
    const float braw = beta_logits[(int64_t)c * gate_stride + h];
    const float araw = alpha_logits[(int64_t)c * gate_stride + h] + dt_bias[h];
    const float Ah = A[h];
    __builtin_amdgcn_sched_barrier(0);
    const int s = __builtin_amdgcn_readfirstlane(s_v);
    const bool s_ok = s >= 0 && s < d.P;
    v4f hv[NI][3];  // history of the item's 4 channels, layout [ch][3]: 12 consecutive floats
#pragma unroll
    for (int u = 0; u < NI; ++u)
#pragma unroll
        for (int k = 0; k < 3; ++k)
            hv[u][k] = reinterpret_cast<const v4f *>(conv_hist + ((int64_t)(s_ok ? s : 0) * d.Ch + ch[u]) * 3)[k];
    v4f *S4 = reinterpret_cast<v4f *>(state_pool + ((int64_t)(s_ok ? s : 0) * d.Hv + h) * DK * DV + j0) + q;
    v4f sv[RPL];
#pragma unroll
    for (int e = 0; e < RPL; ++e) sv[e] = __builtin_nontemporal_load(S4 + (i0 + e) * (DV / 4));

    // conv + SiLU of the items' channels (the conv step's order of taps and accumulation)
#pragma unroll
    for (int u = 0; u < NI; ++u) {
        if (GQK + GV < 64 * NI && lane + 64 * u >= GQK + GV) continue;
        const v4f h0 = hv[u][0], h1 = hv[u][1], h2 = hv[u][2];
        const v4f a = v4f{h0.x, h0.w, h1.z, h2.y}, b = v4f{h0.y, h1.x, h1.w, h2.z}, cc = v4f{h0.z, h1.y, h2.x, h2.w};
        v4f y;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            float z = a[e] * w[u][e][0];
            z = fmaf(b[e], w[u][e][1], z);
            z = fmaf(cc[e], w[u][e][2], z);
            z = fmaf(xv[u][e], w[u][e][3], z);
            y[e] = fast_silu(z);
        }
        *reinterpret_cast<v4f *>(s_y + at[u]) = y;
    }
    // Count this wave among the readers of its q/k history as soon as its reads are back (the
    // conv above consumed them, and the count is not moved above those stores); its return
    // is needed only at the end.  Every wave of the group counts, whatever the verdict, so
    // the last one can always set the count back to zero.
    asm volatile("" ::: "memory");
    int last = 0;
    if (lane == 0) last = atomicAdd(&sync[(c * d.Hk + kh) * GDN_SYNC_STRIDE], 1) == (d.Hv / d.Hk) * NB - 1;
    lds_barrier();
    float qq[RPL], kq[RPL];
#pragma unroll
    for (int e = 0; e < RPL; ++e) {
        qq[e] = s_y[i0 + e];
        kq[e] = s_y[DK + i0 + e];
    }
    const v4f v = *reinterpret_cast<const v4f *>(s_y + 2 * DK + 4 * q);

    const int bits = slot_preflight<64>(lanes, slot_ids, d.C, d.P, s_bitmap, &s_word);
    if (bits || st_in || s < 0) {  // rejected step, or a padding lane (uniform over the wave)
        if (bits && blockIdx.x == 0 && blockIdx.y == 0 && lane == 0) atomicOr(status, bits);
        if (__builtin_amdgcn_readfirstlane(last) && lane == 0) atomicExch(&sync[(c * d.Hk + kh) * GDN_SYNC_STRIDE], 0);
        return;
    }

    // the new history [column 1, column 2, token] of item u's channels
    auto write_hist = [&](int u) {
        const v4f h0 = hv[u][0], h1 = hv[u][1], h2 = hv[u][2];
        const v4f b = v4f{h0.y, h1.x, h1.w, h2.z}, cc = v4f{h0.z, h1.y, h2.x, h2.w}, xt = xv[u];
        v4f *hp = reinterpret_cast<v4f *>(conv_hist + ((int64_t)s * d.Ch + ch[u]) * 3);
        hp[0] = v4f{b.x, cc.x, xt.x, b.y};
        hp[1] = v4f{cc.y, xt.y, b.z, cc.z};
        hp[2] = v4f{xt.z, b.w, cc.w, xt.w};
    };
#pragma unroll
    for (int u = 0; u < NI; ++u) {
        const int f = lane + 64 * u;
        if (f >= GQK && f < GQK + GV) write_hist(u);  // this wave's value channels
    }
    decode_block<DK, DV>(qq, kq, v, braw, araw, Ah, sv, S4, i0, r, reinterpret_cast<v4f *>(out + ((int64_t)c * d.Hv + h) * DV + j0) + q);
    if (__builtin_amdgcn_readfirstlane(last)) {  // the last reader of the q/k history
#pragma unroll
        for (int u = 0; u < NI; ++u)
            if (lane + 64 * u < GQK) write_hist(u);
        if (lane == 0) atomicExch(&sync[(c * d.Hk + kh) * GDN_SYNC_STRIDE], 0);
    }
}

// ---- fused plain step, one workgroup per (lane, q/k head): its 8 waves share one conv of
//      the group's channels (the q/k slab once, the value channels of every block of the
//      group), so after the workgroup's barrier every reader of the history is done and each
//      conv thread writes its channels' new history itself; wave w then runs the recurrence
//      of blocks w, w + 8, ... (value head, column block) of the group.  For groups of at most
//      kGroupBlocks blocks; larger ones take conv_decode_kernel.
constexpr int kGroupWaves = 8, kGroupBlocks = 16;
template <int DK, int DV>
__global__ __launch_bounds__(64 * kGroupWaves) void conv_decode_group_kernel(
    Dims d, const float *__restrict__ x, const float *__restrict__ conv_w, float *__restrict__ conv_hist,
    const float *__restrict__ beta_logits, const float *__restrict__ alpha_logits, int64_t gate_stride,
    const float *__restrict__ dt_bias, const float *__restrict__ A, float *__restrict__ state_pool,
    const int32_t *__restrict__ slot_ids, float *__restrict__ out, int32_t *__restrict__ status) {
    using Cfg = DecodeCfg<DK, DV>;
    constexpr int JB = Cfg::JB, NB = Cfg::NB, Q4 = Cfg::Q4, RPL = Cfg::RPL, kT = 64 * kGroupWaves;
    constexpr int GQK = DK / 2, GVB = JB / 4;  // 4-channel groups: the q/k slab, one value block
    static_assert(GQK + kGroupBlocks * GVB <= kT, "one channel group per thread");
    __shared__ unsigned int s_bitmap[kBitmapSlots / 32];
    __shared__ int s_word;
    __shared__ __align__(16) float s_y[2 * DK + kGroupBlocks * JB];  // q rows, k rows, value columns

    const int c = blockIdx.y, kh = blockIdx.x;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int nblk = (d.Hv / d.Hk) * NB;  // (value head, column block) pairs of the group
    const int q = lane % Q4, r = lane / Q4, i0 = r * RPL;
    const int s_v = __builtin_bit_cast(
        int, __builtin_amdgcn_raw_buffer_load_b32(
                 __builtin_amdgcn_make_buffer_rsrc(const_cast<int32_t *>(slot_ids), 0, 4 * d.C, 0x00020000), 4 * c, 0,
                 0));
    const LaneSlotsT<kT> lanes(slot_ids, d.C);
    const int st_in = *status;
    // this thread's channel group: tid < GQK the q/k slab, then GVB groups per block
    const int nitems = GQK + nblk * GVB;
    const int f = min(tid, nitems - 1);
    const int vb = (f - GQK) / GVB, vg = f - GQK - vb * GVB;
    const int ch = f < DK / 4 ? kh * DK + 4 * f
                   : f < GQK  ? d.Hk * DK + kh * DK + 4 * (f - DK / 4)
                              : 2 * d.Hk * DK + (kh + d.Hk * (vb / NB)) * DV + (vb % NB) * JB + 4 * vg;
    const int at = f < GQK ? 4 * f : 2 * DK + vb * JB + 4 * vg;
    v4f w[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) w[e] = reinterpret_cast<const v4f *>(conv_w)[ch + e];
    const v4f xv = *reinterpret_cast<const v4f *>(x + (int64_t)c * d.Ch + ch);
    // this wave's first block: its gates
    const int blk0 = min(wave, nblk - 1), h0 = kh + d.Hk * (blk0 / NB);
    float braw = beta_logits[(int64_t)c * gate_stride + h0];
    float araw = alpha_logits[(int64_t)c * gate_stride + h0] + dt_bias[h0];
    float Ah = A[h0];
    __builtin_amdgcn_sched_barrier(0);
    const int s = __builtin_amdgcn_readfirstlane(s_v);
    const bool s_ok = s >= 0 && s < d.P;
    v4f hv[3];
#pragma unroll
    for (int k = 0; k < 3; ++k)
        hv[k] = reinterpret_cast<const v4f *>(conv_hist + ((int64_t)(s_ok ? s : 0) * d.Ch + ch) * 3)[k];
    auto state_rows = [&](int blk) {
        return reinterpret_cast<v4f *>(state_pool + ((int64_t)(s_ok ? s : 0) * d.Hv + kh + d.Hk * (blk / NB)) * DK * DV +
                                       (blk % NB) * JB) + q;
    };
    v4f sv[RPL];
    {
        v4f *S4 = state_rows(blk0);
#pragma unroll
        for (int e = 0; e < RPL; ++e) sv[e] = __builtin_nontemporal_load(S4 + (i0 + e) * (DV / 4));
    }
    // conv + SiLU of this thread's channel group (the conv step's order of taps and accumulation)
    const v4f ha = v4f{hv[0].x, hv[0].w, hv[1].z, hv[2].y}, hb = v4f{hv[0].y, hv[1].x, hv[1].w, hv[2].z},
              hc = v4f{hv[0].z, hv[1].y, hv[2].x, hv[2].w};
    if (tid < nitems) {
        v4f y;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            float z = ha[e] * w[e][0];
            z = fmaf(hb[e], w[e][1], z);
            z = fmaf(hc[e], w[e][2], z);
            z = fmaf(xv[e], w[e][3], z);
            y[e] = fast_silu(z);
        }
        *reinterpret_cast<v4f *>(s_y + at) = y;
    }
    // (the preflight's barriers also order the conv's LDS stores before the reads below, and
    // every history read of the workgroup before the history writes)
    const int bits = slot_preflight<kT>(lanes, slot_ids, d.C, d.P, s_bitmap, &s_word);
    if (bits || st_in) {
        if (bits && blockIdx.x == 0 && blockIdx.y == 0 && tid == 0) atomicOr(status, bits);
        return;
    }
    if (s < 0) return;  // padding lane (uniform over the workgroup)
    if (tid < nitems) {  // the new history [column 1, column 2, token] of this thread's channels
        v4f *hp = reinterpret_cast<v4f *>(conv_hist + ((int64_t)s * d.Ch + ch) * 3);
        hp[0] = v4f{hb.x, hc.x, xv.x, hb.y};
        hp[1] = v4f{hc.y, xv.y, hb.z, hc.z};
        hp[2] = v4f{xv.z, hb.w, hc.w, xv.w};
    }
    float qq[RPL], kq[RPL];
#pragma unroll
    for (int e = 0; e < RPL; ++e) {
        qq[e] = s_y[i0 + e];
        kq[e] = s_y[DK + i0 + e];
    }
    for (int blk = wave; blk < nblk; blk += kGroupWaves) {
        const int h = kh + d.Hk * (blk / NB), j0 = (blk % NB) * JB;
        v4f *S4 = state_rows(blk);
        if (blk != blk0) {  // a second block of this wave (groups of more than 8 blocks)
            braw = beta_logits[(int64_t)c * gate_stride + h];
            araw = alpha_logits[(int64_t)c * gate_stride + h] + dt_bias[h];
            Ah = A[h];
#pragma unroll
            for (int e = 0; e < RPL; ++e) sv[e] = __builtin_nontemporal_load(S4 + (i0 + e) * (DV / 4));
        }
        const v4f v = *reinterpret_cast<const v4f *>(s_y + 2 * DK + blk * JB + 4 * q);
        decode_block<DK, DV>(qq, kq, v, braw, araw, Ah, sv, S4, i0, r,
                             reinterpret_cast<v4f *>(out + ((int64_t)c * d.Hv + h) * DV + j0) + q);
    }
}

template <int DK, int DV>
hipError_t launch_conv_decode(const Dims &d, const float *x, const float *conv_w, float *conv_hist,
                              const float *beta_logits, const float *alpha_logits, int64_t gate_stride,
                              const float *dt_bias, const float *A, float *state_pool, const int32_t *slot_ids,
                              int32_t *sync, float *out, int32_t *status, hipStream_t stream) {
    if ((d.Hv / d.Hk) * DecodeCfg<DK, DV>::NB <= kGroupBlocks)
        hipLaunchKernelGGL((conv_decode_group_kernel<DK, DV>), dim3(d.Hk, d.C), dim3(64 * kGroupWaves), 0, stream, d,
                           x, conv_w, conv_hist, beta_logits, alpha_logits, gate_stride, dt_bias, A, state_pool,
                           slot_ids, out, status);
    else
        hipLaunchKernelGGL((conv_decode_kernel<DK, DV>), dim3(DecodeCfg<DK, DV>::NB * d.Hv, d.C), dim3(64), 0, stream,
                           d, x, conv_w, conv_hist, beta_logits, alpha_logits, gate_stride, dt_bias, A, state_pool,
                           slot_ids, sync, out, status);
    return hipGetLastError();
}

template <int DK, int DV>
hipError_t launch_decode(const Dims &d, const float *qkv, const float *beta_logits, const float *alpha_logits,
                         int64_t gate_stride, const float *dt_bias, const float *A, float *state_pool,
                         const int32_t *slot_ids, float *out, int32_t *status, hipStream_t stream) {
    hipLaunchKernelGGL((decode_step_kernel<DK, DV>), dim3(DecodeCfg<DK, DV>::NB * d.Hv, d.C), dim3(64), 0,
                       stream, d, qkv, beta_logits, alpha_logits, gate_stride, dt_bias, A, state_pool, slot_ids, out,
                       status);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_conv_step(const Dims &d, const float *x, const float *conv_w, float *conv_hist,
                            const int32_t *slot_ids, float *conv_out, int32_t *status, hipStream_t stream) {
    const int groups = d.Ch / 4;
    const dim3 grid((groups + kThreads - 1) / kThreads, d.C, (d.N + kTokRun - 1) / kTokRun);
    hipLaunchKernelGGL(conv_step_kernel, grid, dim3(kThreads), 0, stream, d, x, conv_w, conv_hist, slot_ids, conv_out,
                       status);
    return hipGetLastError();
}

hipError_t launch_decode_step(const Dims &d, const float *qkv, const float *beta_logits, const float *alpha_logits,
                              int64_t gate_stride, const float *dt_bias, const float *A, float *state_pool,
                              const int32_t *slot_ids, float *out, int32_t *status, hipStream_t stream) {
#define GDN_DECODE_CASE(K, V)                                                                                      \
    if (d.dk == K && d.dv == V)                                                                                    \
        return launch_decode<K, V>(d, qkv, beta_logits, alpha_logits, gate_stride, dt_bias, A, state_pool, slot_ids, \
                                   out, status, stream);
#define GDN_DECODE_ROW(K) GDN_DECODE_CASE(K, 16) GDN_DECODE_CASE(K, 32) GDN_DECODE_CASE(K, 64) GDN_DECODE_CASE(K, 128)
    GDN_DECODE_ROW(16) GDN_DECODE_ROW(32) GDN_DECODE_ROW(64) GDN_DECODE_ROW(128)
#undef GDN_DECODE_ROW
#undef GDN_DECODE_CASE
    return hipErrorInvalidValue;
}

hipError_t launch_conv_decode_step(const Dims &d, const float *x, const float *conv_w, float *conv_hist,
                                   const float *beta_logits, const float *alpha_logits, int64_t gate_stride,
                                   const float *dt_bias, const float *A, float *state_pool, const int32_t *slot_ids,
                                   int32_t *sync, float *out, int32_t *status, hipStream_t stream) {
#define GDN_FUSED_CASE(K, V)                                                                                       \
    if (d.dk == K && d.dv == V)                                                                                    \
        return launch_conv_decode<K, V>(d, x, conv_w, conv_hist, beta_logits, alpha_logits, gate_stride, dt_bias, A, \
                                        state_pool, slot_ids, sync, out, status, stream);
#define GDN_FUSED_ROW(K) GDN_FUSED_CASE(K, 16) GDN_FUSED_CASE(K, 32) GDN_FUSED_CASE(K, 64) GDN_FUSED_CASE(K, 128)
    GDN_FUSED_ROW(16) GDN_FUSED_ROW(32) GDN_FUSED_ROW(64) GDN_FUSED_ROW(128)
#undef GDN_FUSED_ROW
#undef GDN_FUSED_CASE
    return hipErrorInvalidValue;
}

}  // namespace gdn
