// Plain decode step for gfx950: the step of a lane without a draft, which commits its
// post-step state to the slot at once instead of going through a verify and a commit.
// Two launches on the caller's stream:
//   conv_step_kernel    causal conv + SiLU over a chain of tokens per lane, writing the
//                       slot's new history (the last 3 columns) back in place;
//   decode_step_kernel  one token of the gated delta rule applied to the slot's state
//                       in place, with the output row.
// The conv must finish before the recurrence reads its output: a q/k channel feeds
// every value head of its group, so one launch could not write the history in place
// while other workgroups still read it.
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
constexpr int kBitmapSlots = 65536;  // duplicate-slot check via an LDS bitmap up to this pool size
constexpr int kTokChunk = 8;         // conv step: tokens loaded together
constexpr int kLanesPerThread = (GDN_MAX_SEQS + kThreads - 1) / kThreads;

// The slot ids of lanes tid, tid + kThreads, ... (for slot_preflight), loaded ahead of
// the bulk loads so the preflight does not wait for them.
struct LaneSlots {
    int v[kLanesPerThread];
    __device__ LaneSlots(const int32_t *__restrict__ slot_ids, int C) {
#pragma unroll
        for (int k = 0; k < kLanesPerThread; ++k) v[k] = slot_ids[min((int)threadIdx.x + kThreads * k, C - 1)];
    }
};

// Slot preflight of a call that mutates the pools: GDN_STATUS_SLOT_RANGE /
// GDN_STATUS_SLOT_DUP over every non-padding lane.  Every thread of the workgroup must
// call it (it contains barriers); all threads receive the same bits.
__device__ int slot_preflight(const LaneSlots &ls, const int32_t *__restrict__ slot_ids, const Dims &d,
                              unsigned int *bitmap, int *word) {
    const bool use_bitmap = d.P <= kBitmapSlots;
    if (use_bitmap)
        for (int w = threadIdx.x; w < (d.P + 31) / 32; w += kThreads) bitmap[w] = 0u;
    if (threadIdx.x == 0) *word = 0;
    lds_barrier();
    int bits = 0;
#pragma unroll
    for (int k = 0; k < kLanesPerThread; ++k) {
        const int t = threadIdx.x + kThreads * k;
        const int st = ls.v[k];
        if (t >= d.C || st == -1) continue;
        if (st < -1 || st >= d.P) {
            bits |= GDN_STATUS_SLOT_RANGE;
        } else if (use_bitmap) {
            const unsigned int m = 1u << (st & 31);
            if (atomicOr(&bitmap[st >> 5], m) & m) bits |= GDN_STATUS_SLOT_DUP;
        } else {
            for (int o = 0; o < d.C; ++o)
                if (o != t && slot_ids[o] == st) bits |= GDN_STATUS_SLOT_DUP;
        }
    }
    if (bits) atomicOr(word, bits);
    lds_barrier();
    return *word;
}

// Sum over the lanes of a wave that share lane % Q (Q = 4 or 8): rotations within each
// row of 16 lanes, then the row pairs and wave halves exchanged by permlane swaps (with
// both operands equal, the two results of a swap add up to the pairwise sum).
template <int M>
__device__ inline float row_ror(float x) {  // lane (i - M) mod 16 of each row of 16 lanes (DPP row_ror)
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x120 + M, 0xF, 0xF, false));
}

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

// ---- conv step: thread = (lane c = blockIdx.y, 4-channel group g); the window slides
//      over the chain in registers, oldest column first (tap 0 multiplies it).
__global__ __launch_bounds__(kThreads) void conv_step_kernel(Dims d, const float *__restrict__ x,
                                                             const float *__restrict__ conv_w,
                                                             float *__restrict__ conv_hist,
                                                             const int32_t *__restrict__ slot_ids,
                                                             float *__restrict__ conv_out, int32_t *__restrict__ status) {
    __shared__ unsigned int s_bitmap[kBitmapSlots / 32];
    __shared__ int s_word;
    const int c = blockIdx.y, G4 = d.Ch / 4;
    const int g = blockIdx.x * kThreads + threadIdx.x, gc = g < G4 ? g : G4 - 1;
    const LaneSlots lanes(slot_ids, d.C);
    const int s = slot_ids[c];
    const int st_in = *status;
    const bool s_ok = s >= 0 && s < d.P;
    // loads first: taps, the slot's history (slot clamped into range), the first tokens
    v4f w[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) w[e] = reinterpret_cast<const v4f *>(conv_w)[4 * gc + e];
    v4f *hp = reinterpret_cast<v4f *>(conv_hist + ((int64_t)(s_ok ? s : 0) * d.Ch + 4 * gc) * 3);
    const v4f h0 = hp[0], h1 = hp[1], h2 = hp[2];
    const v4f *xr = reinterpret_cast<const v4f *>(x + (int64_t)c * d.N * d.Ch) + gc;
    v4f xt[kTokChunk];
#pragma unroll
    for (int t = 0; t < kTokChunk; ++t) xt[t] = xr[(int64_t)min(t, d.N - 1) * G4];

    const int bits = slot_preflight(lanes, slot_ids, d, s_bitmap, &s_word);
    if (bits || st_in) {
        if (bits && blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x == 0) atomicOr(status, bits);
        return;
    }
    if (s < 0 || g >= G4) return;  // padding lane, or past the channels

    // history columns of the 4 channels (layout [ch][3]: 12 consecutive floats)
    v4f a = {h0.x, h0.w, h1.z, h2.y}, b = {h0.y, h1.x, h1.w, h2.z}, cc = {h0.z, h1.y, h2.x, h2.w};
    v4f *orow = reinterpret_cast<v4f *>(conv_out + (int64_t)c * d.N * d.Ch) + g;
    for (int t0 = 0; t0 < d.N; t0 += kTokChunk) {
        if (t0 > 0) {
#pragma unroll
            for (int t = 0; t < kTokChunk; ++t) xt[t] = xr[(int64_t)min(t0 + t, d.N - 1) * G4];
        }
#pragma unroll
        for (int t = 0; t < kTokChunk; ++t) {
            if (t0 + t >= d.N) break;
            v4f y;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                float z = a[e] * w[e][0];
                z = fmaf(b[e], w[e][1], z);
                z = fmaf(cc[e], w[e][2], z);
                z = fmaf(xt[t][e], w[e][3], z);
                y[e] = z / (1.0f + expf(-z));
            }
            orow[(int64_t)(t0 + t) * G4] = y;
            a = b;
            b = cc;
            cc = xt[t];
        }
    }
    // the slot's new history: the last 3 columns, in place (only this thread reads or
    // writes these 12 floats)
    hp[0] = v4f{a.x, b.x, cc.x, a.y};
    hp[1] = v4f{b.y, cc.y, a.z, b.z};
    hp[2] = v4f{cc.z, a.w, b.w, cc.w};
}

// ---- decode step: workgroup = (lane c = blockIdx.y, value head h, block of JB value
//      columns); thread (r, q) = (tid / Q4, tid % Q4) holds the 4 columns q of the rows
//      r, r + RG, ... of the block, so one load instruction covers whole rows.
template <int DK, int DV>
struct DecodeCfg {
    static constexpr int JB = DV < 32 ? DV : 32;  // value columns per workgroup
    static constexpr int NB = DV / JB;
    static constexpr int Q4 = JB / 4;             // 4-column groups
    static constexpr int RG = kThreads / Q4;      // row groups
    static constexpr int RPT = (DK + RG - 1) / RG;  // rows per thread
};

template <int DK, int DV>
__global__ __launch_bounds__(kThreads) void decode_step_kernel(
    Dims d, const float *__restrict__ qkv, const float *__restrict__ beta_logits,
    const float *__restrict__ alpha_logits, int64_t gate_stride, const float *__restrict__ dt_bias,
    const float *__restrict__ A, float *__restrict__ state_pool, const int32_t *__restrict__ slot_ids,
    float *__restrict__ out, int32_t *__restrict__ status) {
    using Cfg = DecodeCfg<DK, DV>;
    constexpr int JB = Cfg::JB, NB = Cfg::NB, Q4 = Cfg::Q4, RG = Cfg::RG, RPT = Cfg::RPT;
    static_assert(DK / 4 <= 64, "q and k rows staged by one wave each");
    __shared__ unsigned int s_bitmap[kBitmapSlots / 32];
    __shared__ int s_word;
    __shared__ float s_q[DK], s_k[DK], s_dot[3];
    __shared__ v4f s_part[kThreads / 64][2][Q4];

    const int c = blockIdx.y, h = blockIdx.x / NB, jb = blockIdx.x - h * NB, j0 = jb * JB;
    const int kh = h % d.Hk;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int q = tid % Q4, r = tid / Q4;
    // loads in the order they are needed, all issued before any is consumed: this lane's
    // slot id (a vector load, so that its wait does not hold up the loads behind it),
    // the preflight's slot ids, q / k rows, value columns and gates, then the state block
    const int s_v = __builtin_bit_cast(
        int, __builtin_amdgcn_raw_buffer_load_b32(
                 __builtin_amdgcn_make_buffer_rsrc(const_cast<int32_t *>(slot_ids), 0, 4 * d.C, 0x00020000), 4 * c, 0,
                 0));
    const LaneSlots lanes(slot_ids, d.C);
    const int st_in = *status;
    const float *row = qkv + (int64_t)c * d.Ch;
    v4f qk4 = {0.f, 0.f, 0.f, 0.f};
    if (wave < 2 && lane < DK / 4)  // wave 0: q row, wave 1: k row of q/k head kh
        qk4 = reinterpret_cast<const v4f *>(row + wave * d.Hk * DK + kh * DK)[lane];
    const v4f v = reinterpret_cast<const v4f *>(row + 2 * d.Hk * DK + h * DV + j0)[q];
    const float braw = beta_logits[(int64_t)c * gate_stride + h];
    const float araw = alpha_logits[(int64_t)c * gate_stride + h] + dt_bias[h];
    const float Ah = A[h];
    __builtin_amdgcn_sched_barrier(0);
    const int s = __builtin_amdgcn_readfirstlane(s_v);
    const bool s_ok = s >= 0 && s < d.P;
    v4f *S4 = reinterpret_cast<v4f *>(state_pool + ((int64_t)(s_ok ? s : 0) * d.Hv + h) * DK * DV + j0) + q;
    v4f sv[RPT];  // the state block (slot clamped into range; written back only if the step commits)
#pragma unroll
    for (int k = 0; k < RPT; ++k) sv[k] = S4[min(r + RG * k, DK - 1) * (DV / 4)];

    if (wave < 2 && lane < DK / 4) reinterpret_cast<v4f *>(wave == 0 ? s_q : s_k)[lane] = qk4;
    const int bits = slot_preflight(lanes, slot_ids, d, s_bitmap, &s_word);  // its barriers also publish s_q / s_k
    if (bits || st_in) {
        if (bits && blockIdx.x == 0 && blockIdx.y == 0 && tid == 0) atomicOr(status, bits);
        return;
    }
    if (s < 0) return;  // padding lane (uniform over the workgroup)

    // |q|^2, |k|^2 and q . k, one wave each
    if (wave < 3) {
        const float *u = wave == 1 ? s_k : s_q;
        const float *w = wave == 0 ? s_q : s_k;
        float acc = 0.f;
        for (int e = lane; e < DK; e += 64) acc = fmaf(u[e], w[e], acc);
#pragma unroll
        for (int m = 32; m >= 1; m >>= 1) acc += __shfl_xor(acc, m);
        if (lane == 0) s_dot[wave] = acc;
    }
    lds_barrier();
    const float rq = inv_norm(s_dot[0]), rk = inv_norm(s_dot[1]);
    const float qk = s_dot[2] * rq * rk;  // q^ . k^

    // column sums of k^_i S[i][j] and q^_i S[i][j] over this thread's rows, then over the
    // row groups: lanes of a wave that share q, then the waves through LDS
    v4f pu = {0.f, 0.f, 0.f, 0.f}, pw = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int k = 0; k < RPT; ++k) {
        const int i = r + RG * k;
        if (RG * RPT == DK || i < DK) {
            pu += (s_k[i] * rk) * sv[k];
            pw += (s_q[i] * rq) * sv[k];
        }
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        pu[e] = sum_lanes_sharing<Q4>(pu[e]);
        pw[e] = sum_lanes_sharing<Q4>(pw[e]);
    }
    if (lane < Q4) {
        s_part[wave][0][q] = pu;
        s_part[wave][1][q] = pw;
    }
    lds_barrier();
    v4f U = s_part[0][0][q], W = s_part[0][1][q];
#pragma unroll
    for (int w = 1; w < kThreads / 64; ++w) {
        U += s_part[w][0][q];
        W += s_part[w][1][q];
    }
    // S' = g S;  delta = beta (v - S'^T k^);  S_new = S' + k^ delta^T;
    // o = S_new^T q^ / sqrt(d_k) = (g S^T q^ + (q^ . k^) delta) / sqrt(d_k)
    const float g = fast_exp(fast_softplus(araw) * Ah), beta = fast_sigmoid(braw);
    const v4f delta = beta * (v - g * U);
#pragma unroll
    for (int k = 0; k < RPT; ++k) {
        const int i = r + RG * k;
        if (RG * RPT == DK || i < DK) __builtin_nontemporal_store(g * sv[k] + (s_k[i] * rk) * delta, S4 + i * (DV / 4));
    }
    if (r == 0)
        reinterpret_cast<v4f *>(out + ((int64_t)c * d.Hv + h) * DV + j0)[q] =
            (g * W + qk * delta) * (1.0f / sqrtf((float)DK));
}

template <int DK, int DV>
hipError_t launch_decode(const Dims &d, const float *qkv, const float *beta_logits, const float *alpha_logits,
                         int64_t gate_stride, const float *dt_bias, const float *A, float *state_pool,
                         const int32_t *slot_ids, float *out, int32_t *status, hipStream_t stream) {
    hipLaunchKernelGGL((decode_step_kernel<DK, DV>), dim3(DecodeCfg<DK, DV>::NB * d.Hv, d.C), dim3(kThreads), 0,
                       stream, d, qkv, beta_logits, alpha_logits, gate_stride, dt_bias, A, state_pool, slot_ids, out,
                       status);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_conv_step(const Dims &d, const float *x, const float *conv_w, float *conv_hist,
                            const int32_t *slot_ids, float *conv_out, int32_t *status, hipStream_t stream) {
    const int groups = d.Ch / 4;
    hipLaunchKernelGGL(conv_step_kernel, dim3((groups + kThreads - 1) / kThreads, d.C), dim3(kThreads), 0, stream, d,
                       x, conv_w, conv_hist, slot_ids, conv_out, status);
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

}  // namespace gdn
