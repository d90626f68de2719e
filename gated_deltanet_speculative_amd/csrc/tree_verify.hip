// Read-only slot-mapped tree verify for gfx950: the gated delta rule over each lane's
// draft tree with the gates applied in-kernel, writing the attention output and the
// replay log and never the state.
//
// What is computed: "perf(qwen35): fuse the DFlash2 concurrent verify Gated DeltaNet
// route", Optimizations, second and third bullets; gates from "qwen35: DSpark
// speculative decoding", raw-gate commit message; log row width 1 + d_k + d_v from
// "perf(qwen38): various DFlash2 optimizations concurrency C1-C5", Summary item 3.
//
// Design.  The recurrence is separable in value columns, and unrolling it along a
// node's root path gives, with G_i the product of decays on the path of i,
//   S_i = G_i S0 + sum_{a on path(i)} (G_i/G_a) k^_a delta_a^T,
// so per value column j:
//   u_i[j]   = G_i (k^_i . S0[:,j]) + sum_{a strict ancestor} (G_i/G_a)(k^_a.k^_i) delta_a[j]
//   delta_i  = beta_i (v_i - u_i)
//   o_i[j]   = (G_i (q^_i . S0[:,j]) + sum_{a on path(i)} (G_i/G_a)(k^_a.q^_i) delta_a[j]) / sqrt(d_k)
// The only O(d_k d_v) work is the dense product [K^;Q^] S0 (2N rows); per-node states
// are never formed, the slot's state is read exactly once per value column and the
// tree enters only through N x N ancestor-masked coefficient matrices.  Decay ratios
// are exp(L_i - L_a) of cumulative log-decays, which cannot overflow.
//
// One workgroup per (lane, value head, block of 32 value columns).
#include "gdn_internal.h"

namespace gdn {
namespace {

constexpr int kThreads = 256;

template <int DK, int DV>
struct VerifyCfg {
    static constexpr int JB = DV < 32 ? DV : 32;  // value columns per workgroup
    static constexpr int NB = DV / JB;            // column blocks per head
    static size_t lds_bytes(int N) {
        return sizeof(float) * (size_t)(2 * N * DK + DK * JB + 3 * N * JB + 2 * N * N);
    }
};

__device__ inline float wave_sum(float v) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off);
    return v;
}

template <int DK, int DV>
__global__ __launch_bounds__(kThreads) void tree_verify_kernel(
    Dims d, const float *__restrict__ qkv, const float *__restrict__ beta_logits,
    const float *__restrict__ alpha_logits, int64_t gate_stride, const float *__restrict__ dt_bias,
    const float *__restrict__ A, const float *__restrict__ state_pool, const int32_t *__restrict__ slot_ids,
    const int32_t *__restrict__ parents, float *__restrict__ out, float *__restrict__ replay_log,
    int32_t *__restrict__ status) {
    using Cfg = VerifyCfg<DK, DV>;
    constexpr int JB = Cfg::JB;
    constexpr int R = 1 + DK + DV;
    extern __shared__ float lds[];
    __shared__ int s_bits;
    __shared__ int s_par[GDN_MAX_NODES];
    __shared__ float s_beta[GDN_MAX_NODES], s_lg[GDN_MAX_NODES], s_L[GDN_MAX_NODES];
    __shared__ unsigned long long s_anc[GDN_MAX_NODES];

    const int jb = blockIdx.x, h = blockIdx.y, c = blockIdx.z;
    const int s = slot_ids[c];
    if (s == -1) return;  // padding lane
    const int bits = lane_status_bits(slot_ids, parents, d, c, s, &s_bits);
    if (bits) {
        if (jb == 0 && h == 0 && threadIdx.x == 0 && status) atomicOr(status, bits);
        return;
    }

    const int N = d.N, Ch = d.Ch, Hv = d.Hv, tid = threadIdx.x;
    const int kh = h % d.Hk;
    const int j0 = jb * JB;
    float *qh = lds;            // [N][DK] normalised queries
    float *kk = qh + N * DK;    // [N][DK] normalised keys
    float *S0 = kk + N * DK;    // [DK][JB] state columns j0 .. j0+JB
    float *PK = S0 + DK * JB;   // [N][JB] k^_i . S0[:,j]
    float *PQ = PK + N * JB;    // [N][JB] q^_i . S0[:,j]
    float *Vd = PQ + N * JB;    // [N][JB] v, overwritten in place by delta
    float *Ck = Vd + N * JB;    // [N][N]  Ck[a*N+i] = (G_i/G_a) k^_a.k^_i, a strict ancestor of i
    float *Cq = Ck + N * N;     // [N][N]  Cq[a*N+i] = (G_i/G_a) k^_a.q^_i, a on path(i)

    // ---- gates and tree bookkeeping
    if (tid < N) {
        const int64_t row = (int64_t)c * N + tid;
        s_par[tid] = parents[row];
        const float b = beta_logits[row * gate_stride + h];
        const float a = alpha_logits[row * gate_stride + h] + dt_bias[h];
        s_beta[tid] = 1.0f / (1.0f + expf(-b));
        s_lg[tid] = (fmaxf(a, 0.0f) + log1pf(expf(-fabsf(a)))) * A[h];  // log g = softplus(a + dt_bias) * A
    }
    __syncthreads();
    if (tid < N) {
        float L = 0.0f;
        unsigned long long m = 0ull;
        for (int a = tid; a >= 0; a = s_par[a]) {
            L += s_lg[a];
            m |= 1ull << a;
        }
        s_L[tid] = L;
        s_anc[tid] = m;
    }

    // ---- q/k L2 normalisation (one wave per vector), replay-log g and k^ (column block 0)
    const int wave = tid >> 6, lane = tid & 63;
    float *logc = replay_log + ((int64_t)c * N * Hv + h) * R;  // row (c, i, h) at logc + i*Hv*R
    for (int vec = wave; vec < 2 * N; vec += kThreads / 64) {
        const int i = vec >> 1;
        const bool is_k = vec & 1;
        const float *src = qkv + ((int64_t)c * N + i) * Ch + (is_k ? d.Hk * DK : 0) + kh * DK;
        float v0 = lane < DK ? src[lane] : 0.0f;
        float v1 = lane + 64 < DK ? src[lane + 64] : 0.0f;
        const float inv = 1.0f / fmaxf(sqrtf(wave_sum(v0 * v0 + v1 * v1)), 1e-6f);
        v0 *= inv;
        v1 *= inv;
        float *dst = (is_k ? kk : qh) + i * DK;
        if (lane < DK) dst[lane] = v0;
        if (lane + 64 < DK) dst[lane + 64] = v1;
        if (is_k && jb == 0) {
            float *lrow = logc + (int64_t)i * Hv * R;
            if (lane < DK) lrow[1 + lane] = v0;
            if (lane + 64 < DK) lrow[1 + lane + 64] = v1;
            if (lane == 0) lrow[0] = expf(s_lg[i]);
        }
    }
    // ---- state columns and values
    const float *Sg = state_pool + (((int64_t)s * Hv + h) * DK) * DV + j0;
    for (int idx = tid; idx < DK * JB / 4; idx += kThreads) {
        const int r = idx / (JB / 4), q = idx - r * (JB / 4);
        reinterpret_cast<float4 *>(S0)[idx] = reinterpret_cast<const float4 *>(Sg + (int64_t)r * DV)[q];
    }
    for (int idx = tid; idx < N * JB; idx += kThreads) {
        const int i = idx / JB, j = idx - i * JB;
        Vd[idx] = qkv[((int64_t)c * N + i) * Ch + 2 * d.Hk * DK + h * DV + j0 + j];
    }
    __syncthreads();

    // ---- ancestor-masked coefficient matrices
    for (int idx = tid; idx < N * N; idx += kThreads) {
        const int a = idx / N, i = idx - a * N;
        float ck = 0.0f, cq = 0.0f;
        if (a <= i && ((s_anc[i] >> a) & 1ull)) {
            const float r = expf(s_L[i] - s_L[a]);
            float dq = 0.0f, dk = 0.0f;
            for (int k = 0; k < DK; ++k) {
                dq = fmaf(kk[a * DK + k], qh[i * DK + k], dq);
                dk = fmaf(kk[a * DK + k], kk[i * DK + k], dk);
            }
            cq = r * dq;
            ck = a < i ? r * dk : 0.0f;
        }
        Ck[idx] = ck;
        Cq[idx] = cq;
    }
    // ---- [K^; Q^] S0 for this column block
    for (int idx = tid; idx < 2 * N * JB; idx += kThreads) {
        const int r = idx / JB, j = idx - r * JB;
        const float *vec = r < N ? kk + r * DK : qh + (r - N) * DK;
        float acc = 0.0f;
        for (int k = 0; k < DK; ++k) acc = fmaf(vec[k], S0[k * JB + j], acc);
        (r < N ? PK : PQ)[(r < N ? r : r - N) * JB + j] = acc;
    }
    __syncthreads();

    // ---- forward substitution over nodes (parents precede children), one thread per column
    if (tid < JB) {
        const int j = tid;
        for (int i = 0; i < N; ++i) {
            float u = expf(s_L[i]) * PK[i * JB + j];
            for (int a = 0; a < i; ++a) u = fmaf(Ck[a * N + i], Vd[a * JB + j], u);
            Vd[i * JB + j] = s_beta[i] * (Vd[i * JB + j] - u);
        }
    }
    __syncthreads();

    // ---- outputs and the delta part of the log rows
    const float scale = 1.0f / sqrtf((float)DK);
    for (int idx = tid; idx < N * JB; idx += kThreads) {
        const int i = idx / JB, j = idx - i * JB;
        float o = expf(s_L[i]) * PQ[idx];
        for (int a = 0; a <= i; ++a) o = fmaf(Cq[a * N + i], Vd[a * JB + j], o);
        out[(((int64_t)c * N + i) * Hv + h) * DV + j0 + j] = o * scale;
        logc[(int64_t)i * Hv * R + 1 + DK + j0 + j] = Vd[idx];
    }
}

template <int DK, int DV>
hipError_t launch(const Dims &d, const float *qkv, const float *bl, const float *al, int64_t gs, const float *dt,
                  const float *A, const float *pool, const int32_t *slots, const int32_t *parents, float *out,
                  float *log, int32_t *status, hipStream_t stream) {
    using Cfg = VerifyCfg<DK, DV>;
    const size_t lds = Cfg::lds_bytes(d.N);
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(&tree_verify_kernel<DK, DV>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((tree_verify_kernel<DK, DV>), dim3(Cfg::NB, d.Hv, d.C), dim3(kThreads), lds, stream, d, qkv,
                       bl, al, gs, dt, A, pool, slots, parents, out, log, status);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_tree_verify(const Dims &d, const float *qkv, const float *beta_logits, const float *alpha_logits,
                              int64_t gate_stride, const float *dt_bias, const float *A, const float *state_pool,
                              const int32_t *slot_ids, const int32_t *parents, float *out, float *replay_log,
                              int32_t *status, hipStream_t stream) {
#define GDN_VERIFY_CASE(K, V)                                                                                   \
    if (d.dk == K && d.dv == V)                                                                                 \
        return launch<K, V>(d, qkv, beta_logits, alpha_logits, gate_stride, dt_bias, A, state_pool, slot_ids, \
                            parents, out, replay_log, status, stream);
#define GDN_VERIFY_ROW(K) GDN_VERIFY_CASE(K, 16) GDN_VERIFY_CASE(K, 32) GDN_VERIFY_CASE(K, 64) GDN_VERIFY_CASE(K, 128)
    GDN_VERIFY_ROW(16) GDN_VERIFY_ROW(32) GDN_VERIFY_ROW(64) GDN_VERIFY_ROW(128)
#undef GDN_VERIFY_ROW
#undef GDN_VERIFY_CASE
    return hipErrorInvalidValue;
}

}  // namespace gdn
