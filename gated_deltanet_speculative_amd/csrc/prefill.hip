// Prefill for gfx950: the gated delta rule over a chain of T tokens per lane, starting from
// and replacing the slot's state in place, 16 tokens at a time, with an optional closing
// output gate.
//
// What is computed: "Feature/support dflash2", first-version commit message (prefill's
// recurrence on a chunked GDN kernel that closes with a SiLU or, by gate_mode, a sigmoid
// output gate); the per-token rule and the in-kernel gates as in the tree verify
// ("qwen35: DSpark speculative decoding (Qwen3.8-27B drafters)", raw-gate commit message).
//
// Chunked form.  Within a chunk of B = 16 tokens, with cumulative log-decays L_t from the
// chunk start (G_t = exp(L_t)), raw rows q_t, k_t, inverse norms rq_t, rk_t and the state
// S at the chunk start:
//   (I + Lm) D = rhs,  rhs_t = beta_t (v_t - G_t rk_t (K S)_t),
//   Lm[t][u] = beta_t exp(L_t - L_u) rk_t rk_u (k_t . k_u)                 (u < t)
//   O_t = G_t rq_t (Q S)_t / sqrt(d_k) + sum_{u <= t} Cq[t][u] D_u,
//   Cq[t][u] = exp(L_t - L_u) rq_t rk_u (q_t . k_u) / sqrt(d_k)            (u <= t)
//   S <- G_B S + sum_u exp(L_B - L_u) rk_u k_u D_u^T
// i.e. the tree verify's formulation on a chain, followed by the state update.  Every
// product with d_k or d_v in it runs on v_mfma_f32_16x16x4_f32 with the operand
// permutation of mfma4, so the state tile stays in registers across chunks in exactly the
// layout in which the next chunk's products and the update consume and produce it.
//
// Mapping: one workgroup (4 waves) per (lane, value head, block of 64 value columns);
// wave w owns the 16-column tile w of the state for the whole prompt.  Per chunk: stage
// the chunk's rows in LDS (padding tokens of the last chunk as zero rows), issue the next
// chunk's loads, then norms + gates, the Gram products (split over the waves by d_k
// chunk) and each wave's [K; Q] S; coefficients; T = (I + Lm)^-1 by broadcast forward
// substitution; D, O, the output gate and the state update per wave; outputs leave as
// 16-byte chunks of whole rows.  The state is read once before the first chunk and
// written once after the last.
#include "gdn_device.h"
#include "gdn_internal.h"

namespace gdn {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int BC = 16;  // tokens per chunk

template <int DK, int DV>
struct PrefillCfg {
    static constexpr int JB = DV < 64 ? DV : 64;      // value columns per workgroup
    static constexpr int NB = DV / JB;                // column blocks per head
    static constexpr int CT = JB / 16;                // 16-column tiles: wave w < CT owns tile w
    static constexpr int KC = DK / 16;                // 16-wide chunks of d_k
    static constexpr int SX = DK + 4;                 // raw q / k rows in LDS (4 mod 8 floats)
    static constexpr int SV = JB + 4;                 // value, gate and output rows
    static constexpr int SG = BC + 4;                 // 16 x 16 matrices
    static constexpr int QK4 = BC * DK / 4;           // float4 groups of a chunk's q (or k) rows
    static constexpr int QPT = (2 * QK4 + kThreads - 1) / kThreads;
    static constexpr int V4 = BC * JB / 4;            // float4 groups of a chunk's value block
    static_assert(V4 <= kThreads, "one value group per thread");
};

// element (i, a) of a 16 x 16 accumulator tile stored lane-major (lane * 4 + component)
__device__ inline int tile_index(int i, int a) { return (16 * (i >> 2) + a) * 4 + (i & 3); }

template <int DK, int DV>
__global__ __launch_bounds__(kThreads) void prefill_kernel(
    Dims d, int T, const float *__restrict__ qkv, const float *__restrict__ beta_logits,
    const float *__restrict__ alpha_logits, int64_t gate_stride, const float *__restrict__ dt_bias,
    const float *__restrict__ A, float *__restrict__ state_pool, const int32_t *__restrict__ slot_ids,
    const float *__restrict__ gate_z, int gate_mode, float *__restrict__ out, int32_t *__restrict__ status) {
    using Cfg = PrefillCfg<DK, DV>;
    constexpr int JB = Cfg::JB, NB = Cfg::NB, CT = Cfg::CT, KC = Cfg::KC, SX = Cfg::SX, SV = Cfg::SV;
    constexpr int SG = Cfg::SG, QK4 = Cfg::QK4, QPT = Cfg::QPT, V4 = Cfg::V4;
    __shared__ unsigned int s_bitmap[kBitmapSlots / 32];
    __shared__ int s_word;
    __shared__ __align__(16) float Ql[BC * SX], Kl[BC * SX], Vl[BC * SV], Zl[BC * SV], Ot[BC * SV];
    __shared__ __align__(16) float s_gram[kWaves][2][256];
    __shared__ __align__(16) float Lm[BC * SG], Cq[BC * SG], Tm[BC * SG];
    __shared__ float s_rk[BC], s_rq[BC], s_beta[BC], s_L[BC];

    const int c = blockIdx.y, h = blockIdx.x / NB, jb = blockIdx.x - h * NB, j0 = jb * JB;
    const int kh = h % d.Hk, Ch = d.Ch, Hv = d.Hv;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, g4 = lane >> 4, l16 = lane & 15;
    const bool gated = gate_z != nullptr;
    const float isd = 1.0f / sqrtf((float)DK);

    // ---- loads that do not need the slot first (the slot id through a vector load, so
    //      its wait does not hold up the loads behind it), then the state tile
    const int s_v = __builtin_bit_cast(
        int, __builtin_amdgcn_raw_buffer_load_b32(
                 __builtin_amdgcn_make_buffer_rsrc(const_cast<int32_t *>(slot_ids), 0, 4 * d.C, 0x00020000), 4 * c, 0,
                 0));
    const LaneSlotsT<kThreads> lanes(slot_ids, d.C);
    const int st_in = *status;
    const float dt = dt_bias[h], Ah = A[h];

    // one chunk's loads: item u of a thread is float4 group f = tid + kThreads * u of the
    // q rows (f < QK4) or k rows; the value / gate group tid (< V4); token tid's gates
    v4f xq[QPT], xv, xz;
    float xb, xa;
    auto load_chunk = [&](int k0) {
        const float *row0 = qkv + (int64_t)c * T * Ch;
#pragma unroll
        for (int u = 0; u < QPT; ++u) {
            const int f = min(tid + kThreads * u, 2 * QK4 - 1);
            const int m = f / QK4, r = f - m * QK4, t = r / (DK / 4), grp = r - t * (DK / 4);
            const int tok = min(k0 + t, T - 1);
            xq[u] = *reinterpret_cast<const v4f *>(row0 + (int64_t)tok * Ch + m * d.Hk * DK + kh * DK + 4 * grp);
        }
        const int tv = min(tid, V4 - 1) / (JB / 4), cg = min(tid, V4 - 1) % (JB / 4);
        const int tokv = min(k0 + tv, T - 1);
        xv = *reinterpret_cast<const v4f *>(row0 + (int64_t)tokv * Ch + 2 * d.Hk * DK + h * DV + j0 + 4 * cg);
        if (gated)
            xz = *reinterpret_cast<const v4f *>(gate_z + (((int64_t)c * T + tokv) * Hv + h) * DV + j0 + 4 * cg);
        const int tokg = min(k0 + min(tid, BC - 1), T - 1);
        xb = beta_logits[((int64_t)c * T + tokg) * gate_stride + h];
        xa = alpha_logits[((int64_t)c * T + tokg) * gate_stride + h];
    };
    load_chunk(0);
    __builtin_amdgcn_sched_barrier(0);
    const int s = __builtin_amdgcn_readfirstlane(s_v);
    const bool s_ok = s >= 0 && s < d.P;
    // the state tile of this wave in the MFMA operand layout:
    // sreg[q][e] = S[16q + 4*g4 + e][j0 + 16*wave + l16]   (waves w < CT)
    float *Sp = state_pool + ((int64_t)(s_ok ? s : 0) * Hv + h) * DK * DV + j0 + 16 * min(wave, CT - 1) + l16;
    v4f sreg[KC];
#pragma unroll
    for (int q = 0; q < KC; ++q)
#pragma unroll
        for (int e = 0; e < 4; ++e) sreg[q][e] = Sp[(16 * q + 4 * g4 + e) * DV];

    const int bits = slot_preflight<kThreads>(lanes, slot_ids, d.C, d.P, s_bitmap, &s_word);
    if (bits || st_in) {
        if (bits && blockIdx.x == 0 && blockIdx.y == 0 && tid == 0) atomicOr(status, bits);
        return;
    }
    if (s < 0) return;  // padding lane (uniform over the workgroup)

    for (int k0 = 0; k0 < T; k0 += BC) {
        const int nc = min(BC, T - k0);  // tokens of this chunk (the rest are zero rows)
        // ---- stage the chunk; wave 0 forms the gates and the cumulative log-decay
#pragma unroll
        for (int u = 0; u < QPT; ++u) {
            const int f = tid + kThreads * u;
            if (f < 2 * QK4) {
                const int m = f / QK4, r = f - m * QK4, t = r / (DK / 4), grp = r - t * (DK / 4);
                *reinterpret_cast<v4f *>((m ? Kl : Ql) + t * SX + 4 * grp) = t < nc ? xq[u] : v4f{0.f, 0.f, 0.f, 0.f};
            }
        }
        if (tid < V4) {
            const int tv = tid / (JB / 4), cg = tid % (JB / 4);
            *reinterpret_cast<v4f *>(Vl + tv * SV + 4 * cg) = tv < nc ? xv : v4f{0.f, 0.f, 0.f, 0.f};
            if (gated) *reinterpret_cast<v4f *>(Zl + tv * SV + 4 * cg) = xz;
        }
        if (wave == 0) {
            const bool real = lane < nc;
            const float ell = real ? fast_softplus(xa + dt) * Ah : 0.f;  // log g
            const float L = group_sum_last<16>(ell);                     // inclusive prefix over tokens
            if (lane < BC) {
                s_beta[lane] = real ? fast_sigmoid(xb) : 0.f;
                s_L[lane] = L;
            }
        }
        lds_barrier();

        // ---- the next chunk's loads go out now, under this chunk's arithmetic
        if (k0 + BC < T) load_chunk(k0 + BC);

        // ---- inverse norms of the 32 raw rows: 8 threads per row
        {
            const int r = tid >> 3, p = tid & 7;
            const float *x = (r < BC ? Kl + r * SX : Ql + (r - BC) * SX);
            float ss = 0.f;
#pragma unroll
            for (int e = p; e < DK; e += 8) ss = fmaf(x[e], x[e], ss);
            ss = group_sum_last<8>(ss);
            if (p == 7) (r < BC ? s_rk[r] : s_rq[r - BC]) = inv_norm(ss);
        }
        // ---- Gram partials (d_k chunk q on wave q % 4) and this wave's [K; Q] S tile
        v4f ks = {0.f, 0.f, 0.f, 0.f}, qs = ks, gkk = ks, gqk = ks;
#pragma unroll
        for (int q = 0; q < KC; ++q) {
            const v4f ak = *reinterpret_cast<const v4f *>(Kl + l16 * SX + 16 * q + 4 * g4);
            const v4f aq = *reinterpret_cast<const v4f *>(Ql + l16 * SX + 16 * q + 4 * g4);
            if (q % kWaves == wave) {
                gkk = mfma4(ak, ak, gkk);
                gqk = mfma4(aq, ak, gqk);
            }
            if (wave < CT) {
                ks = mfma4(ak, sreg[q], ks);
                qs = mfma4(aq, sreg[q], qs);
            }
        }
        *reinterpret_cast<v4f *>(&s_gram[wave][0][lane * 4]) = gkk;
        *reinterpret_cast<v4f *>(&s_gram[wave][1][lane * 4]) = gqk;
        lds_barrier();

        // ---- coefficients, thread (i, a)
        {
            const int i = tid >> 4, a = tid & 15, idx = tile_index(i, a);
            float kk = 0.f, qk = 0.f;
#pragma unroll
            for (int w = 0; w < kWaves; ++w) {
                kk += s_gram[w][0][idx];
                qk += s_gram[w][1][idx];
            }
            const float r = a <= i ? fast_exp(s_L[i] - s_L[a]) * s_rk[a] : 0.f;
            Lm[i * SG + a] = a < i ? r * kk * (s_beta[i] * s_rk[i]) : 0.f;
            Cq[i * SG + a] = r * qk * (s_rq[i] * isd);
        }
        lds_barrier();

        // ---- T = (I + Lm)^-1: lane (column a, row i) over rows of 16 lanes
        {
            const int a = 4 * wave + (lane >> 4), i = lane & 15;
            v4f Lr[4];
#pragma unroll
            for (int k4 = 0; k4 < 4; ++k4) Lr[k4] = *reinterpret_cast<const v4f *>(Lm + i * SG + 4 * k4);
            Tm[i * SG + a] = bcast_solve(i == a ? 1.f : 0.f, Lr, std::make_integer_sequence<int, 16>());
        }
        lds_barrier();

        // ---- per wave: D = T rhs, O = diag(gq) QS + Cq D, the gate, and the state update
        if (wave < CT) {
            const int jj = 16 * wave + l16;
            const float Lend = s_L[BC - 1];  // padding tokens add no decay
            v4f rhs, o, bw;
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int t = 4 * g4 + v;
                const float G = fast_exp(s_L[t]);
                rhs[v] = s_beta[t] * (Vl[t * SV + jj] - G * s_rk[t] * ks[v]);
                o[v] = G * s_rq[t] * isd * qs[v];
            }
            const v4f dl = mfma4(*reinterpret_cast<const v4f *>(Tm + l16 * SG + 4 * g4), rhs, v4f{0.f, 0.f, 0.f, 0.f});
            o = mfma4(*reinterpret_cast<const v4f *>(Cq + l16 * SG + 4 * g4), dl, o);
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int t = 4 * g4 + v;
                if (gated) {
                    const float z = Zl[t * SV + jj];
                    o[v] *= gate_mode == 0 ? fast_silu(z) : fast_sigmoid(z);
                }
                Ot[t * SV + jj] = o[v];
                bw[v] = fast_exp(Lend - s_L[t]) * s_rk[t] * dl[v];
            }
            // S <- G_end S + K^T diag(w) D, tile by tile of 16 d_k rows: the A operand is
            // K^T (lane supplies K[token 4*g4 + s][16 rt + l16] in step s)
            const float Gend = fast_exp(Lend);
#pragma unroll
            for (int rt = 0; rt < KC; ++rt) {
                v4f a4;
#pragma unroll
                for (int e = 0; e < 4; ++e) a4[e] = Kl[(4 * g4 + e) * SX + 16 * rt + l16];
                sreg[rt] = mfma4(a4, bw, Gend * sreg[rt]);
            }
        }
        lds_barrier();

        // ---- outputs of the chunk: 16-byte chunks of whole rows from consecutive lanes
        for (int f = tid; f < nc * (JB / 4); f += kThreads) {
            const int t = f / (JB / 4), cg = f - t * (JB / 4);
            __builtin_nontemporal_store(*reinterpret_cast<const v4f *>(Ot + t * SV + 4 * cg),
                                        reinterpret_cast<v4f *>(out + (((int64_t)c * T + k0 + t) * Hv + h) * DV + j0) + cg);
        }
    }

    // ---- the slot's state, in place
    if (wave < CT) {
#pragma unroll
        for (int q = 0; q < KC; ++q)
#pragma unroll
            for (int e = 0; e < 4; ++e) __builtin_nontemporal_store(sreg[q][e], Sp + (16 * q + 4 * g4 + e) * DV);
    }
}

template <int DK, int DV>
hipError_t launch(const Dims &d, int T, const float *qkv, const float *beta_logits, const float *alpha_logits,
                  int64_t gate_stride, const float *dt_bias, const float *A, float *state_pool,
                  const int32_t *slot_ids, const float *gate_z, int gate_mode, float *out, int32_t *status,
                  hipStream_t stream) {
    hipLaunchKernelGGL((prefill_kernel<DK, DV>), dim3(PrefillCfg<DK, DV>::NB * d.Hv, d.C), dim3(kThreads), 0, stream, d,
                       T, qkv, beta_logits, alpha_logits, gate_stride, dt_bias, A, state_pool, slot_ids, gate_z,
                       gate_mode, out, status);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill(const Dims &d, int n_tokens, const float *qkv, const float *beta_logits,
                          const float *alpha_logits, int64_t gate_stride, const float *dt_bias, const float *A,
                          float *state_pool, const int32_t *slot_ids, const float *gate_z, int gate_mode, float *out,
                          int32_t *status, hipStream_t stream) {
#define GDN_PREFILL_CASE(K, V)                                                                                  \
    if (d.dk == K && d.dv == V)                                                                                 \
        return launch<K, V>(d, n_tokens, qkv, beta_logits, alpha_logits, gate_stride, dt_bias, A, state_pool, \
                            slot_ids, gate_z, gate_mode, out, status, stream);
#define GDN_PREFILL_ROW(K) GDN_PREFILL_CASE(K, 16) GDN_PREFILL_CASE(K, 32) GDN_PREFILL_CASE(K, 64) GDN_PREFILL_CASE(K, 128)
    GDN_PREFILL_ROW(16) GDN_PREFILL_ROW(32) GDN_PREFILL_ROW(64) GDN_PREFILL_ROW(128)
#undef GDN_PREFILL_ROW
#undef GDN_PREFILL_CASE
    return hipErrorInvalidValue;
}

}  // namespace gdn
