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
// chunk start (G_t = exp(L_t)), raw rows q_t, k_t, inverse norms rk_t, rq_t and the state
// S at the chunk start:
//   (I + Lm) D = rhs,  rhs_t = beta_t (v_t - G_t rk_t (K S)_t),
//   Lm[t][u] = beta_t exp(L_t - L_u) rk_t rk_u (k_t . k_u)                 (u < t)
//   O_t = G_t rq_t (Q S)_t / sqrt(d_k) + sum_{u <= t} Cq[t][u] D_u,
//   Cq[t][u] = exp(L_t - L_u) rq_t rk_u (q_t . k_u) / sqrt(d_k)            (u <= t)
//   S <- G_B S + sum_u exp(L_B - L_u) rk_u k_u D_u^T
// i.e. the tree verify's formulation on a chain, followed by the state update.
//
// Two launches.  Everything that does not involve the state -- norms, gates, the Gram
// products, Lm, Cq and T = (I + Lm)^-1 -- depends on one chunk's tokens only, so the first
// kernel computes it for every chunk at once (a workgroup per lane, q/k head and chunk,
// sharing the norms and Gram products among the value heads of the q/k head), into one
// package of kPackFloats floats per value head in the caller's workspace.  The second kernel
// carries the state through the chunks in order and does only what involves it: the
// products [K; Q] S (split bf16), D = T rhs, O = diag(c) QS + Cq D (float32), the output gate
// and the update (split bf16, three parts), with the operand permutation of mfma4, so the
// state tile stays in float32 registers across chunks in exactly the layout in which the next
// chunk's products and the update consume and produce it.
//
// Package of (lane c, value head h, chunk j), at float offset ((c H_v + h) n_chunks + j) *
// kPackFloats of the workspace.  T is unit lower triangular (the substitution leaves its
// diagonal exactly 1 and the part above it exactly 0) and Cq lower triangular, so each row
// travels only as far as the 4-float groups that hold its entries below (T) or on and below
// (Cq) the diagonal: row t of T as its first 4 ceil(t / 4) floats, row t of Cq as its first
// 4 ceil((t + 1) / 4), rows one after another (every group is a 16-byte piece of one row):
//   [0, 144)    T row segments                     [144, 304)  Cq row segments
//   [304, 320)  a_t = beta_t                       [320, 336)  b_t = G_t rk_t
//   [336, 352)  c_t = G_t rq_t / sqrt(d_k)         [352, 368)  w_t = exp(L_B - L_t) rk_t
//   [368]       G_B                                [369, 372)  unused
// Padding tokens of the last chunk are zero rows: beta = 0 and no decay, so they write
// nothing into D, O or the state.
#include <mutex>

#include "gdn_device.h"
#include "gdn_internal.h"

namespace gdn {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int BC = kPrefillChunk;  // tokens per chunk
static_assert(BC == 16, "one 16 x 16 MFMA tile of tokens per chunk");
// row segments of the packed T (strictly lower) and Cq (lower) rows: length and start, with
// ceil_sum(n) = sum over s = 1..n of ceil(s / 4) = (m + 1) (2m + r) for n = 4m + r
__host__ __device__ constexpr int seg_t(int t) { return (t + 3) / 4 * 4; }
__host__ __device__ constexpr int seg_c(int t) { return (t + 4) / 4 * 4; }
__host__ __device__ constexpr int ceil_sum(int n) { return n <= 0 ? 0 : (n / 4 + 1) * (2 * (n / 4) + n % 4); }
__host__ __device__ constexpr int seg_t_start(int t) { return 4 * ceil_sum(t - 1); }
__host__ __device__ constexpr int seg_c_start(int t) { return 4 * ceil_sum(t); }
static_assert(seg_t_start(2) == 4 && seg_t_start(5) == 16 && seg_c_start(1) == 4 && seg_c_start(4) == 16 &&
                  seg_c_start(5) == 24,
              "row segment starts");
constexpr int PK_T = 0, PK_CQ = seg_t_start(BC), PK_A = PK_CQ + seg_c_start(BC), PK_B = PK_A + BC, PK_C = PK_B + BC,
              PK_W = PK_C + BC, PK_GEND = PK_W + BC;
static_assert(PK_CQ == 144 && PK_A == 304, "package layout");
static_assert(PK_GEND + 4 == kPackFloats && kPackFloats % 4 == 0, "package layout");

template <int DK, int DV>
struct PrefillCfg {
    static constexpr int JB = DV < 64 ? DV : 64;      // value columns per state workgroup
    static constexpr int NB = DV / JB;                // column blocks per head
    static constexpr int CT = JB / 16;                // 16-column tiles: wave w < CT owns tile w
    static constexpr int KC = DK / 16;                // 16-wide chunks of d_k
    static constexpr int SX = DK + 4;                 // raw q / k rows in LDS (4 mod 8 floats)
    static constexpr int SG = BC + 4;                 // 16 x 16 matrices
    static constexpr int QK4 = BC * DK / 4;           // float4 groups of a chunk's q (or k) rows
    static constexpr int QPT = (2 * QK4 + kThreads - 1) / kThreads;
};

// x = hi + mid + lo + r, each part the bf16 rounding (to nearest even) of what the parts
// before it leave (so hi and mid are also the two-part split), |r| <= 2^-26 |x|; by pairs of
// consecutive values, each part of a pair as one packed word (element 0 in the low half)
__device__ inline void split3_bf16(const float (&x)[4], unsigned (&h)[2], unsigned (&m)[2], unsigned (&l)[2]) {
#pragma unroll
    for (int e = 0; e < 2; ++e) {
        unsigned u = __builtin_bit_cast(unsigned, bf2{(__bf16)x[2 * e], (__bf16)x[2 * e + 1]});
        asm("" : "+v"(u));  // (opaque: keeps one packed conversion per pair)
        const float r0 = x[2 * e] - __builtin_bit_cast(float, u << 16);
        const float r1 = x[2 * e + 1] - __builtin_bit_cast(float, u & 0xffff0000u);
        unsigned v = __builtin_bit_cast(unsigned, bf2{(__bf16)r0, (__bf16)r1});
        asm("" : "+v"(v));
        const float s0 = r0 - __builtin_bit_cast(float, v << 16), s1 = r1 - __builtin_bit_cast(float, v & 0xffff0000u);
        h[e] = u;
        m[e] = v;
        l[e] = __builtin_bit_cast(unsigned, bf2{(__bf16)s0, (__bf16)s1});
    }
}

// element (i, a) of a 16 x 16 accumulator tile stored lane-major (lane * 4 + component)
__device__ inline int tile_index(int i, int a) { return (16 * (i >> 2) + a) * 4 + (i & 3); }

// Raw buffer resources: word 3 of the descriptor for the gfx9 family (32-bit data,
// unswizzled).  A load whose byte offset lies outside [0, num_records) returns zero and
// a store there is dropped, without a memory access.
constexpr int kRsrcWord3 = 0x00020000;
constexpr int kNonTemporal = 2;  // cache-policy operand of the buffer stores: nt
typedef int v4i __attribute__((ext_vector_type(4)));
typedef unsigned v4u __attribute__((ext_vector_type(4)));
typedef float v2f __attribute__((ext_vector_type(2)));

__device__ inline __amdgpu_buffer_rsrc_t rsrc(const float *base, int bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<float *>(base), 0, bytes, kRsrcWord3);
}
__device__ inline float load1(__amdgpu_buffer_rsrc_t r, int off) {
    return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0));
}
__device__ inline v4f load4(__amdgpu_buffer_rsrc_t r, int off) {
    return __builtin_bit_cast(v4f, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}
__device__ inline v2f load2(__amdgpu_buffer_rsrc_t r, int off, int soff) {
    return __builtin_bit_cast(v2f, __builtin_amdgcn_raw_buffer_load_b64(r, off, soff, 0));
}

// The q and k rows of q/k head kh of one chunk, as float4 groups: item u of a thread is
// group f = tid + kThreads * u of the q rows (f < QK4), then of the k rows.  `off` is the
// group's byte offset from the chunk's first row; the chunk's resource ends after its last
// real token, so the rows of padding tokens read as zero.
template <int DK>
struct ChunkRows {
    using Cfg = PrefillCfg<DK, 16>;
    int off[Cfg::QPT], lds[Cfg::QPT];  // byte offset in the chunk, float offset in [Q; K] LDS rows
    v4f x[Cfg::QPT];
    __device__ ChunkRows(int Ch, int Hk, int kh) {
#pragma unroll
        for (int u = 0; u < Cfg::QPT; ++u) {
            const int f = min((int)threadIdx.x + kThreads * u, 2 * Cfg::QK4 - 1);
            const int m = f / Cfg::QK4, r = f - m * Cfg::QK4, t = r / (DK / 4), grp = r - t * (DK / 4);
            off[u] = (t * Ch + m * Hk * DK + kh * DK + 4 * grp) * 4;
            lds[u] = (m * BC + t) * Cfg::SX + 4 * grp;
        }
    }
    __device__ void load(__amdgpu_buffer_rsrc_t r) {
#pragma unroll
        for (int u = 0; u < Cfg::QPT; ++u) x[u] = load4(r, off[u]);
    }
    // into LDS: q rows at [0, BC), k rows at [BC, 2 BC) of rows of Cfg::SX floats
    __device__ void stage(float *QK) const {
#pragma unroll
        for (int u = 0; u < Cfg::QPT; ++u)
            if ((int)threadIdx.x + kThreads * u < 2 * Cfg::QK4) *reinterpret_cast<v4f *>(QK + lds[u]) = x[u];
    }
};

// ---- kernel 1: the packages of one (lane, q/k head, chunk), for each value head that
// shares the q/k head.  Grid (chunks * H_k, C).
template <int DK>
__global__ __launch_bounds__(kThreads) void prefill_prep_kernel(
    Dims d, int T, const float *__restrict__ qkv, const float *__restrict__ beta_logits,
    const float *__restrict__ alpha_logits, int64_t gate_stride, const float *__restrict__ dt_bias,
    const float *__restrict__ A, float *__restrict__ pack) {
    using Cfg = PrefillCfg<DK, 16>;
    constexpr int SX = Cfg::SX, SG = Cfg::SG, KC = Cfg::KC;
    constexpr int HG = kThreads / BC;  // value heads whose gates are formed together
    __shared__ __align__(16) float QK[2 * BC * SX];  // q rows, then k rows
    __shared__ __align__(16) float s_gram[kWaves][2][256];
    __shared__ __align__(16) float Lm[BC * SG], Tm[BC * BC];
    __shared__ float s_rk[BC], s_rq[BC], s_kk[256], s_qk[256];
    __shared__ float s_beta[HG][BC];
    __shared__ double s_L[HG][BC];
    const float *Ql = QK, *Kl = QK + BC * SX;

    const int nch = (T + BC - 1) / BC;
    const int j = blockIdx.x % nch, kh = blockIdx.x / nch, c = blockIdx.y;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, g4 = lane >> 4, l16 = lane & 15;
    const int k0 = j * BC, nc = min(BC, T - k0);
    const int R = d.Hv / d.Hk;  // value heads h = kh + H_k m, m < R
    // (a padding lane's packages are computed like any other and never read)

    ChunkRows<DK> rows(d.Ch, d.Hk, kh);
    rows.load(rsrc(qkv + ((int64_t)c * T + k0) * d.Ch, nc * d.Ch * 4));
    // gate inputs of value heads m0 .. m0 + HG - 1 for thread (m, t): a row of 16 lanes per
    // head (the first group's go out with the rows)
    float xb, xa, xA;
    auto load_gates = [&](int m0) {
        const int h = kh + d.Hk * min(m0 + (tid >> 4), R - 1);
        const int64_t trow = (int64_t)c * T + min(k0 + (tid & 15), T - 1);
        xb = beta_logits[trow * gate_stride + h];
        xa = alpha_logits[trow * gate_stride + h] + dt_bias[h];
        xA = A[h];
    };
    load_gates(0);
    rows.stage(QK);
    lds_barrier();

    // inverse norms of the 32 raw rows, 8 threads per row
    {
        const int r = tid >> 3, p = tid & 7;
        const float *x = r < BC ? Kl + r * SX : Ql + (r - BC) * SX;
        float ss = 0.f;
#pragma unroll
        for (int e = 0; e < DK / 8; ++e) ss = fmaf(x[p + 8 * e], x[p + 8 * e], ss);
        ss = group_sum_last<8>(ss);
        if (p == 7) (r < BC ? s_rk[r] : s_rq[r - BC]) = inv_norm(ss);
    }
    // Gram partials K K^T and Q K^T, d_k chunk q on wave q % 4
    {
        v4f gkk = {0.f, 0.f, 0.f, 0.f}, gqk = gkk;
#pragma unroll
        for (int q = 0; q < KC; ++q) {
            if (q % kWaves != wave) continue;
            const v4f ak = *reinterpret_cast<const v4f *>(Kl + l16 * SX + 16 * q + 4 * g4);
            const v4f aq = *reinterpret_cast<const v4f *>(Ql + l16 * SX + 16 * q + 4 * g4);
            gkk = mfma4(ak, ak, gkk);
            gqk = mfma4(aq, ak, gqk);
        }
        *reinterpret_cast<v4f *>(&s_gram[wave][0][lane * 4]) = gkk;
        *reinterpret_cast<v4f *>(&s_gram[wave][1][lane * 4]) = gqk;
    }
    lds_barrier();
    {  // thread (i, a): k_i . k_a and q_i . k_a
        const int i = tid >> 4, a = tid & 15, idx = tile_index(i, a);
        float kk = 0.f, qk = 0.f;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
            kk += s_gram[w][0][idx];
            qk += s_gram[w][1][idx];
        }
        s_kk[tid] = kk;
        s_qk[tid] = qk;
    }

    const float isd = 1.0f / sqrtf((float)DK);
    for (int m0 = 0; m0 < R; m0 += HG) {
        // gates of value heads m0 .. m0 + HG - 1 and the inclusive prefix of the log-decays
        // over the chunk
        if (m0 > 0) load_gates(m0);
        {
            const int t = tid & 15;
            const bool real = t < nc;
            // the prefix in double: a chunk of strong decays reaches hundreds, where a float
            // sum would lose about 1e-4 of every ratio exp(L_t - L_u) formed from it
            const double ell = real ? fast_softplus(xa) * xA : 0.f;  // log g
            const double L = group_sum_last<16>(ell);
            s_beta[tid >> 4][t] = real ? fast_sigmoid(xb) : 0.f;
            s_L[tid >> 4][t] = L;
        }
        for (int m = m0; m < min(R, m0 + HG); ++m) {
            lds_barrier();  // gates formed; the previous head's Tm and Lm consumed
            const int h = kh + d.Hk * m, mg = m - m0;
            float *pk = pack + (((int64_t)c * d.Hv + h) * nch + j) * kPackFloats;
            {
                const int i = tid >> 4, a = tid & 15;
                const float r = a <= i ? fast_exp((float)(s_L[mg][i] - s_L[mg][a])) * s_rk[a] : 0.f;
                Lm[i * SG + a] = a < i ? r * s_kk[tid] * (s_beta[mg][i] * s_rk[i]) : 0.f;
                if (a < seg_c(i)) pk[PK_CQ + seg_c_start(i) + a] = r * s_qk[tid] * (s_rq[i] * isd);
            }
            if (tid < BC) {
                const float G = fast_exp((float)s_L[mg][tid]);
                const double Lend = s_L[mg][BC - 1];  // padding adds no decay
                pk[PK_A + tid] = s_beta[mg][tid];
                pk[PK_B + tid] = G * s_rk[tid];
                pk[PK_C + tid] = G * s_rq[tid] * isd;
                pk[PK_W + tid] = fast_exp((float)(Lend - s_L[mg][tid])) * s_rk[tid];
                if (tid == 0) pk[PK_GEND] = fast_exp((float)Lend);
            }
            lds_barrier();
            // T = (I + Lm)^-1: lane (column a, row i) over rows of 16 lanes
            {
                const int a = 4 * wave + (lane >> 4), i = lane & 15;
                v4f Lr[4];
#pragma unroll
                for (int k4 = 0; k4 < 4; ++k4) Lr[k4] = *reinterpret_cast<const v4f *>(Lm + i * SG + 4 * k4);
                Tm[i * BC + a] = bcast_solve(i == a ? 1.f : 0.f, Lr, std::make_integer_sequence<int, 16>());
            }
            lds_barrier();
            {  // T's row segments: thread (row i, group a4) stores a 16-byte group of row i
                const int i = tid >> 2, a4 = tid & 3;
                if (tid < 4 * BC && 4 * a4 < seg_t(i))
                    *reinterpret_cast<v4f *>(pk + PK_T + seg_t_start(i) + 4 * a4) =
                        *reinterpret_cast<const v4f *>(Tm + i * BC + 4 * a4);
            }
        }
        lds_barrier();  // s_beta / s_L of this group consumed
    }
}

// A chunk's package in LDS: T and Cq with rows of LP_S floats (so that 16 lanes reading a
// 16-byte piece of one row each hit distinct banks), then the four per-token vectors and
// G_B.  T's diagonal and the parts of both matrices past their rows' segments are set once
// (1 on T's diagonal, 0 elsewhere) and never staged; thread t < kPkGroups stages group t of
// the package, a 16-byte piece of one row.
constexpr int LP_S = BC + 4, LP_T = 0, LP_CQ = BC * LP_S, LP_V = 2 * BC * LP_S, LP_G = LP_V + 4 * BC;
constexpr int LP_FLOATS = LP_G + 4, kPkGroups = kPackFloats / 4;
static_assert(kPkGroups <= kThreads, "one package group per thread");
__device__ inline int package_lds_offset(int g) {  // float offset in LDS of package group g
    const int f = 4 * g;
    if (f < PK_CQ) {  // a segment of T's row t
        int t = 1;
        while (seg_t_start(t + 1) <= f) ++t;
        return LP_T + t * LP_S + (f - seg_t_start(t));
    }
    if (f < PK_A) {  // a segment of Cq's row t
        int t = 0;
        while (seg_c_start(t + 1) <= f - PK_CQ) ++t;
        return LP_CQ + t * LP_S + (f - PK_CQ - seg_c_start(t));
    }
    return f < PK_GEND ? LP_V + (f - PK_A) : LP_G;  // the vectors; G_B and the unused floats
}

// ---- kernel 2: the state through the chunks.  One workgroup (4 waves) per (lane, value
// head, block of 64 value columns); wave w owns the 16-column tile w of the state for the
// whole prompt.  Workgroup ids are ordered so that the workgroups sharing one (lane, q/k
// head) are congruent modulo C * H_k and read the shared q/k rows through one L2.
//
// Per chunk, in order: the products [K; Q] S in split bf16 (three bf16 products of hi / lo
// parts, accumulated in float32), then D = T rhs, O = diag(c) QS + Cq D and the output gate on
// float32 MFMA, and the update S <- G_B S + K^T diag(w) D as three bf16 products of
// three-part splits (accumulated in float32).  On this chip the float32 matrix instructions
// and the vector ALU share one arithmetic rate, so the chunk costs the sum of its float32 MFMA
// and VALU work: the split forms replace [K; Q] S's 64 float32 MFMAs per wave with 24 bf16
// ones and the split of the state tile, and the update's 32 with 24 bf16 ones and the split
// of diag(w) D (the q / k rows and K^T are split once per workgroup at staging).  A two-part
// split of the update would drop terms near 2^-17 of it, which a prompt of near-parallel keys
// accumulates to about 1e-4 of the state; the three-part form keeps every term above 2^-24.
//
// One barrier per chunk: chunk j's rows (bf16 parts of q / k rows and of K^T), package, values and
// gate values are staged in LDS buffers j % 2 from registers loaded during the iteration
// before, so a stage never overlaps a wave still reading chunk j - 1.  Every global access of
// the loop is a raw buffer access whose range ends at the chunk's last real token and is
// empty past the last chunk, so no load or store needs a branch; the values, gate values and
// package are one 16-byte load per thread each (a wave's vector memory instructions, not
// their bytes, set the address unit's time).
template <int DK, int DV, bool GATED>
__global__ __launch_bounds__(kThreads) void prefill_state_kernel(
    Dims d, int T, const float *__restrict__ qkv, const float *__restrict__ pack, float *__restrict__ state_pool,
    const int32_t *__restrict__ slot_ids, const float *__restrict__ gate_z, int gate_mode, float *__restrict__ out,
    int32_t *__restrict__ status) {
    using Cfg = PrefillCfg<DK, DV>;
    constexpr int JB = Cfg::JB, NB = Cfg::NB, CT = Cfg::CT, KC = Cfg::KC;
    constexpr int OG = JB / 4;               // 16-byte groups of a block row
    constexpr int VW = JB + 4;               // value rows in LDS (16 lanes of a row group on distinct banks)
    constexpr int VROWS = kThreads / OG;     // rows written by the staging threads (>= BC)
    constexpr int KM = (DK + 31) / 32;       // 32-wide chunks of d_k in the bf16 products (d_k = 16: one, half zero)
    constexpr int SXB = 32 * KM + 8;         // bf16 row stride (16 rows read with ds_read_b128 hit distinct banks)
    constexpr int XSB = 2 * BC * SXB;        // bf16 parts of one buffer: q rows, then k rows
    __shared__ unsigned int s_bitmap[kBitmapSlots / 32];
    __shared__ int s_word;
    constexpr int KAS = 8 * (BC / 4) + 8;    // K^T rows (d_k index) of the update's operands, in bf16
    // the 16-byte groups of a K^T row sit at group index (token quad) ^ ((row >> KSW) & 3), so
    // that neither the staging writes (rows 2i and 2i + 1 by lane i) nor the operand reads (rows
    // 16 rt + l by lane group l) of 16 lanes share a bank
    constexpr int KSW = 4;
    __shared__ __align__(16) __bf16 XS[2][2][XSB];        // per buffer: hi parts, lo parts of the q and k rows
    __shared__ __align__(16) __bf16 KA[2][DK * KAS];      // per buffer: K^T as [hi | mid] per 4 tokens
    __shared__ __align__(16) __bf16 KB[2][DK * KAS];      // per buffer: K^T as [lo | hi] per 4 tokens
    __shared__ __align__(16) float PK[2][LP_FLOATS + 4];  // (+ a slot the threads without a package group write)
    __shared__ __align__(16) float VZ[2][2][VROWS * VW];  // per buffer: value rows, gate value rows
    __shared__ __align__(16) float OT[2][BC * JB];        // per buffer: a chunk's output rows of the block

    const int n_groups = d.C * d.Hk;
    const int grp = blockIdx.x % n_groups, ws = blockIdx.x / n_groups;
    const int c = grp / d.Hk, kh = grp - c * d.Hk;
    const int jb = ws % NB, h = kh + d.Hk * (ws / NB), j0 = jb * JB;
    const int Ch = d.Ch, HvDV = d.Hv * DV;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, g4 = lane >> 4, l16 = lane & 15;
    const int cw = min(wave, CT - 1), jj = j0 + 16 * cw + l16;  // this lane's value column
    const int nch = (T + BC - 1) / BC;

    // ---- loads that do not need the slot first (the slot id through a vector load, so
    //      its wait does not hold up the loads behind it), then the state tile
    const int s_v = __builtin_bit_cast(
        int, __builtin_amdgcn_raw_buffer_load_b32(
                 __builtin_amdgcn_make_buffer_rsrc(const_cast<int32_t *>(slot_ids), 0, 4 * d.C, kRsrcWord3), 4 * c, 0,
                 0));
    const LaneSlotsT<kThreads> lanes(slot_ids, d.C);
    const int st_in = *status;

    // Per-thread pieces of the chunk buffers: thread t holds 16-byte group t % OG of block row
    // t / OG of the values, gate values and outputs (rows past BC read as zero and store
    // nothing) and package group t.
    const int b_row = tid / OG, b_grp = tid - b_row * OG;
    constexpr int kPast = 0x7ffffff0;  // a byte offset past every range: loads read zero, stores drop
    const int v_off = b_row < BC ? (b_row * Ch + 2 * d.Hk * DK + h * DV + j0 + 4 * b_grp) * 4 : kPast;
    const int z_off = b_row < BC ? (b_row * HvDV + h * DV + j0 + 4 * b_grp) * 4 : kPast;
    const int vz_lds = b_row * VW + 4 * b_grp;
    const int pk_off = tid < kPkGroups ? 16 * tid : kPast;
    const int pk_lds = tid < kPkGroups ? package_lds_offset(tid) : LP_FLOATS;
    const float *pk0 = pack + ((int64_t)c * d.Hv + h) * nch * kPackFloats;
    // chunk jc's tokens (0 past the end), and a buffer resource over rows of `row_floats`
    // floats of chunk jc of this lane, empty past the end
    auto chunk_len = [&](int jc) { return jc < nch ? min(BC, T - jc * BC) : 0; };
    auto chunk_rsrc = [&](const float *buf, int row_floats, int jc) {
        const int jcc = min(jc, nch - 1);
        return rsrc(buf + ((int64_t)c * T + jcc * BC) * row_floats, chunk_len(jc) * row_floats * 4);
    };
    // Per-thread pieces of a chunk's q and k rows.  k: half-block b = tid + kThreads u (u < KPT),
    // tokens 4 qd .. 4 qd + 3 of the columns 2 cp, 2 cp + 1 (qd = b / (DK / 2), cp = b % (DK / 2)),
    // four 8-byte loads (a wave's load covers whole rows); q: group f = tid + kThreads u
    // (u < QPT), columns 4 p .. 4 p + 3 of token t (t = f / (DK / 4), p = f % (DK / 4)).  Pieces
    // past the end (d_k < 128) load a real piece again and are not staged.
    constexpr int NKB = BC / 4 * (DK / 2), KPT = (NKB + kThreads - 1) / kThreads;
    constexpr int NQG = BC * DK / 4, QPT = (NQG + kThreads - 1) / kThreads;
    // In the bf16 parts of the rows (the products with the state) the columns of each 32-wide
    // chunk m of d_k are permuted so that lane group g of a product supplies, in slots 8g ..
    // 8g + 7, the columns 32m + 4g + 0..3 and 32m + 16 + 4g + 0..3: the same d_k rows as the
    // state tile's registers sreg[2m] and sreg[2m + 1] (column 32m + 16h + 4g + e sits at
    // 32m + 8g + 4h + e).
    auto xs_col = [](int col) { return 32 * (col >> 5) + 8 * ((col >> 2) & 3) + 4 * ((col >> 4) & 1) + (col & 3); };
    int k_off[KPT], ka_at[KPT], kx_at[KPT], q_off[QPT], qx_at[QPT];
#pragma unroll
    for (int u = 0; u < KPT; ++u) {
        const int b = min(tid + kThreads * u, NKB - 1), qd = b / (DK / 2), col = 2 * (b - qd * (DK / 2));
        k_off[u] = (4 * qd * Ch + d.Hk * DK + kh * DK + col) * 4;
        ka_at[u] = col * KAS + 8 * (qd ^ ((col >> KSW) & 3));  // (rows col and col + 1 alike)
        kx_at[u] = (BC + 4 * qd) * SXB + xs_col(col);
    }
#pragma unroll
    for (int u = 0; u < QPT; ++u) {
        const int f = min(tid + kThreads * u, NQG - 1), t = f / (DK / 4), col = 4 * (f - t * (DK / 4));
        q_off[u] = (t * Ch + kh * DK + col) * 4;
        qx_at[u] = t * SXB + xs_col(col);
    }
    // Two chunks' loads are in flight at a time (register sets A and B, loaded two iterations
    // before their chunk is staged): one iteration does not cover the loads' latency.
    struct ChunkRegs {
        v2f kx[KPT][4];  // the k half-blocks of this thread: kx[u][s] = token 4 qd + s
        v4f qx[QPT];     // the q groups
        v4f pk, v, z;    // package group, values, gate values
    };
    auto load_chunk = [&](ChunkRegs &r, int jc) {  // rows, package, values and gate values of chunk jc
        const __amdgpu_buffer_rsrc_t rr = chunk_rsrc(qkv, Ch, jc);
#pragma unroll
        for (int u = 0; u < KPT; ++u)
#pragma unroll
            for (int s = 0; s < 4; ++s) r.kx[u][s] = load2(rr, k_off[u], s * Ch * 4);
#pragma unroll
        for (int u = 0; u < QPT; ++u) r.qx[u] = load4(rr, q_off[u]);
        r.pk = load4(rsrc(pk0 + (int64_t)min(jc, nch - 1) * kPackFloats, jc < nch ? kPackFloats * 4 : 0), pk_off);
        r.v = load4(chunk_rsrc(qkv, Ch, jc), v_off);
        if constexpr (GATED) r.z = load4(chunk_rsrc(gate_z, HvDV, jc), z_off);
    };
    ChunkRegs ra, rb;
    load_chunk(ra, 0);
    load_chunk(rb, 1);
    __builtin_amdgcn_sched_barrier(0);
    const int s = __builtin_amdgcn_readfirstlane(s_v);
    const bool s_ok = s >= 0 && s < d.P;
    // the state tile of this wave in the MFMA operand layout (waves past the last tile, CT < 4,
    // hold tile CT - 1): sreg[q][e] = S[16q + 4*g4 + e][jj]
    float *Sp = state_pool + ((int64_t)(s_ok ? s : 0) * d.Hv + h) * DK * DV + jj;
    v4f sreg[KC];
#pragma unroll
    for (int q = 0; q < KC; ++q)
#pragma unroll
        for (int e = 0; e < 4; ++e) sreg[q][e] = Sp[(16 * q + 4 * g4 + e) * DV];

    const int bits = slot_preflight<kThreads>(lanes, slot_ids, d.C, d.P, s_bitmap, &s_word);
    if (bits || st_in) {
        if (bits && blockIdx.x == 0 && tid == 0) atomicOr(status, bits);
        return;
    }
    if (s < 0) return;  // padding lane (uniform over the workgroup)

    // a chunk's outputs wait in OT[jc % 2] until the next barrier, then every thread stores a
    // 16-byte piece of whole rows of the block (JB consecutive floats of a row): a row's lines
    // are written by one store instruction instead of a 64-byte segment by each of CT waves
    const int o_off = b_row < BC ? (b_row * HvDV + h * DV + j0 + 4 * b_grp) * 4 : kPast;
    const int o_lds = min(b_row, BC - 1) * JB + 4 * b_grp;
    auto store_outputs = [&](int jc) {  // chunk jc's outputs (none for jc < 0)
        const v4f ov = *reinterpret_cast<const v4f *>(&OT[jc & 1][o_lds]);
        const int jcc = max(jc, 0), live = jc >= 0;  // (a product, not a select: no branch)
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(v4i, ov),
                                               rsrc(out + ((int64_t)c * T + jcc * BC) * HvDV,
                                                    live * chunk_len(jcc) * HvDV * 4),
                                               o_off, 0, kNonTemporal);
    };

    // Staging of a chunk: the q and k rows as their bf16 hi / lo parts (the products with the
    // state), K^T in three bf16 parts (the update's left operand), the package, the values and
    // the gate values.  The k rows' hi / lo parts are the hi / mid of their three-part split.
    auto stage_chunk = [&](int buf, const ChunkRegs &r) {
        __bf16 *xh = XS[buf][0], *xl = XS[buf][1];
#pragma unroll
        for (int u = 0; u < KPT; ++u) {
            if (NKB % kThreads != 0 && tid + kThreads * u >= NKB) continue;
            unsigned hi[2][2], mi[2][2], lo[2][2];  // [column j][token pair], packed bf16 pairs
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const float c4[4] = {r.kx[u][0][j], r.kx[u][1][j], r.kx[u][2][j], r.kx[u][3][j]};
                split3_bf16(c4, hi[j], mi[j], lo[j]);
                *reinterpret_cast<v4u *>(KA[buf] + ka_at[u] + j * KAS) = v4u{hi[j][0], hi[j][1], mi[j][0], mi[j][1]};
                *reinterpret_cast<v4u *>(KB[buf] + ka_at[u] + j * KAS) = v4u{lo[j][0], lo[j][1], hi[j][0], hi[j][1]};
            }
#pragma unroll
            for (int s = 0; s < 4; ++s) {  // token 4 qd + s: its two columns' hi and mid parts
                const int w = s >> 1;
                const unsigned h = s & 1 ? (hi[0][w] >> 16) | (hi[1][w] & 0xffff0000u)
                                         : (hi[0][w] & 0xffffu) | (hi[1][w] << 16);
                const unsigned m = s & 1 ? (mi[0][w] >> 16) | (mi[1][w] & 0xffff0000u)
                                         : (mi[0][w] & 0xffffu) | (mi[1][w] << 16);
                *reinterpret_cast<unsigned *>(xh + kx_at[u] + s * SXB) = h;
                *reinterpret_cast<unsigned *>(xl + kx_at[u] + s * SXB) = m;
            }
        }
#pragma unroll
        for (int u = 0; u < QPT; ++u) {
            if (NQG % kThreads != 0 && tid + kThreads * u >= NQG) continue;
            const v4f x = r.qx[u];
            const float xa[4] = {x[0], x[1], x[2], x[3]};
            __bf16 hi[4], lo[4];
            split_bf16(xa, hi, lo);
            *reinterpret_cast<bf4 *>(xh + qx_at[u]) = bf4{hi[0], hi[1], hi[2], hi[3]};
            *reinterpret_cast<bf4 *>(xl + qx_at[u]) = bf4{lo[0], lo[1], lo[2], lo[3]};
        }
        *reinterpret_cast<v4f *>(PK[buf] + pk_lds) = r.pk;
        *reinterpret_cast<v4f *>(VZ[buf][0] + vz_lds) = r.v;
        if constexpr (GATED) *reinterpret_cast<v4f *>(VZ[buf][1] + vz_lds) = r.z;
    };
    // T's diagonal (1) and the parts above T's and Cq's diagonals (0) in both package buffers,
    // once; (d_k = 16) the missing half of the one 32-wide chunk of the bf16 parts reads as zero
    for (int i = tid; i < 2 * 2 * BC * LP_S; i += kThreads) {
        const int b = i / (2 * BC * LP_S), r = i - b * 2 * BC * LP_S, row = (r / LP_S) % BC, col = r % LP_S;
        PK[b][r] = r < BC * LP_S && col == row ? 1.f : 0.f;
    }
    if constexpr (DK < 32)
        for (int i = tid; i < 2 * 2 * XSB; i += kThreads) (&XS[0][0][0])[i] = (__bf16)0.f;
    lds_barrier();

    // one chunk: stage it from its register set, which then loads the chunk two ahead
    auto step = [&](int jc, ChunkRegs &r) {
        const int buf = jc & 1;
        stage_chunk(buf, r);
        lds_barrier();
        // (every wave computes: with fewer tiles than waves, CT < 4, the waves past the last
        // tile repeat tile CT - 1's arithmetic and write the same values; no branch, so that the
        // products, the loads and the update share one scheduling region)
        v4f ks = {0.f, 0.f, 0.f, 0.f}, qs = ks;
        {
            // [K; Q] S: per 32-wide chunk m of d_k, the state tile's rows split into bf16 hi /
            // lo parts in registers, against the staged parts of the rows
            const __bf16 *xh = XS[buf][0];
#pragma unroll
            for (int m = 0; m < KM; ++m) {
                const v4f s1 = 2 * m + 1 < KC ? sreg[min(2 * m + 1, KC - 1)] : v4f{0.f, 0.f, 0.f, 0.f};
                const float x[8] = {sreg[2 * m][0], sreg[2 * m][1], sreg[2 * m][2], sreg[2 * m][3],
                                    s1[0],          s1[1],          s1[2],          s1[3]};
                __bf16 bh[8], bl[8];
                split_bf16(x, bh, bl);
                const bf8 vbh = {bh[0], bh[1], bh[2], bh[3], bh[4], bh[5], bh[6], bh[7]};
                const bf8 vbl = {bl[0], bl[1], bl[2], bl[3], bl[4], bl[5], bl[6], bl[7]};
#pragma unroll
                for (int rt = 0; rt < 2; ++rt) {  // q rows, k rows
                    const int off = (BC * rt + l16) * SXB + 32 * m + 8 * g4;
                    const bf8 ah = *reinterpret_cast<const bf8 *>(xh + off);
                    const bf8 al = *reinterpret_cast<const bf8 *>(xh + XSB + off);
                    v4f &acc = rt ? ks : qs;
                    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al, vbh, acc, 0, 0, 0);
                    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, vbl, acc, 0, 0, 0);
                    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, vbh, acc, 0, 0, 0);
                }
            }
        }
        {
            // the package operands and the values
            const float *Pb = PK[buf], *Vb = VZ[buf][0], *Zb = VZ[buf][1];
            const v4f tf = *reinterpret_cast<const v4f *>(Pb + LP_T + l16 * LP_S + 4 * g4);
            const v4f cf = *reinterpret_cast<const v4f *>(Pb + LP_CQ + l16 * LP_S + 4 * g4);
            const v4f pa = *reinterpret_cast<const v4f *>(Pb + LP_V + 4 * g4);
            const v4f pb = *reinterpret_cast<const v4f *>(Pb + LP_V + BC + 4 * g4);
            const v4f pc = *reinterpret_cast<const v4f *>(Pb + LP_V + 2 * BC + 4 * g4);
            const v4f pw = *reinterpret_cast<const v4f *>(Pb + LP_V + 3 * BC + 4 * g4);
            const float gp = Pb[LP_G], gend = jc < nch ? gp : 1.f;  // (past the last chunk: S unchanged)
            // D = T rhs, O = diag(c) QS + Cq D, the gate; outputs of padding tokens are dropped
            // at the store
            v4f rhs, o, bw;
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                rhs[v] = pa[v] * (Vb[(4 * g4 + v) * VW + 16 * cw + l16] - pb[v] * ks[v]);
                o[v] = pc[v] * qs[v];
            }
            const v4f dl = mfma4(tf, rhs, v4f{0.f, 0.f, 0.f, 0.f});
            o = mfma4(cf, dl, o);
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                if constexpr (GATED) {
                    const float zz = Zb[(4 * g4 + v) * VW + 16 * cw + l16];
                    const float sg = fast_sigmoid(zz);
                    o[v] *= gate_mode == 0 ? zz * sg : sg;  // silu(z) = z sigmoid(z)
                }
                // (the element goes through a scalar: this compiler's __builtin_bit_cast of a vector
                // element lvalue reads element 0 whatever the index)
                const float ov = o[v];
                OT[buf][(4 * g4 + v) * JB + 16 * cw + l16] = ov;
                bw[v] = pw[v] * dl[v];
            }
            // S <- G_B S + K^T diag(w) D, tile by tile of 16 d_k rows, in three bf16 products
            // over 32 slots: lane group g supplies tokens 4g .. 4g + 3 twice, in two parts each,
            // so that with K^T = Kh + Km + Kl and diag(w) D = Bh + Bm + Bl the products
            // [Kh | Km] [Bh; Bh], [Kh | Km] [Bm; Bm] and [Kl | Kh] [Bh; Bl] sum the six terms that
            // matter (all but those below 2^-24 of the product).  The loads of the chunk two
            // ahead and the previous chunk's output store are spread between the products
            // (issued in a cluster they stall the wave on the address unit).
            unsigned bh[2], bm[2], bl[2];
            {
                const float bwa[4] = {bw[0], bw[1], bw[2], bw[3]};
                split3_bf16(bwa, bh, bm, bl);
            }
            const bf8 b1 = __builtin_bit_cast(bf8, v4u{bh[0], bh[1], bh[0], bh[1]});
            const bf8 b2 = __builtin_bit_cast(bf8, v4u{bm[0], bm[1], bm[0], bm[1]});
            const bf8 b3 = __builtin_bit_cast(bf8, v4u{bh[0], bh[1], bl[0], bl[1]});
            __builtin_amdgcn_sched_barrier(0);  // the update and the memory operations in a region of their own
            load_chunk(r, jc + 2);
            store_outputs(jc - 1);  // complete since the barrier
            bf8 a1[KC], a2[KC];
#pragma unroll
            for (int rt = 0; rt < KC; ++rt) {
                const int row = 16 * rt + l16, at = row * KAS + 8 * (g4 ^ ((row >> KSW) & 3));
                a1[rt] = *reinterpret_cast<const bf8 *>(KA[buf] + at);
                a2[rt] = *reinterpret_cast<const bf8 *>(KB[buf] + at);
            }
#pragma unroll
            for (int rt = 0; rt < KC; ++rt) {
                v4f acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a2[rt], b3, gend * sreg[rt], 0, 0, 0);
                acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1[rt], b2, acc, 0, 0, 0);
                sreg[rt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1[rt], b1, acc, 0, 0, 0);
            }
            // the operand reads of tiles 0 and 1 first; then per tile its three products, the
            // reads of the tile two ahead and a share of the loads and the store
            constexpr int kVmem = 4 * KPT + QPT + 4;  // loads and the store of one step
            constexpr int kAhead = KC < 2 ? KC : 2;
            __builtin_amdgcn_sched_group_barrier(0x100, 2 * kAhead + 1, 0);  // (+ the output row read)
#pragma unroll
            for (int rt = 0; rt < KC; ++rt) {
                __builtin_amdgcn_sched_group_barrier(0x008, 3, 0);
                if (rt + kAhead < KC) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
                __builtin_amdgcn_sched_group_barrier(0x010, 1, 0);
            }
            if constexpr (kVmem > KC) __builtin_amdgcn_sched_group_barrier(0x010, kVmem > KC ? kVmem - KC : 1, 0);
        }
    };
    // the state tile and the first two chunks are in before the loop: a load still pending at
    // the loop's entry would have the compiler wait for every younger load in each iteration
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0), lgkmcnt and expcnt left open
    // Steps in pairs, with no branch between them (a conditional step would have the compiler
    // wait for every pending load at the loop's head): an odd count ends with a step past the
    // last chunk, whose buffers are zero (beta = 0, so D = 0) and whose decay is taken as 1,
    // so it leaves the state as it is and stores nothing.
    for (int jc = 0; jc < nch; jc += 2) {
        step(jc, ra);
        step(jc + 1, rb);
    }

    lds_barrier();
    store_outputs(((nch + 1) & ~1) - 1);  // the last step's outputs (none past the last chunk)

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
                  const int32_t *slot_ids, const float *gate_z, int gate_mode, float *out, float *workspace,
                  int32_t *status, hipStream_t stream) {
    const int nch = (T + BC - 1) / BC;
    hipLaunchKernelGGL((prefill_prep_kernel<DK>), dim3(nch * d.Hk, d.C), dim3(kThreads), 0, stream, d, T, qkv,
                       beta_logits, alpha_logits, gate_stride, dt_bias, A, workspace);
    if (hipError_t e = hipGetLastError(); e != hipSuccess) return e;
    const dim3 grid(PrefillCfg<DK, DV>::NB * d.Hv * d.C);
    if (gate_z)
        hipLaunchKernelGGL((prefill_state_kernel<DK, DV, true>), grid, dim3(kThreads), 0, stream, d, T, qkv, workspace,
                           state_pool, slot_ids, gate_z, gate_mode, out, status);
    else
        hipLaunchKernelGGL((prefill_state_kernel<DK, DV, false>), grid, dim3(kThreads), 0, stream, d, T, qkv,
                           workspace, state_pool, slot_ids, gate_z, gate_mode, out, status);
    return hipGetLastError();
}

}  // namespace

// Workspace of gdn_prefill_noalloc: a file-scope device array, one copy per GPU the library's
// code object is loaded on, held until the process ends.  On the host the array's name is a
// stand-in, not a device address: kernels get each device's address from hipGetSymbolAddress.
static __device__ __align__(256) float scratch[kStaticScratchFloats];

hipError_t static_scratch(hipStream_t stream, float **ptr) {
    constexpr int kMaxDevices = 64;
    static std::mutex mu;
    static float *addr[kMaxDevices] = {};
    int cur = 0;
    if (hipError_t e = hipGetDevice(&cur); e != hipSuccess) return e;
    int dev = cur;  // the device the launches go to: the stream's, or the current one
    if (stream)
        if (hipError_t e = hipStreamGetDevice(stream, &dev); e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(mu);
    if (!addr[dev]) {  // once per device, with that device current
        if (dev != cur)
            if (hipError_t e = hipSetDevice(dev); e != hipSuccess) return e;
        void *p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (dev != cur) (void)hipSetDevice(cur);
        if (e != hipSuccess) return e;
        addr[dev] = static_cast<float *>(p);
    }
    *ptr = addr[dev];
    return hipSuccess;
}

hipError_t launch_prefill(const Dims &d, int n_tokens, const float *qkv, const float *beta_logits,
                          const float *alpha_logits, int64_t gate_stride, const float *dt_bias, const float *A,
                          float *state_pool, const int32_t *slot_ids, const float *gate_z, int gate_mode, float *out,
                          float *workspace, int32_t *status, hipStream_t stream) {
#define GDN_PREFILL_CASE(K, V)                                                                                  \
    if (d.dk == K && d.dv == V)                                                                                 \
        return launch<K, V>(d, n_tokens, qkv, beta_logits, alpha_logits, gate_stride, dt_bias, A, state_pool, \
                            slot_ids, gate_z, gate_mode, out, workspace, status, stream);
#define GDN_PREFILL_ROW(K) GDN_PREFILL_CASE(K, 16) GDN_PREFILL_CASE(K, 32) GDN_PREFILL_CASE(K, 64) GDN_PREFILL_CASE(K, 128)
    GDN_PREFILL_ROW(16) GDN_PREFILL_ROW(32) GDN_PREFILL_ROW(64) GDN_PREFILL_ROW(128)
#undef GDN_PREFILL_ROW
#undef GDN_PREFILL_CASE
    return hipErrorInvalidValue;
}

}  // namespace gdn
