// Read-only slot-mapped tree verify for gfx950: the gated delta rule over each lane's
// draft tree with the gates applied in-kernel, writing the attention output and the
// replay log and never the state.
//
// What is computed: "perf(qwen35): fuse the DFlash2 concurrent verify Gated DeltaNet
// route", Optimizations, second and third bullets; gates from "qwen35: DSpark
// speculative decoding", raw-gate commit message; log row width 1 + d_k + d_v from
// "perf(qwen38): various DFlash2 optimizations concurrency C1-C5", Summary item 3.
//
// Formulation.  Unrolling the recurrence along a node's root path, with G_i the product
// of the decays on path(i), gives S_i = G_i S0 + sum_{a on path(i)} (G_i/G_a) k^_a d_a^T.
// For value column j this yields a triangular system over the tree
//   d_i = beta_i (v_i - G_i k^_i.S0 - sum_{a strict ancestor} (G_i/G_a)(k^_a.k^_i) d_a)
//   o_i = (G_i q^_i.S0 + sum_{a on path(i)} (G_i/G_a)(k^_a.q^_i) d_a) / sqrt(d_k).
// With Ck[a][i] = (G_i/G_a) k^_a.k^_i on strict ancestors, Cq[a][i] = (G_i/G_a) k^_a.q^_i
// on the path, T = (I + diag(beta) Ck^T)^-1, M1 = T diag(beta):
//   d = M1 V - K' S0,                 K' = T diag(beta G) K^
//   o = (Q' S0 + W V) / sqrt(d_k),    Q' = diag(G) Q^ - Cq^T K',  W = Cq^T M1.
// Everything but the slot's state S0 is known before S0 arrives, so a workgroup first
// builds the (2N) x (d_k + N) matrix A = [[-K', M1], [Q'/sqrt(d_k), W/sqrt(d_k)]] from
// q, k, gates and the tree while its S0 block is in flight, then one MFMA product
// A x [S0; V] yields the delta rows (replay log) and output rows directly from the
// accumulators.  Per-node states are never formed and S0 is read once.  q and k are
// never normalised explicitly: their norms come from the diagonal of the Gram product
// and fold into the coefficients.  Decay ratios are exp(L_i - L_a) of cumulative
// log-decays, which cannot overflow.
//
// Mapping: one workgroup (4 waves) per (lane, value head, block of 32 value columns);
// products run on v_mfma_f32_16x16x4_f32 from LDS.  N is padded to NP (16 or 32) with
// zero rows.  Barriers wait only for LDS traffic, so the state block requested at the
// start stays in flight through the whole tree phase.  Workgroup ids are ordered so that
// the workgroups sharing one (lane, q/k head) are congruent modulo the number of such
// groups: with round-robin dispatch over the 8 XCDs they land on one XCD and read the
// shared q/k rows through its L2.
//
// Fused route (conv + verify, "perf(qwen35): fuse the DFlash2 concurrent verify Gated
// DeltaNet route", Optimizations): the workgroup reads the raw projected tokens x of its
// q/k slab and value block, stages them in LDS, and computes the tree conv + SiLU of its
// channels in registers (sources of node i, oldest first: the tokens of i's nearest
// ancestors, then the slot's history columns), writing the results straight into the
// product operands; the conv output never goes to memory.  The commit windows are
// written once: value channels by their owning workgroup, the q/k channels split evenly
// over the workgroups that share them.
#include "gdn_internal.h"

namespace gdn {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;

typedef float v4f __attribute__((ext_vector_type(4)));

// Workgroup barrier for LDS communication only: waits for this wave's LDS operations,
// not for its outstanding global loads, so prefetched data keeps streaming in.
__device__ inline void lds_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0), vmcnt and expcnt left open
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

template <int DK, int DV, int NP, bool FUSED>
struct VerifyLayout {
    static constexpr int JB = DV < 32 ? DV : 32;  // value columns per workgroup
    static constexpr int NB = DV / JB;            // column blocks per head
    static constexpr int R = 1 + DK + DV;         // replay-log row
    static constexpr int KA = DK + NP;            // contraction length of the main product
    // row strides (floats) are 4 mod 8 so 16 rows read with ds_read_b128 hit distinct banks
    static constexpr int SA = (KA + 7) / 8 * 8 + 4;  // A: [2NP][SA]
    static constexpr int SBT = SA;                   // [S0; V] transposed: [JB][SBT]
    static constexpr int SG = NP + 4;                // small matrices
    static constexpr int OFF_CQ = 2 * NP * SA;       // Cq^T [NP][SG] (own region)
    static constexpr int OFF_X = OFF_CQ + NP * SG;   // late: [S0; V]^T; early aliases:
    static constexpr int OFF_G = OFF_X;              //   Gram [2NP][SG]
    static constexpr int OFF_CK = OFF_G + 2 * NP * SG;  // Ck^T [NP][SG]
    static constexpr int OFF_MK = OFF_CK + NP * SG;     // -T diag(beta G / |k|) [NP][SG]
    static constexpr int X_FLOATS = (JB * SBT > 4 * NP * SG) ? JB * SBT : 4 * NP * SG;
    // fused route: raw token rows [NP][SX] (q|k slab, then the value block) staged over
    // the Cq / late region, which is free until the coefficients are formed
    static constexpr int SX = 2 * DK + JB;
    static constexpr int OFF_STG = OFF_CQ;
    static constexpr int STAGE = FUSED ? NP * SX : 0;
    static constexpr int TAIL = NP * SG + X_FLOATS;
    static constexpr int LDS_FLOATS = OFF_CQ + (TAIL > STAGE ? TAIL : STAGE);
};

// One 16x16 tile of A[m0.., 0:K] x B[0:K, n0..] with both operands k-contiguous:
// A(m, k) = A[m*AM + k], B(k, n) = B[n*BN + k].  Each 16-wide k chunk is read with one
// ds_read_b128 per operand; lane group g = l/16 supplies k = k0 + 4g + s in MFMA step s,
// a permutation of the contraction index shared by both operands.  Lane l receives
// rows 4*(l/16) + v (v = 0..3) of column l % 16.
template <int K, int AM, int BN>
__device__ inline v4f mma_kc(const float *A, const float *B) {
    const int l = threadIdx.x & 63;
    const float *a = A + (l & 15) * AM + 4 * (l >> 4);
    const float *b = B + (l & 15) * BN + 4 * (l >> 4);
    v4f acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int k0 = 0; k0 < K; k0 += 16) {
        const v4f av = *reinterpret_cast<const v4f *>(a + k0);
        const v4f bv = *reinterpret_cast<const v4f *>(b + k0);
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(av[0], bv[0], acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(av[1], bv[1], acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(av[2], bv[2], acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(av[3], bv[3], acc, 0, 0, 0);
    }
    return acc;
}

// Same tile with A k-contiguous and B row-major in k: B(k, n) = B[k*BK + n].
template <int K, int AM, int BK>
__device__ inline v4f mma_kr(const float *A, const float *B) {
    const int l = threadIdx.x & 63;
    const float *a = A + (l & 15) * AM + (l >> 4);
    const float *b = B + (l >> 4) * BK + (l & 15);
    v4f acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int k0 = 0; k0 < K; k0 += 4) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[k0], b[k0 * BK], acc, 0, 0, 0);
    return acc;
}

// 1 / max(|x|, 1e-6) from |x|^2, and the gate nonlinearities, on the hardware
// transcendental units (about 1 ulp each; the outputs carry a 2e-4 tolerance)
__device__ inline float inv_norm(float sq) { return fminf(__builtin_amdgcn_rsqf(sq), 1e6f); }
__device__ inline float fast_exp(float x) { return __builtin_amdgcn_exp2f(x * 1.4426950408889634f); }
__device__ inline float fast_softplus(float x) {
    return fmaxf(x, 0.f) + 0.6931471805599453f * __builtin_amdgcn_logf(1.0f + fast_exp(-fabsf(x)));
}
__device__ inline float fast_sigmoid(float x) { return __builtin_amdgcn_rcpf(1.0f + fast_exp(-x)); }
__device__ inline float fast_silu(float z) { return z * __builtin_amdgcn_rcpf(1.0f + fast_exp(-z)); }

// Tree conv + SiLU of 4 channels at one node.  xi: the node's own tokens; X(n): tokens of
// node n from the staged rows; hc[j]: history column j (2 = newest); w[e]: the 4 taps of
// channel e (tap 0 = oldest).  n1..n3 are the node's parent, grandparent and
// great-grandparent (-1 past the root).  Returns silu(conv) and the 3 newest sources
// (t1, t2, t3 = the node itself), which form the node's commit window.
__device__ inline v4f conv_node(v4f xi, const float *stg, int sx, int n1, int n2, int n3, const v4f hc[3],
                                const v4f w[4], v4f &t1, v4f &t2) {
    const v4f x1 = *reinterpret_cast<const v4f *>(stg + (n1 > 0 ? n1 : 0) * sx);
    const v4f x2 = *reinterpret_cast<const v4f *>(stg + (n2 > 0 ? n2 : 0) * sx);
    const v4f x3 = *reinterpret_cast<const v4f *>(stg + (n3 > 0 ? n3 : 0) * sx);
    t2 = n1 >= 0 ? x1 : hc[2];
    t1 = n1 >= 0 ? (n2 >= 0 ? x2 : hc[2]) : hc[1];
    const v4f t0 = n1 >= 0 ? (n2 >= 0 ? (n3 >= 0 ? x3 : hc[2]) : hc[1]) : hc[0];
    v4f y;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        float z = t0[e] * w[e][0];  // taps summed from the oldest column
        z = fmaf(t1[e], w[e][1], z);
        z = fmaf(t2[e], w[e][2], z);
        z = fmaf(xi[e], w[e][3], z);
        y[e] = fast_silu(z);
    }
    return y;
}

// window of 4 channels in the history layout [ch][3]: 12 consecutive floats
__device__ inline void store_window(float *dst, v4f t1, v4f t2, v4f t3) {
    v4f *w = reinterpret_cast<v4f *>(dst);
    w[0] = v4f{t1.x, t2.x, t3.x, t1.y};
    w[1] = v4f{t2.y, t3.y, t1.z, t2.z};
    w[2] = v4f{t3.z, t1.w, t2.w, t3.w};
}

// history columns of 4 channels from their 12 consecutive floats
__device__ inline void hist_columns(const float *src, v4f hc[3]) {
    const v4f *p = reinterpret_cast<const v4f *>(src);
    const v4f a = p[0], b = p[1], e = p[2];  // ch0: a.x a.y a.z | ch1: a.w b.x b.y | ch2: b.z b.w e.x | ch3: e.y e.z e.w
    hc[0] = v4f{a.x, a.w, b.z, e.y};
    hc[1] = v4f{a.y, b.x, b.w, e.z};
    hc[2] = v4f{a.z, b.y, e.x, e.w};
}

template <int DK, int DV, int NP, bool FUSED>
__device__ __forceinline__ void verify_body(const VerifyArgs &args) {
    using Ly = VerifyLayout<DK, DV, NP, FUSED>;
    constexpr int JB = Ly::JB, NB = Ly::NB, R = Ly::R, KA = Ly::KA, SA = Ly::SA, SBT = Ly::SBT, SG = Ly::SG;
    constexpr int Q4 = JB / 4;  // 4-float groups per block row
    extern __shared__ float lds[];
    float *Am = lds;                // A: rows 0..NP-1 delta rows, NP..2NP-1 output rows
    float *CqT = lds + Ly::OFF_CQ;  // Cq^T[i][a]
    float *BmT = lds + Ly::OFF_X;   // [S0 block; V block]^T, written last
    float *Gm = lds + Ly::OFF_G;    // early aliases of the [S0; V] region
    float *CkT = lds + Ly::OFF_CK;
    float *Mk = lds + Ly::OFF_MK;
    __shared__ int s_wbits[kWaves];
    __shared__ float s_beta[NP], s_g[NP], s_L[NP], s_G[NP], s_rk[NP], s_rq[NP], s_gq[NP];
    __shared__ unsigned int s_anc[NP];

    const Dims d = args.d;
    const float *__restrict__ state_pool = args.state_pool;
    const int32_t *__restrict__ slot_ids = args.slot_ids;
    float *__restrict__ out = args.out;
    float *__restrict__ replay_log = args.replay_log;
    const int N = d.N, Hv = d.Hv;
    // workgroup -> (lane c, q/k head kh, share index ws); ws -> (value head h, column block jb)
    const int n_groups = d.C * d.Hk;
    const int grp = blockIdx.x % n_groups, ws = blockIdx.x / n_groups;
    const int c = grp / d.Hk, kh = grp - c * d.Hk;
    const int jb = ws % NB, h = kh + d.Hk * (ws / NB);
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int j0 = jb * JB;

    // ---- loads, in the order they are consumed (global loads complete in order): tree
    //      and gates, duplicate-slot check, q/k (raw tokens when fused), the V block, then
    //      the state block.  Indices are clamped and out-of-range values selected to zero,
    //      so every load is unconditional and all of them are in flight together.
    const int par = args.parents[(int64_t)c * N + (lane < N ? lane : 0)];  // lane i of every wave: parent of node i
    const int tn = tid < N ? tid : 0;
    const int64_t trow = (int64_t)c * N + tn;
    const float braw = args.beta_logits[trow * args.gate_stride + h];
    const float araw = args.alpha_logits[trow * args.gate_stride + h] + args.dt_bias[h];
    const float Ah = args.A[h];
    const int so = slot_ids[tid < d.C ? tid : 0];  // this thread's share of the duplicate check
    const int s = slot_ids[c];

    // separate route: conv output rows; fused route: raw token rows of the same channels
    constexpr int G = DK / 2;  // 4-channel groups of one head's q|k slab (kThreads % G == 0)
    constexpr int QI = (G * NP + kThreads - 1) / kThreads;
    constexpr int QF4 = 2 * NP * (DK / 4), QPT = FUSED ? QI : (QF4 + kThreads - 1) / kThreads;
    const int gq = tid % G;
    const int chq = gq < DK / 4 ? kh * DK + 4 * gq : d.Hk * DK + kh * DK + 4 * (gq - DK / 4);
    v4f qreg[QPT];  // separate: row r < NP k of node r, NP + i q of node i; fused: x of (node, gq)
#pragma unroll
    for (int u = 0; u < QPT; ++u) {
        if constexpr (FUSED) {
            const int i = min((tid + kThreads * u) / G, NP - 1);
            const v4f x = reinterpret_cast<const v4f *>(args.x + ((int64_t)c * N + (i < N ? i : 0)) * d.Ch + chq)[0];
            qreg[u] = i < N ? x : v4f{0.f, 0.f, 0.f, 0.f};
        } else {
            const int f = min(tid + kThreads * u, QF4 - 1), r = f / (DK / 4), q = f - r * (DK / 4);
            const int i = r < NP ? r : r - NP;
            const float *src =
                args.qkv + ((int64_t)c * N + (i < N ? i : 0)) * d.Ch + (r < NP ? d.Hk * DK : 0) + kh * DK;
            const v4f x = reinterpret_cast<const v4f *>(src)[q];
            qreg[u] = i < N ? x : v4f{0.f, 0.f, 0.f, 0.f};
        }
    }
    // V block: this thread's 4-column group gv is fixed (kThreads % Q4 == 0); surplus
    // items are clamped to the last row, so their duplicate writes carry the same value
    constexpr int VF4 = NP * Q4, VPT = (VF4 + kThreads - 1) / kThreads;
    const int gv = tid % Q4;
    const int chv = 2 * d.Hk * DK + h * DV + j0 + 4 * gv;
    const float *vsrc = FUSED ? args.x : args.qkv;
    v4f vreg[VPT];
#pragma unroll
    for (int u = 0; u < VPT; ++u) {
        const int i = min((tid + kThreads * u) / Q4, NP - 1);
        const v4f x = reinterpret_cast<const v4f *>(vsrc + ((int64_t)c * N + (i < N ? i : 0)) * d.Ch + chv)[0];
        vreg[u] = i < N ? x : v4f{0.f, 0.f, 0.f, 0.f};
    }
    // fused: the taps of this thread's q/k and value channel groups
    v4f wq[4], wv[4];
    if constexpr (FUSED) {
        const v4f *w4 = reinterpret_cast<const v4f *>(args.conv_w);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            wq[e] = w4[chq + e];
            wv[e] = w4[chv + e];
        }
    }
    if (s == -1) return;  // padding lane
    const bool s_ok = s >= 0 && s < d.P;
    const int sc = s_ok ? s : 0;
    v4f hq[3], hv[3];  // fused: history columns of the two channel groups
    if constexpr (FUSED) {
        hist_columns(args.conv_hist + ((int64_t)sc * d.Ch + chq) * 3, hq);
        hist_columns(args.conv_hist + ((int64_t)sc * d.Ch + chv) * 3, hv);
    }
    constexpr int SF4 = DK * Q4, SPT = (SF4 + kThreads - 1) / kThreads;
    v4f sreg[SPT];
    {
        const float *Sg = state_pool + ((int64_t)sc * Hv + h) * DK * DV + j0;
#pragma unroll
        for (int u = 0; u < SPT; ++u) {
            const int f = min(tid + kThreads * u, SF4 - 1), r = f / Q4, q = f - r * Q4;
            sreg[u] = reinterpret_cast<const v4f *>(Sg + (int64_t)r * DV)[q];
        }
    }

    // ---- lane validity (slot range, duplicate slot, parents); nothing is written for a bad lane
    int bits = s_ok ? 0 : GDN_STATUS_SLOT_RANGE;
    if (tid < d.C && tid != c && so == s) bits |= GDN_STATUS_SLOT_DUP;
    for (int o = tid + kThreads; o < d.C; o += kThreads)  // lanes beyond the first 256
        if (o != c && slot_ids[o] == s) bits |= GDN_STATUS_SLOT_DUP;
    if (tid < N && (par < -1 || par >= tid)) bits |= GDN_STATUS_PARENT;
    {
        int wb = 0;
#pragma unroll
        for (int b = 0; b < 3; ++b)
            if (__builtin_amdgcn_ballot_w64((bits >> b) & 1)) wb |= 1 << b;
        if (lane == 0) s_wbits[wave] = wb;
    }
    float *stg = lds + Ly::OFF_STG;  // fused: staged token rows [NP][SX]
    if constexpr (FUSED) {
#pragma unroll
        for (int u = 0; u < QPT; ++u) {
            const int f = tid + kThreads * u;
            if (f < G * NP) *reinterpret_cast<v4f *>(stg + (f / G) * Ly::SX + 4 * gq) = qreg[u];
        }
#pragma unroll
        for (int u = 0; u < VPT; ++u) {
            const int f = tid + kThreads * u;
            if (f < VF4) *reinterpret_cast<v4f *>(stg + (f / Q4) * Ly::SX + 2 * DK + 4 * gv) = vreg[u];
        }
    } else {
        // conv rows into A (k rows 0..NP-1, q rows NP..2NP-1)
#pragma unroll
        for (int u = 0; u < QPT; ++u) {
            const int f = min(tid + kThreads * u, QF4 - 1), r = f / (DK / 4), q = f - r * (DK / 4);
            *reinterpret_cast<v4f *>(Am + r * SA + 4 * q) = qreg[u];
        }
    }
    lds_barrier();
    {
        int all = 0;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) all |= s_wbits[w];
        if (all) {
            if (ws == 0 && tid == 0 && args.status) atomicOr(args.status, all);
            return;
        }
    }

    // ---- tree, wave 0: cumulative log-decay L_i and ancestor set by pointer jumping
    //      (log2(NP) rounds of lane shuffles, independent of the tree depth)
    if (wave == 0) {
        const bool real = lane < N;
        int jump = real ? par : -1;
        float L = 0.f;
        if (real) L = fast_softplus(araw) * Ah;  // log g = softplus(a + dt_bias) * A
        if (lane < NP) s_g[lane] = fast_exp(L);
        unsigned int anc = real ? 1u << lane : 0u;
#pragma unroll
        for (int r = 1; r < NP; r <<= 1) {
            const int src = jump < 0 ? lane : jump;
            const float Lj = __shfl(L, src);
            const unsigned int aj = __shfl(anc, src);
            const int jj = __shfl(jump, src);
            if (jump >= 0) {
                L += Lj;
                anc |= aj;
                jump = jj;
            }
        }
        if (lane < NP) {
            s_L[lane] = L;
            s_G[lane] = real ? fast_exp(L) : 0.f;
            s_anc[lane] = anc;
            s_beta[lane] = real ? fast_sigmoid(braw) : 0.f;
        }
    }
    // ---- fused: tree conv + SiLU of the block's channels from the staged rows, into the
    //      q/k rows of A and the V registers; commit windows of the owned channels
    if constexpr (FUSED) {
        // lane i of every wave: parent, grandparent and great-grandparent of node i
        const int a1 = lane < N ? par : -1;
        const int a2s = __shfl(a1, a1 >= 0 ? a1 : 0);
        const int a2 = a1 >= 0 ? a2s : -1;
        const int a3s = __shfl(a2, a1 >= 0 ? a1 : 0);
        const int a3 = a1 >= 0 ? a3s : -1;
        const int n_share = NB * (Hv / d.Hk);
        const bool own_q = (gq * n_share) / G == ws;  // the q/k windows of group gq are written here
        float *win = args.commit_win + (int64_t)c * N * d.Ch * 3;
        const v4f zero = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int u = 0; u < QPT; ++u) {
            const int f = tid + kThreads * u, i = min(f / G, NP - 1);
            const int n1 = __shfl(a1, i), n2 = __shfl(a2, i), n3 = __shfl(a3, i);
            v4f t1, t2;
            const v4f y = conv_node(qreg[u], stg + 4 * gq, Ly::SX, n1, n2, n3, hq, wq, t1, t2);
            if (f < G * NP) {
                const int row = gq < DK / 4 ? NP + i : i, col = 4 * (gq < DK / 4 ? gq : gq - DK / 4);
                *reinterpret_cast<v4f *>(Am + row * SA + col) = i < N ? y : zero;
                if (own_q && i < N) store_window(win + ((int64_t)i * d.Ch + chq) * 3, t1, t2, qreg[u]);
            }
        }
#pragma unroll
        for (int u = 0; u < VPT; ++u) {
            const int f = tid + kThreads * u, i = min(f / Q4, NP - 1);
            const int n1 = __shfl(a1, i), n2 = __shfl(a2, i), n3 = __shfl(a3, i);
            v4f t1, t2;
            const v4f y = conv_node(vreg[u], stg + 2 * DK + 4 * gv, Ly::SX, n1, n2, n3, hv, wv, t1, t2);
            if (f < VF4 && i < N) store_window(win + ((int64_t)i * d.Ch + chv) * 3, t1, t2, vreg[u]);
            vreg[u] = i < N ? y : zero;
        }
        lds_barrier();
    }

    // ---- Gram of the raw vectors: Gm[r][a] = (row r of A) . k_a; the diagonal tiles of
    //      Q Q^T give |q_i|^2
    {
        constexpr int NT = NP / 16, TG = 2 * NP / 16 * NT, TQ = NP / 16;
        for (int t = wave; t < TG + TQ; t += kWaves) {
            if (t < TG) {
                const int mt = t / NT, nt = t - mt * NT;
                const v4f acc = mma_kc<DK, SA, SA>(Am + mt * 16 * SA, Am + nt * 16 * SA);
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    Gm[(mt * 16 + 4 * (lane >> 4) + v) * SG + nt * 16 + (lane & 15)] = acc[v];
                    if (mt == nt && 4 * (lane >> 4) + v == (lane & 15)) s_rk[mt * 16 + (lane & 15)] = inv_norm(acc[v]);
                }
            } else {
                const int qt = t - TG;
                const float *Qb = Am + (NP + qt * 16) * SA;
                const v4f acc = mma_kc<DK, SA, SA>(Qb, Qb);
#pragma unroll
                for (int v = 0; v < 4; ++v)
                    if (4 * (lane >> 4) + v == (lane & 15)) s_rq[qt * 16 + (lane & 15)] = inv_norm(acc[v]);
            }
        }
    }
    lds_barrier();

    // ---- decayed, ancestor-masked, norm-scaled coefficients (stored transposed) and the
    //      replay-log header (g, k^) of every node, once per (lane, head)
    //      (CkT[i][a] carries beta_i: it is the strictly lower matrix of the solve below)
    for (int p = tid; p < NP * NP; p += kThreads) {
        const int i = p / NP, a = p - i * NP;
        const bool on = (s_anc[i] >> a) & 1u;
        const float r = on ? fast_exp(s_L[i] - s_L[a]) * s_rk[a] : 0.f;
        CkT[i * SG + a] = (on && a < i) ? r * Gm[a * SG + i] * (s_rk[i] * s_beta[i]) : 0.f;
        CqT[i * SG + a] = on ? r * Gm[(NP + i) * SG + a] * s_rq[i] : 0.f;
    }
    if (tid < NP) s_gq[tid] = s_G[tid] * s_rq[tid];
    if (jb == 0) {
        float *logc = replay_log + ((int64_t)c * N * Hv + h) * R;
        for (int f = tid; f < N * DK; f += kThreads) {
            const int i = f / DK, e = f - i * DK;
            float *lrow = logc + (int64_t)i * Hv * R;
            lrow[1 + e] = Am[i * SA + e] * s_rk[i];
            if (e == 0) lrow[0] = s_g[i];
        }
    }
    lds_barrier();

    // ---- T = (I + diag(beta) Ck^T)^-1 by forward substitution, one column per thread;
    //      M1 = T diag(beta) goes into A (rows 0..NP-1, columns DK..),
    //      Mk = -T diag(beta G / |k|) multiplies the raw k rows
    if (tid < NP) {
        const int a = tid;
        float t[NP];
        // row i of the solve matrix is read (i / 4 + 1 four-float groups) while row i - 1
        // is being solved, so each row costs its FMA chain rather than an LDS round trip
        v4f cur[NP / 4], nxt[NP / 4];
        cur[0] = *reinterpret_cast<const v4f *>(CkT);
#pragma unroll
        for (int i = 0; i < NP; ++i) {
            if (i + 1 < NP)
#pragma unroll
                for (int m4 = 0; m4 <= (i + 1) / 4; ++m4)
                    nxt[m4] = *reinterpret_cast<const v4f *>(CkT + (i + 1) * SG + 4 * m4);
            float s0 = 0.f, s1 = 0.f;
#pragma unroll
            for (int m = 0; m < i; ++m) {
                if (m & 1) s1 = fmaf(cur[m / 4][m % 4], t[m], s1);
                else s0 = fmaf(cur[m / 4][m % 4], t[m], s0);
            }
            t[i] = i < a ? 0.f : (i == a ? 1.f : -(s0 + s1));
#pragma unroll
            for (int m4 = 0; m4 < NP / 4; ++m4) cur[m4] = nxt[m4];
        }
        const float ba = s_beta[a], ga = ba * s_G[a] * s_rk[a];
#pragma unroll
        for (int i = 0; i < NP; ++i) {
            Am[i * SA + DK + a] = t[i] * ba;
            Mk[i * SG + a] = -t[i] * ga;
        }
    }
    lds_barrier();

    const float isd = 1.0f / sqrtf((float)DK);
    // ---- -K' = Mk K (in place over the k rows once every tile has read them) and
    //      W / sqrt(d_k) = Cq^T M1 / sqrt(d_k) (rows NP.., columns DK.. of A)
    {
        constexpr int NTK = DK / 16, TK = NP / 16 * NTK, TKW = (TK + kWaves - 1) / kWaves;
        v4f kacc[TKW];
#pragma unroll
        for (int u = 0; u < TKW; ++u) {
            const int t = wave + kWaves * u;
            if (t < TK) {
                const int mt = t / NTK, nt = t - mt * NTK;
                kacc[u] = mma_kr<NP, SG, SA>(Mk + mt * 16 * SG, Am + nt * 16);
            }
        }
        constexpr int NTW = NP / 16;
        for (int t = wave; t < NTW * NTW; t += kWaves) {
            const int mt = t / NTW, nt = t - mt * NTW;
            const v4f acc = mma_kr<NP, SG, SA>(CqT + mt * 16 * SG, Am + DK + nt * 16);
#pragma unroll
            for (int v = 0; v < 4; ++v)
                Am[(NP + mt * 16 + 4 * (lane >> 4) + v) * SA + DK + nt * 16 + (lane & 15)] = acc[v] * isd;
        }
        lds_barrier();
#pragma unroll
        for (int u = 0; u < TKW; ++u) {
            const int t = wave + kWaves * u;
            if (t < TK) {
                const int mt = t / NTK, nt = t - mt * NTK;
#pragma unroll
                for (int v = 0; v < 4; ++v)
                    Am[(mt * 16 + 4 * (lane >> 4) + v) * SA + nt * 16 + (lane & 15)] = kacc[u][v];
            }
        }
    }
    lds_barrier();

    // ---- Q' / sqrt(d_k) = (diag(G / |q|) Q + Cq^T (-K')) / sqrt(d_k) in place over the
    //      q rows; meanwhile the state and V blocks become the transposed right operand
    {
        constexpr int NTK = DK / 16, TQ = NP / 16 * NTK;
        for (int t = wave; t < TQ; t += kWaves) {
            const int mt = t / NTK, nt = t - mt * NTK;
            const v4f acc = mma_kr<NP, SG, SA>(CqT + mt * 16 * SG, Am + nt * 16);
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int i = mt * 16 + 4 * (lane >> 4) + v;
                float *q = Am + (NP + i) * SA + nt * 16 + (lane & 15);
                *q = fmaf(s_gq[i], *q, acc[v]) * isd;
            }
        }
    }
    // (indices clamped as at load time: surplus threads rewrite the last element with the
    // value they loaded for it, so the stores need no condition)
#pragma unroll
    for (int u = 0; u < SPT; ++u) {
        const int f = min(tid + kThreads * u, SF4 - 1), r = f / Q4, q = f - r * Q4;
#pragma unroll
        for (int e = 0; e < 4; ++e) BmT[(4 * q + e) * SBT + r] = sreg[u][e];
    }
#pragma unroll
    for (int u = 0; u < VPT; ++u) {
        const int i = min((tid + kThreads * u) / Q4, NP - 1);
#pragma unroll
        for (int e = 0; e < 4; ++e) BmT[(4 * gv + e) * SBT + DK + i] = vreg[u][e];
    }
    lds_barrier();

    // ---- [delta; o] = A x [S0; V]
    {
        constexpr int NTJ = JB / 16, TM = 2 * NP / 16 * NTJ;
        float *logc = replay_log + ((int64_t)c * N * Hv + h) * R;
        for (int t = wave; t < TM; t += kWaves) {
            const int mt = t / NTJ, nt = t - mt * NTJ;
            const v4f acc = mma_kc<KA, SA, SBT>(Am + mt * 16 * SA, BmT + nt * 16 * SBT);
            const int col = j0 + nt * 16 + (lane & 15);
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int row = mt * 16 + 4 * (lane >> 4) + v;
                if (row < NP) {
                    if (row < N) logc[(int64_t)row * Hv * R + 1 + DK + col] = acc[v];
                } else if (row - NP < N) {
                    out[(((int64_t)c * N + row - NP) * Hv + h) * DV + col] = acc[v];
                }
            }
        }
    }
}

template <int DK, int DV, int NP>
__global__ __launch_bounds__(kThreads) void tree_verify_kernel(const VerifyArgs args) {
    verify_body<DK, DV, NP, false>(args);
}

template <int DK, int DV, int NP>
__global__ __launch_bounds__(kThreads) void conv_tree_verify_kernel(const VerifyArgs args) {
    verify_body<DK, DV, NP, true>(args);
}

template <int DK, int DV, int NP, bool FUSED>
hipError_t launch(const VerifyArgs &a, hipStream_t stream) {
    using Ly = VerifyLayout<DK, DV, NP, FUSED>;
    const size_t lds = sizeof(float) * Ly::LDS_FLOATS;
    // the LDS limit is a property of the kernel, set once (also keeps stream capture clean)
    const void *kernel = FUSED ? reinterpret_cast<const void *>(&conv_tree_verify_kernel<DK, DV, NP>)
                               : reinterpret_cast<const void *>(&tree_verify_kernel<DK, DV, NP>);
    static const hipError_t attr = hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (attr != hipSuccess) return attr;
    const int grid = Ly::NB * a.d.Hv * a.d.C;
    if constexpr (FUSED)
        hipLaunchKernelGGL((conv_tree_verify_kernel<DK, DV, NP>), dim3(grid), dim3(kThreads), lds, stream, a);
    else
        hipLaunchKernelGGL((tree_verify_kernel<DK, DV, NP>), dim3(grid), dim3(kThreads), lds, stream, a);
    return hipGetLastError();
}

template <int DK, int DV>
hipError_t launch_np(const VerifyArgs &a, hipStream_t stream) {
    const bool fused = a.x != nullptr;
    if (a.d.N <= 16) return fused ? launch<DK, DV, 16, true>(a, stream) : launch<DK, DV, 16, false>(a, stream);
    return fused ? launch<DK, DV, 32, true>(a, stream) : launch<DK, DV, 32, false>(a, stream);
}

}  // namespace

hipError_t launch_tree_verify(const VerifyArgs &a, hipStream_t stream) {
#define GDN_VERIFY_CASE(K, V) \
    if (a.d.dk == K && a.d.dv == V) return launch_np<K, V>(a, stream);
#define GDN_VERIFY_ROW(K) GDN_VERIFY_CASE(K, 16) GDN_VERIFY_CASE(K, 32) GDN_VERIFY_CASE(K, 64) GDN_VERIFY_CASE(K, 128)
    GDN_VERIFY_ROW(16) GDN_VERIFY_ROW(32) GDN_VERIFY_ROW(64) GDN_VERIFY_ROW(128)
#undef GDN_VERIFY_ROW
#undef GDN_VERIFY_CASE
    return hipErrorInvalidValue;
}

}  // namespace gdn
