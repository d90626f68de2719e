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
// For the raw (un-normalised) q and k rows, with rk_i = 1/|k_i|, rq_i = 1/|q_i| and the
// products KS = K S0, QS = Q S0 of the raw rows with the slot's state:
//   (I + Lm) D = rhs,  rhs_i = beta_i (v_i - G_i rk_i KS_i),
//   Lm[i][a] = beta_i (G_i/G_a) rk_i rk_a (k_i . k_a)   for a a strict ancestor of i,
//   O_i = G_i rq_i QS_i / sqrt(d_k) + sum_{a on path(i)} Cq[i][a] D_a,
//   Cq[i][a] = (G_i/G_a) rq_i rk_a (q_i . k_a) / sqrt(d_k),
// where D holds the delta rows (replay log) and O the output rows.  The tree algebra
// (norms, Gram products, Lm, Cq and T = (I + Lm)^-1, all N x N) needs only q, k, the
// gates and the tree, so it runs while the state block is still arriving; the state
// enters through one dense product [K; Q] x S0, after which D = T rhs and O are two
// small products on the accumulators.  Per-node states are never formed and S0 is read
// once.  Decay ratios are exp(L_i - L_a) of cumulative log-decays, which cannot
// overflow.
//
// Mapping: one workgroup (8 waves) per (lane, value head, block of 64 value columns).
// Products run on v_mfma_f32_16x16x4_f32.  Within a 16-wide chunk of a contraction,
// lane group g = lane/16 supplies index 4g + s in MFMA step s (a permutation shared by
// both operands), so a tile's accumulators (lane holds rows 4g..4g+3 of column lane%16)
// are directly the right operand of the next product, and the state block is loaded
// from memory straight into that operand layout: no LDS copy, no transpose.  The
// contractions over d_k are split by 16-row chunks: the Gram products over waves 0..3
// (chunk q on wave q mod 4), the state product over all 8 waves (wave w takes one
// 16-column tile and every (8 / tiles)-th chunk), and the partial tiles are summed
// through LDS.  N is padded to NP (16 or 32) with zero rows.  Barriers wait only for
// LDS traffic, so global loads stay in flight across them.  Workgroup ids are ordered
// so that the workgroups sharing one (lane, q/k head) are congruent modulo the number
// of such groups: with round-robin dispatch over the 8 XCDs they land on one XCD and
// read the shared q/k rows through its L2.
//
// Load order.  Every load that does not depend on the slot (tree, gates, token rows,
// taps) is issued before the slot id is consumed and the slot-mapped history right
// after it; the state block is requested only once the token rows are staged, so that
// the rows the conv needs first do not queue behind it, and it arrives during the conv.
//
// Fused route (conv + verify, "perf(qwen35): fuse the DFlash2 concurrent verify Gated
// DeltaNet route", Optimizations): the workgroup reads the raw projected tokens x of its
// q/k slab and value block, stages them in LDS, and computes the tree conv + SiLU of its
// channels in registers (sources of node i, oldest first: the tokens of i's nearest
// ancestors, then the slot's history columns), writing the results straight into the
// product operands; the conv output never goes to memory.  The commit windows are
// written once, by copy-only workgroups appended to the same launch (one per lane and
// block of channels), which run beside the verify workgroups; in the wide variant with two
// or more verify workgroups per CU, by the verify workgroups from their staged rows.
#include "gdn_device.h"
#include "gdn_internal.h"

namespace gdn {
namespace {

constexpr int kThreads = 512;
constexpr int kWaves = kThreads / 64;

// Raw buffer resources: word 3 of the descriptor for the gfx9 family (32-bit data,
// unswizzled); a load whose byte offset lies outside [0, num_records) returns zero and
// makes no memory access.
constexpr int kRsrcWord3 = 0x00020000;
constexpr int kOutOfRange = 0x40000000;  // past every buffer range used here (at most 1 GiB)
typedef int v4i __attribute__((ext_vector_type(4)));
constexpr int kNonTemporal = 2;  // cache-policy operand of the buffer stores: nt

__device__ inline float load1(__amdgpu_buffer_rsrc_t r, int byte_offset) {
    return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, byte_offset, 0, 0));
}

__device__ inline v4f load4(__amdgpu_buffer_rsrc_t r, int byte_offset) {
    return __builtin_bit_cast(v4f, __builtin_amdgcn_raw_buffer_load_b128(r, byte_offset, 0, 0));
}

// Wide variant, fused route: the commit windows are written by the verify workgroups
// themselves once the grid spans more than one workgroup per CU (two or more per CU on
// 256 CUs); below that, copy-only workgroups in the free slots beside them write the windows
// sooner.
__host__ __device__ inline bool windows_in_verify(const Dims &d) { return d.C * d.Hv >= 512; }

// WIDE: a workgroup covers all d_v columns of its value head (eight 16-column tiles, one per
// wave, each over the whole of d_k) instead of 64 of them; see launch_np.  WINV (fused, wide):
// the verify workgroups also write the commit windows, so the staged rows stay until then.
template <int DK, int DV, int NP, bool FUSED, bool WIDE = false, bool WINV = false>
struct VerifyLayout {
    static constexpr int JB = WIDE ? DV : (DV < 64 ? DV : 64);  // value columns per workgroup
    static constexpr int NB = DV / JB;            // column blocks per head
    static constexpr int CT = JB / 16;            // 16-column tiles of the block
    static constexpr int NT = NP / 16;            // 16-row tiles of K (and of Q)
    static constexpr int RT = 2 * NT;             // row tiles of [K; Q]
    static constexpr int KC = DK / 16;            // 16-wide chunks of the d_k contraction
    static constexpr int GW = 4;                            // Gram: waves 0..3, chunk q on wave q % 4
    static constexpr int LCG = (KC + GW - 1) / GW;          // Gram: chunks per wave
    static constexpr int KP = kWaves / CT;                  // state product: waves per column tile
    static constexpr int LCQ = (KC + KP - 1) / KP;          // state product: chunks per wave
    static constexpr int R = 1 + DK + DV;         // replay-log row
    static constexpr int G = DK / 2;              // 4-channel groups of one node's q|k slab
    static constexpr int Q4 = JB / 4;             // 4-channel groups of one node's value block
    static constexpr int NPART = DK / 4 > 16 ? 2 : 1;  // 16-lane partial sums per |row|^2
    // row strides (floats) are 4 mod 8 so 16 rows read with ds_read_b128 hit distinct banks
    static constexpr int SX = DK + 4;   // [K; Q] raw rows [2NP][SX]
    static constexpr int SV = JB + 4;   // value rows [NP][SV]
    static constexpr int SG = NP + 4;   // N x N matrices
    static constexpr int SXS = 2 * DK + JB;  // fused: staged rows [NP + 3][SXS] of the block's channels
    static constexpr int OFF_XQK = 0;
    static constexpr int OFF_V = OFF_XQK + 2 * NP * SX;
    static constexpr int OFF_LM = (OFF_V + NP * SV + 3) / 4 * 4;
    static constexpr int OFF_CQ = OFF_LM + NP * SG;
    static constexpr int OFF_T = OFF_CQ + NP * SG;
    static constexpr int NG = G + Q4;             // channel groups of the block (q/k slab, then values)
    static constexpr int OFF_TAP = OFF_T + NP * SG;                   // fused: taps [NG][4] of v4f
    static constexpr int OFF_SCR = OFF_TAP + (FUSED ? NG * 16 : 0);
    static constexpr int OFF_STG = OFF_SCR;  // fused: staged rows, dead once the conv is done
    // scratch, reused: staged rows (until the conv; fused and wide: until the commit
    // windows are written, after the Gram products), Gram partials (until the
    // coefficients), partial state products
    static constexpr int STAGE = FUSED ? (NP + 3) * SXS : 0;
    static constexpr int GRAM_TILES = RT * NT;
    static constexpr int GPART = GW * GRAM_TILES * 256;
    // SPLIT: the state product [K; Q] x S0 as three bf16 products of hi/lo parts (see
    // state_product), from the raw rows' bf16 parts [2NP][SXB] in LDS.  SPLIT_B (64-column blocks
    // over at most 16 nodes): the parts are written during the conv, beside the scratch (two
    // workgroups per CU still fit).  SPLIT_W (wide, windows written elsewhere): waves 4..7
    // convert them beside the Gram products into the staging area, dead after the conv, and the
    // Gram partials follow them there.  SPLIT_R (wide, windows written by the verify
    // workgroups, so the staging area stays in use and the LDS is full): each wave splits the
    // fp32 rows it reads in registers instead.
    static constexpr bool SPLIT_B = !WIDE && NP == 16 && DK % 32 == 0 && (DK / 32) % KP == 0;
    static constexpr bool SPLIT_W = WIDE && !(FUSED && WINV) && DK % 32 == 0;
    static constexpr bool SPLIT_R = WIDE && FUSED && WINV && DK % 32 == 0;
    static constexpr bool SPLIT = SPLIT_B || SPLIT_W || SPLIT_R;
    static constexpr int SXB = DK + 8;  // bf16 row stride: 16 rows read with ds_read_b128 hit distinct banks
    static constexpr int XHF = 2 * NP * SXB;  // floats of the hi and lo parts (two bf16 per float)
    static constexpr int LC3 = SPLIT ? DK / 32 / KP : 0;  // state product: 32-wide chunks per wave
    static constexpr int OFF_GRAM = FUSED && WIDE && WINV ? STAGE : (SPLIT_W ? XHF : 0);
    // state-product partials: unit u = wave u covers column tile u % CT and k part u / CT
    static constexpr int UNIT = RT * 256;
    static constexpr int OFF_UNIT = OFF_GRAM + GPART;
    // WIDE: every wave's state-product tiles are complete and stay in its registers
    static constexpr int PARTS = OFF_GRAM + GPART + (WIDE ? 0 : kWaves * UNIT);
    static constexpr int SCR1 = STAGE > PARTS ? STAGE : PARTS;
    static constexpr int SCR = SCR1 > 2 * NP * SV ? SCR1 : 2 * NP * SV;  // also the epilogue's row staging
    static constexpr int OFF_XH = SPLIT_W ? OFF_SCR : OFF_SCR + SCR;  // hi parts, then lo parts
    static constexpr int LDS_FLOATS = OFF_SCR + SCR + (SPLIT_B ? XHF : 0);
    static_assert(4 * LDS_FLOATS <= 160 * 1024 - 2048, "LDS of one workgroup (with the static arrays)");
};

// Tree conv + SiLU of 4 channels at one node from its sources, oldest first (x3 = the
// node's own tokens); w[e] holds the 4 taps of channel e (tap 0 = oldest), summed from
// the oldest source.
__device__ inline v4f conv_silu(v4f x0, v4f x1, v4f x2, v4f x3, const v4f w[4]) {
    v4f y;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const v4f we = w[e];
        float z = x0[e] * we[0];
        z = fmaf(x1[e], we[1], z);
        z = fmaf(x2[e], we[2], z);
        z = fmaf(x3[e], we[3], z);
        y[e] = fast_silu(z);
    }
    return y;
}

// history columns of 4 channels from their 12 consecutive floats
__device__ inline void hist_columns(const v4f raw[3], v4f hc[3]) {
    const v4f a = raw[0], b = raw[1], e = raw[2];  // ch0: a.x a.y a.z | ch1: a.w b.x b.y | ch2: b.z b.w e.x | ch3: e.y e.z e.w
    hc[0] = v4f{a.x, a.w, b.z, e.y};
    hc[1] = v4f{a.y, b.x, b.w, e.z};
    hc[2] = v4f{a.z, b.y, e.x, e.w};
}

// RAGGED: the caller passed per-lane node counts (without them every lane has N nodes and
// the count costs nothing)
template <int DK, int DV, int NP, bool FUSED, bool RAGGED, bool WIDE, bool WINV>
__device__ __forceinline__ void verify_body(const VerifyArgs &args) {
    using Ly = VerifyLayout<DK, DV, NP, FUSED, WIDE, WINV>;
    static_assert(!WIDE || Ly::KP == 1, "wide: one wave per column tile");
    constexpr int JB = Ly::JB, NB = Ly::NB, CT = Ly::CT, NT = Ly::NT, RT = Ly::RT, KC = Ly::KC, LCG = Ly::LCG, KP = Ly::KP, LCQ = Ly::LCQ;
    constexpr int R = Ly::R, G = Ly::G, Q4 = Ly::Q4, SX = Ly::SX, SV = Ly::SV, SG = Ly::SG, SXS = Ly::SXS;
    static_assert(kThreads % G == 0 && kThreads % Q4 == 0 && 64 % G == 0, "channel groups must tile a wave");
    extern __shared__ float lds[];
    float *XQK = lds + Ly::OFF_XQK;  // raw conv rows: k of node i at row i, q of node i at row NP + i
    float *Vl = lds + Ly::OFF_V;     // conv value rows of the block
    float *Lm = lds + Ly::OFF_LM;    // strictly lower solve matrix
    float *Cq = lds + Ly::OFF_CQ;    // output coefficients (1/sqrt(d_k) folded in)
    float *Tm = lds + Ly::OFF_T;     // T = (I + Lm)^-1
    float *scr = lds + Ly::OFF_SCR;
    __bf16 *XH = reinterpret_cast<__bf16 *>(lds + Ly::OFF_XH);  // SPLIT: bf16 parts of the raw rows
    __bf16 *XL = XH + 2 * NP * Ly::SXB;
    __shared__ int s_wbits[kWaves];
    __shared__ float s_beta[NP], s_g[NP], s_G[NP], s_gk[NP], s_gq[NP], s_r[2 * NP];
    // cumulative log-decays in double: along a path of strong decays they reach hundreds, and
    // a float sum would then lose about 1e-4 of every ratio exp(L_i - L_a) formed from them
    __shared__ double s_L[NP];
    __shared__ float s_ssq[2 * NP][Ly::NPART];
    __shared__ unsigned int s_anc[NP];
    // conv sources of node i, oldest first, as staged rows (node rows, or NP + j for
    // history column j): s0 | s1 << 8 | s2 << 16; the node itself is the newest source
    __shared__ int s_src[NP];

    const Dims d = args.d;
    // every kernel argument used for an address, read in the first batch of scalar loads
    asm volatile("" ::"s"(d.C), "s"(d.N), "s"(d.P), "s"(d.Hk), "s"(d.Hv), "s"(d.Ch), "s"(FUSED ? args.x : args.qkv),
                 "s"(args.conv_w), "s"(args.conv_hist), "s"(args.state_pool), "s"(args.slot_ids), "s"(args.parents));
    const int N = d.N, Hv = d.Hv;
    // workgroup -> (lane c, q/k head kh, share index ws); ws -> (value head h, column block jb)
    const int n_groups = d.C * d.Hk;
    const int grp = blockIdx.x % n_groups, ws = blockIdx.x / n_groups;
    const int c = grp / d.Hk, kh = grp - c * d.Hk;
    const int jb = ws % NB, h = kh + d.Hk * (ws / NB);
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int g4 = lane >> 4, l16 = lane & 15;
    const int j0 = jb * JB;

    // ---- loads, all issued before any of them is consumed.  Token rows, history and
    //      state go through range-checked buffer loads: rows past N, and everything of a
    //      padding or invalid lane, fall outside the range and read as zero without a
    //      memory access, so no load sits behind a branch or a select.
    // the slot id goes through a vector load: a scalar load would share its wait counter
    // with the kernel-argument loads and hold up every load issued after it
    // (it stays in a vector register until every load that does not need it is issued)
    const int s_v = __builtin_bit_cast(
        int, __builtin_amdgcn_raw_buffer_load_b32(
                 __builtin_amdgcn_make_buffer_rsrc(const_cast<int32_t *>(args.slot_ids), 0, 4 * d.C, kRsrcWord3), 4 * c, 0,
                 0));
    // ragged lanes: the lane's node count the same way
    int nv_v = 0;
    if constexpr (RAGGED)
        nv_v = __builtin_bit_cast(
            int, __builtin_amdgcn_raw_buffer_load_b32(
                     __builtin_amdgcn_make_buffer_rsrc(const_cast<int32_t *>(args.lane_nodes), 0, 4 * d.C, kRsrcWord3),
                     4 * c, 0, 0));
    const int par = args.parents[(int64_t)c * N + (lane < N ? lane : 0)];  // lane i of every wave: parent of node i
    const int tn = tid < N ? tid : 0;
    const int64_t trow = (int64_t)c * N + tn;
    const float braw = args.beta_logits[trow * args.gate_stride + h];
    const float araw = args.alpha_logits[trow * args.gate_stride + h] + args.dt_bias[h];
    const float Ah = args.A[h];
    constexpr int DUP = (GDN_MAX_SEQS + kThreads - 1) / kThreads;
    int so[DUP];  // slots of lanes tid, tid + 256, ... (duplicate check)
#pragma unroll
    for (int k = 0; k < DUP; ++k) so[k] = args.slot_ids[min(tid + kThreads * k, d.C - 1)];

    // q|k slab (raw tokens when fused, conv rows otherwise): item u of a thread is group
    // gq = tid % G of node (tid / G) * QPT + u; groups 0..DK/4-1 are q channels, the rest k
    constexpr int QPT = (G * NP + kThreads - 1) / kThreads;
    const int gq = tid % G;
    const int chq = gq < DK / 4 ? kh * DK + 4 * gq : d.Hk * DK + kh * DK + 4 * (gq - DK / 4);
    const float *src = FUSED ? args.x : args.qkv;
    const __amdgpu_buffer_rsrc_t xr =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<float *>(src + (int64_t)c * N * d.Ch), 0,
                                          (int)(4u * (unsigned)N * (unsigned)d.Ch), kRsrcWord3);
    v4f qreg[QPT];
#pragma unroll
    for (int u = 0; u < QPT; ++u) {
        const int i = min((tid / G) * QPT + u, NP - 1);
        qreg[u] = load4(xr, (i * d.Ch + chq) * 4);
    }
    // value block: item u of a thread is group gv = tid % Q4 of node (tid / Q4) * VPT + u
    constexpr int VPT = (Q4 * NP + kThreads - 1) / kThreads;
    const int gv = tid % Q4;
    const int chv = 2 * d.Hk * DK + h * DV + j0 + 4 * gv;
    v4f vreg[VPT];
#pragma unroll
    for (int u = 0; u < VPT; ++u) {
        const int i = min((tid / Q4) * VPT + u, NP - 1);
        vreg[u] = load4(xr, (i * d.Ch + chv) * 4);
    }
    // fused: the taps and history of the block's channel groups are loaded once per
    // workgroup (4 + 3 float4 per group, spread over the threads) and staged in LDS
    constexpr int NG = Ly::NG, TPT = (NG * 4 + kThreads - 1) / kThreads;
    static_assert(NG <= kThreads, "one history group per thread");
    auto group_channel = [&](int g) {
        return g < G ? (g < DK / 4 ? kh * DK + 4 * g : d.Hk * DK + kh * DK + 4 * (g - DK / 4))
                     : 2 * d.Hk * DK + h * DV + j0 + 4 * (g - G);
    };
    v4f treg[TPT];
    if constexpr (FUSED) {
        const __amdgpu_buffer_rsrc_t wr4 =
            __builtin_amdgcn_make_buffer_rsrc(const_cast<float *>(args.conv_w), 0, d.Ch * 16, kRsrcWord3);
#pragma unroll
        for (int u = 0; u < TPT; ++u) {
            const int f = tid + kThreads * u;
            treg[u] = load4(wr4, f < NG * 4 ? (group_channel(f >> 2) + (f & 3)) * 16 : kOutOfRange);
        }
    }
    // loads complete in issue order: keep everything the conv needs ahead of the state
    __builtin_amdgcn_sched_barrier(0);
    const int s = __builtin_amdgcn_readfirstlane(s_v);
    // slot-mapped: the 12 history floats of each channel group (fused)
    const bool s_ok = s >= 0 && s < d.P;
    const int sc = s_ok ? s : 0;
    v4f hreg[3];  // fused: the 12 history floats of channel group tid (if tid < NG)
    if constexpr (FUSED) {
        const __amdgpu_buffer_rsrc_t hr = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<float *>(args.conv_hist + (int64_t)sc * d.Ch * 3), 0, s_ok ? d.Ch * 12 : 0, kRsrcWord3);
        const int hb = tid < NG ? group_channel(tid) * 12 : kOutOfRange;
#pragma unroll
        for (int e = 0; e < 3; ++e) hreg[e] = load4(hr, hb + 16 * e);
    }
    __builtin_amdgcn_sched_barrier(0);
    const int wv_u = __builtin_amdgcn_readfirstlane(wave);
    const int pct = wv_u % CT, pkp = wv_u / CT;  // state product: column tile and k part of this wave
    // nodes present in this lane (nodes past them are absent: zero rows, nothing written)
    const int nv = RAGGED ? __builtin_amdgcn_readfirstlane(nv_v) : N;
    const int nvc = min(max(nv, 0), N);

    // ---- lane validity (slot range, duplicate slot, node count, present nodes' parents);
    //      nothing is written for a bad lane and a padding lane (slot -1) is skipped
    //      without a status bit
    int bits = 0;
    if (s != -1) {
        if (!s_ok) bits |= GDN_STATUS_SLOT_RANGE;
#pragma unroll
        for (int k = 0; k < DUP; ++k) {
            const int o = tid + kThreads * k;
            if (o < d.C && o != c && so[k] == s) bits |= GDN_STATUS_SLOT_DUP;
        }
        if (nv != nvc) bits |= GDN_STATUS_NODES;
        if (tid < nvc && (par < -1 || par >= tid)) bits |= GDN_STATUS_PARENT;
    }
    {
        int wb = 0;
#pragma unroll
        for (int b = 0; b < 5; ++b)
            if (__builtin_amdgcn_ballot_w64((bits >> b) & 1)) wb |= 1 << b;
        if (lane == 0) s_wbits[wave] = wb;
    }

    // ---- tree, wave 0: cumulative log-decay L_i, ancestor set (pointer jumping over
    //      log2(NP) rounds of lane shuffles, independent of the tree depth), and the three
    //      nearest ancestors of every node for the conv
    if (wave == 0) {
        const bool real = lane < nvc;
        const int a1 = real ? par : -1;
        int jump = a1;
        double L = 0.0;
        if (real) L = fast_softplus(araw) * Ah;  // log g = softplus(a + dt_bias) * A
        if (lane < NP) s_g[lane] = real ? fast_exp((float)L) : 0.f;
        unsigned int anc = real ? 1u << lane : 0u;
        const int a2s = __shfl(a1, a1 >= 0 ? a1 : 0);
        const int a2 = a1 >= 0 ? a2s : -1;
        const int a3s = __shfl(a2, a1 >= 0 ? a1 : 0);
        const int a3 = a1 >= 0 ? a3s : -1;
#pragma unroll
        for (int r = 1; r < NP; r <<= 1) {
            const int srcl = jump < 0 ? lane : jump;
            const double Lj = __shfl(L, srcl);
            const unsigned int aj = __shfl(anc, srcl);
            const int jj = __shfl(jump, srcl);
            if (jump >= 0) {
                L += Lj;
                anc |= aj;
                jump = jj;
            }
        }
        if (lane < NP) {
            s_L[lane] = L;
            s_G[lane] = real ? fast_exp((float)L) : 0.f;
            s_anc[lane] = anc;
            s_beta[lane] = real ? fast_sigmoid(braw) : 0.f;
            const int r2 = a1 >= 0 ? a1 : NP + 2;
            const int r1 = a1 >= 0 ? (a2 >= 0 ? a2 : NP + 2) : NP + 1;
            const int r0 = a1 >= 0 ? (a2 >= 0 ? (a3 >= 0 ? a3 : NP + 2) : NP + 1) : NP;
            s_src[lane] = r0 | r1 << 8 | r2 << 16;
        }
    }
    // fused: stage the raw token rows for the tree conv
    float *stg = lds + Ly::OFF_STG;  // node rows 0..NP-1, then history columns 0..2
    if constexpr (FUSED) {
#pragma unroll
        for (int u = 0; u < QPT; ++u) {
            const int i = (tid / G) * QPT + u;
            if (i < NP) *reinterpret_cast<v4f *>(stg + i * SXS + 4 * gq) = qreg[u];
        }
#pragma unroll
        for (int u = 0; u < VPT; ++u) {
            const int i = (tid / Q4) * VPT + u;
            if (i < NP) *reinterpret_cast<v4f *>(stg + i * SXS + 2 * DK + 4 * gv) = vreg[u];
        }
#pragma unroll
        for (int u = 0; u < TPT; ++u) {
            const int f = tid + kThreads * u;
            if (f < NG * 4) *reinterpret_cast<v4f *>(lds + Ly::OFF_TAP + 4 * f) = treg[u];
        }
        if (tid < NG) {  // history columns of group tid as staged rows NP..NP+2
            v4f hc[3];
            hist_columns(hreg, hc);
            const int col = tid < G ? 4 * tid : 2 * DK + 4 * (tid - G);
#pragma unroll
            for (int e = 0; e < 3; ++e) *reinterpret_cast<v4f *>(stg + (NP + e) * SXS + col) = hc[e];
        }
    }
    lds_barrier();
    if (s == -1) return;  // padding lane
    {
        int all = 0;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) all |= s_wbits[w];
        if (all) {
            if (ws == 0 && tid == 0 && args.status) atomicOr(args.status, all);
            return;
        }
    }

    // ---- this wave's chunks of the state block, in the right-operand layout
    //      sreg[lc][e] = S0[16q + 4*g4 + e][j0 + 16*pct + l16], chunks q = pkp + KP*lc.  They
    //      are requested only now, once the token rows have arrived, so that the rows the
    //      conv and the tree algebra need first do not queue behind the state in HBM; the
    //      state is first needed after the conv.
    //      SPLIT: the 32-wide chunks m = pkp + KP*l3 of the bf16 products instead, lane group g4
    //      holding rows 32m + 8*g4 + 0..7 (in sreg[2*l3][0..3], sreg[2*l3 + 1][0..3])
    float sreg[LCQ][4];
    {
        const __amdgpu_buffer_rsrc_t sr = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<float *>(args.state_pool + ((int64_t)sc * Hv + h) * DK * DV), 0, s_ok ? DK * DV * 4 : 0,
            kRsrcWord3);
#pragma unroll
        for (int lc = 0; lc < LCQ; ++lc) {
            const int q = pkp + KP * lc;
            const int row0 = Ly::SPLIT ? 32 * (pkp + KP * (lc / 2)) + 8 * g4 + 4 * (lc % 2) : 16 * q + 4 * g4;
            const int base = (Ly::SPLIT || KC % KP == 0 || q < KC) ? (row0 * DV + j0 + 16 * pct + l16) * 4 : kOutOfRange;
#pragma unroll
            for (int e = 0; e < 4; ++e) sreg[lc][e] = load1(sr, base + e * DV * 4);
        }
    }

    // SPLIT_W: the bf16 parts of the raw [K; Q] rows, by 256 threads (t = 0..255), TPR of them
    // per row
    auto convert_rows = [&](int t) {
        constexpr int TPR = 256 / (2 * NP) < DK / 4 ? 256 / (2 * NP) : DK / 4;  // threads per row
        if (t >= 2 * NP * TPR) return;
        const int row = t / TPR, c0 = (t % TPR) * (DK / TPR);
#pragma unroll
        for (int k = 0; k < DK / TPR; k += 4) {
            const v4f x = *reinterpret_cast<const v4f *>(XQK + row * SX + c0 + k);
            const float y[4] = {x.x, x.y, x.z, x.w};
            __bf16 hi[4], lo[4];
            split_bf16(y, hi, lo);
            *reinterpret_cast<bf4 *>(XH + row * Ly::SXB + c0 + k) = bf4{hi[0], hi[1], hi[2], hi[3]};
            *reinterpret_cast<bf4 *>(XL + row * Ly::SXB + c0 + k) = bf4{lo[0], lo[1], lo[2], lo[3]};
        }
    };
    // ---- fused, wide, windows by the verify workgroups: after their state product, waves 4..7
    //      (32 nodes: every wave) write the commit windows of the workgroup's channels from the
    //      staged rows.  The window of node i and channel e is (oldest first) its second and first
    //      nearest sources and its own token, 3 floats; 4 channels take 12 consecutive floats,
    //      stored as three 16-byte chunks (flat float f of a group = source f % 3 of channel
    //      f / 3).  Lane l takes chunk l + 64m of a node's row of chunks, so a store instruction
    //      writes consecutive chunks.  The q/k slab's channel groups are split over the workgroups
    //      that share it (the value heads of the q/k head), the value block is this workgroup's
    //      own.  No global load follows these stores.
    auto write_windows = [&]() {
        const int nshare = Hv / d.Hk;
        const int gq0 = (ws * G) / nshare, nq = ((ws + 1) * G) / nshare - gq0;
        const int cpn = 3 * (nq + Q4);  // chunks of one node
        const __amdgpu_buffer_rsrc_t wr = __builtin_amdgcn_make_buffer_rsrc(
            args.commit_win + (int64_t)c * N * d.Ch * 3, 0, nvc * d.Ch * 12, kRsrcWord3);
        for (int m = 0; 64 * m < cpn; ++m) {
            const int r = lane + 64 * m, gg = r / 3, p = r - 3 * gg;
            const bool slab = gg < nq;
            const int g = slab ? gq0 + gg : min(gg - nq, Q4 - 1);
            const int col = slab ? 4 * g : 2 * DK + 4 * g;
            const int ch = slab ? (g < DK / 4 ? kh * DK + 4 * g : d.Hk * DK + kh * DK + 4 * (g - DK / 4))
                                : 2 * d.Hk * DK + h * DV + j0 + 4 * g;
            const int gofs = r < cpn ? ch * 12 + 16 * p : kOutOfRange;
            constexpr int WW = NP == 32 ? kWaves : 4;  // waves writing windows: the last WW
            for (int i = wv_u - (kWaves - WW); i < nvc; i += WW) {
                const int sr = s_src[i];
                const int rb[3] = {((sr >> 8) & 255) * SXS + col, ((sr >> 16) & 255) * SXS + col, i * SXS + col};
                float w[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int f = 4 * p + e, src = f % 3;  // p + e = f mod 3
                    w[e] = stg[(src == 0 ? rb[0] : src == 1 ? rb[1] : rb[2]) + f / 3];
                }
                const v4f chunk = {w[0], w[1], w[2], w[3]};
                __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(v4i, chunk), wr,
                                                       gofs < kOutOfRange ? i * d.Ch * 12 + gofs : kOutOfRange, 0,
                                                       kNonTemporal);
            }
        }
    };

    // ---- conv + SiLU (fused) of the block's channels, or the loaded conv rows as they are:
    //      raw q/k rows into XQK with their squared norms, value rows into Vl
    {
        const v4f zero = {0.f, 0.f, 0.f, 0.f};
        const v4f *tap = reinterpret_cast<const v4f *>(lds + Ly::OFF_TAP);
        // every LDS read of the phase is issued before its first LDS write (the compiler
        // cannot reorder them across writes to the same array), then compute, then write
        // waves whose value items all lie past the padded node count skip the value part
        const bool has_v = ((64 * wv_u) / Q4) * VPT < NP;
        v4f yq[QPT], yv[VPT], xq[QPT][3], xv[VPT][3], wq[4], wv[4];
        if constexpr (FUSED) {
            int sq[QPT];
#pragma unroll
            for (int u = 0; u < QPT; ++u) sq[u] = s_src[min((tid / G) * QPT + u, NP - 1)];
#pragma unroll
            for (int e = 0; e < 4; ++e) wq[e] = tap[4 * gq + e];
#pragma unroll
            for (int u = 0; u < QPT; ++u)
#pragma unroll
                for (int e = 0; e < 3; ++e)
                    xq[u][e] = *reinterpret_cast<const v4f *>(stg + ((sq[u] >> (8 * e)) & 255) * SXS + 4 * gq);
            if (has_v) {
                int sv[VPT];
#pragma unroll
                for (int u = 0; u < VPT; ++u) sv[u] = s_src[min((tid / Q4) * VPT + u, NP - 1)];
#pragma unroll
                for (int e = 0; e < 4; ++e) wv[e] = tap[4 * (G + gv) + e];
#pragma unroll
                for (int u = 0; u < VPT; ++u)
#pragma unroll
                    for (int e = 0; e < 3; ++e)
                        xv[u][e] =
                            *reinterpret_cast<const v4f *>(stg + ((sv[u] >> (8 * e)) & 255) * SXS + 2 * DK + 4 * gv);
            }
        }
#pragma unroll
        for (int u = 0; u < QPT; ++u) {
            const int i = (tid / G) * QPT + u;
            yq[u] = qreg[u];
            if constexpr (FUSED) yq[u] = conv_silu(xq[u][0], xq[u][1], xq[u][2], qreg[u], wq);
            yq[u] = i < nvc ? yq[u] : zero;
        }
        if (has_v) {
#pragma unroll
            for (int u = 0; u < VPT; ++u) {
                const int i = (tid / Q4) * VPT + u;
                yv[u] = vreg[u];
                if constexpr (FUSED) yv[u] = conv_silu(xv[u][0], xv[u][1], xv[u][2], vreg[u], wv);
                yv[u] = i < nvc ? yv[u] : zero;
            }
        }
        const bool isq = gq < DK / 4;
        const int cg = isq ? gq : gq - DK / 4;  // group within the q or k row
#pragma unroll
        for (int u = 0; u < QPT; ++u) {
            const int i = (tid / G) * QPT + u;
            float ss = yq[u].x * yq[u].x + yq[u].y * yq[u].y + yq[u].z * yq[u].z + yq[u].w * yq[u].w;
            ss = group_sum_last<(DK / 4 < 16 ? DK / 4 : 16)>(ss);
            if (i < NP) {
                const int row = isq ? NP + i : i;
                *reinterpret_cast<v4f *>(XQK + row * SX + 4 * cg) = yq[u];
                if ((cg & 15) == (DK / 4 < 16 ? DK / 4 : 16) - 1) s_ssq[row][cg >> 4] = ss;
                if constexpr (Ly::SPLIT_B) {
                    const float y[4] = {yq[u].x, yq[u].y, yq[u].z, yq[u].w};
                    __bf16 hi[4], lo[4];
                    split_bf16(y, hi, lo);
                    *reinterpret_cast<bf4 *>(XH + row * Ly::SXB + 4 * cg) = bf4{hi[0], hi[1], hi[2], hi[3]};
                    *reinterpret_cast<bf4 *>(XL + row * Ly::SXB + 4 * cg) = bf4{lo[0], lo[1], lo[2], lo[3]};
                }
            }
        }
        if (has_v) {
#pragma unroll
            for (int u = 0; u < VPT; ++u) {
                const int i = (tid / Q4) * VPT + u;
                if (i < NP) *reinterpret_cast<v4f *>(Vl + i * SV + 4 * gv) = yv[u];
            }
        }
    }
    lds_barrier();

    // ---- [K; Q] x S0 for this wave's unit (column tile pct, chunks q = pkp + KP*lc) into
    //      LDS partial tiles in accumulator order (WIDE: the complete tiles stay in sp)
    v4f sp[Ly::RT];
    //      SPLIT: per 32-wide chunk three v_mfma_f32_16x16x32_bf16 on the hi/lo parts of both
    //      operands (hi.hi + hi.lo + lo.hi), lane group g4 supplying rows 32m + 8*g4 + 0..7 of
    //      the chunk in both operands; the float32 accumulators have the layout of mfma4's
    auto state_product = [&]() {
        v4f acc[RT];
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) acc[rt] = v4f{0.f, 0.f, 0.f, 0.f};
        if constexpr (Ly::SPLIT) {
#pragma unroll
            for (int l3 = 0; l3 < Ly::LC3; ++l3) {
                const int m = pkp + KP * l3;
                const float x[8] = {sreg[2 * l3][0],     sreg[2 * l3][1],     sreg[2 * l3][2],     sreg[2 * l3][3],
                                    sreg[2 * l3 + 1][0], sreg[2 * l3 + 1][1], sreg[2 * l3 + 1][2], sreg[2 * l3 + 1][3]};
                __bf16 bh[8], bl[8];
                split_bf16(x, bh, bl);
                const bf8 vbh = {bh[0], bh[1], bh[2], bh[3], bh[4], bh[5], bh[6], bh[7]};
                const bf8 vbl = {bl[0], bl[1], bl[2], bl[3], bl[4], bl[5], bl[6], bl[7]};
#pragma unroll
                for (int rt = 0; rt < RT; ++rt) {
                    bf8 ah, al;
                    if constexpr (Ly::SPLIT_R) {
                        const float *xr = XQK + (16 * rt + l16) * SX + 32 * m + 8 * g4;
                        const v4f a0 = *reinterpret_cast<const v4f *>(xr), a1 = *reinterpret_cast<const v4f *>(xr + 4);
                        const float xa[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
                        __bf16 h[8], l[8];
                        split_bf16(xa, h, l);
                        ah = bf8{h[0], h[1], h[2], h[3], h[4], h[5], h[6], h[7]};
                        al = bf8{l[0], l[1], l[2], l[3], l[4], l[5], l[6], l[7]};
                    } else {
                        const int off = (16 * rt + l16) * Ly::SXB + 32 * m + 8 * g4;
                        ah = *reinterpret_cast<const bf8 *>(XH + off);
                        al = *reinterpret_cast<const bf8 *>(XL + off);
                    }
                    acc[rt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al, vbh, acc[rt], 0, 0, 0);
                    acc[rt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, vbl, acc[rt], 0, 0, 0);
                    acc[rt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, vbh, acc[rt], 0, 0, 0);
                }
            }
        } else {
#pragma unroll
            for (int lc = 0; lc < LCQ; ++lc) {
                const int q = pkp + KP * lc;
                if (KC % KP == 0 || q < KC) {
                    const v4f bv = {sreg[lc][0], sreg[lc][1], sreg[lc][2], sreg[lc][3]};
#pragma unroll
                    for (int rt = 0; rt < RT; ++rt)
                        acc[rt] = mfma4(*reinterpret_cast<const v4f *>(XQK + (16 * rt + l16) * SX + 16 * q + 4 * g4),
                                        bv, acc[rt]);
                }
            }
        }
        if constexpr (WIDE) {
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) sp[rt] = acc[rt];
        } else {
            float *pp = scr + Ly::OFF_UNIT + wv_u * Ly::UNIT + lane * 4;
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) *reinterpret_cast<v4f *>(pp + rt * 256) = acc[rt];
        }
    };

    // ---- waves 0..3: Gram products of the raw rows, split by 16-wide chunks of d_k:
    //      tile (rt, at) = rows 16rt.. of [K; Q] against k rows 16at..; partial tiles go to
    //      LDS in accumulator order; the row norms.
    //      Every wave: its unit of the state product (the MFMA work of the round is kept in
    //      this phase: fp32 MFMA and VALU from waves sharing a SIMD barely overlap).
    if (wv_u < Ly::GW) {
        v4f acc[RT][NT];
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
#pragma unroll
            for (int at = 0; at < NT; ++at) acc[rt][at] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int lc = 0; lc < LCG; ++lc) {
            const int q = wv_u + Ly::GW * lc;
            if (q < KC) {
                v4f av[RT];
#pragma unroll
                for (int rt = 0; rt < RT; ++rt)
                    av[rt] = *reinterpret_cast<const v4f *>(XQK + (16 * rt + l16) * SX + 16 * q + 4 * g4);
#pragma unroll
                for (int rt = 0; rt < RT; ++rt)
#pragma unroll
                    for (int at = 0; at < NT; ++at) acc[rt][at] = mfma4(av[rt], av[at], acc[rt][at]);
            }
        }
        float *gp = scr + Ly::OFF_GRAM + wave * Ly::GRAM_TILES * 256;
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
#pragma unroll
            for (int at = 0; at < NT; ++at) *reinterpret_cast<v4f *>(gp + ((rt * NT + at) * 64 + lane) * 4) = acc[rt][at];
        if (tid < 2 * NP) {
            float sq = s_ssq[tid][0];
            if constexpr (Ly::NPART > 1) sq += s_ssq[tid][1];
            s_r[tid] = inv_norm(sq);
        }
    } else if constexpr (Ly::SPLIT_W) {
        // waves 4..7, beside the Gram products: the bf16 parts of the raw [K; Q] rows into the
        // staging area, dead since the conv
        convert_rows(tid - 256);
    }
    if constexpr (Ly::SPLIT_W) lds_barrier();  // the bf16 parts are complete
    state_product();
    // (32 nodes: by every wave, once its product is done -- 146-147 against 151 us on the stress
    // layer; 16 nodes: by waves 4..7, 19.8 against 20.4-20.8 us at 16 lanes)
    if constexpr (FUSED && WIDE && WINV)
        if (NP == 32 || wv_u >= 4) write_windows();
    lds_barrier();

    // the replay-log header (g, k^) of every node, once per lane and value head (jb == 0), by
    // 256 threads (t = 0..255): wide workgroups from waves 0..3 in the solve phase, the others
    // from waves 4..7 beside the epilogue (its stores go out beside the epilogue's)
    auto write_log_header = [&](int t) {
        float *logc = args.replay_log + ((int64_t)c * N * Hv + h) * R;
        for (int f = t; f < nvc * (DK / 4); f += 256) {
            const int i = f / (DK / 4), e4 = f - i * (DK / 4);
            float sq = s_ssq[i][0];
            if constexpr (Ly::NPART > 1) sq += s_ssq[i][1];
            float *lrow = logc + (int64_t)i * Hv * R;
            __builtin_nontemporal_store(*reinterpret_cast<const v4f *>(XQK + i * SX + 4 * e4) * inv_norm(sq),
                                        reinterpret_cast<v4u *>(lrow + 1 + 4 * e4));
            if (e4 == 0) __builtin_nontemporal_store(s_g[i], lrow);
        }
    };

    // ---- decayed, ancestor-masked, norm-scaled coefficients and per-node scales
    const float isd = 1.0f / sqrtf((float)DK);
    for (int p = tid; p < NP * NP; p += kThreads) {
        const int i = p / NP, a = p - i * NP;
        const bool on = (s_anc[i] >> a) & 1u;
        const int ln = ((i & 15) >> 2) * 16 + (a & 15), v = i & 3;
        const float *gk = scr + Ly::OFF_GRAM + ((((i >> 4) * NT + (a >> 4)) * 64 + ln) * 4 + v);  // k_i . k_a
        const float *gqk =
            scr + Ly::OFF_GRAM + (((((NT + (i >> 4)) * NT) + (a >> 4)) * 64 + ln) * 4 + v);  // q_i . k_a
        float skk = 0.f, sqk = 0.f;
#pragma unroll
        for (int w = 0; w < Ly::GW; ++w) {
            skk += gk[w * Ly::GRAM_TILES * 256];
            sqk += gqk[w * Ly::GRAM_TILES * 256];
        }
        const float r = on ? fast_exp((float)(s_L[i] - s_L[a])) * s_r[a] : 0.f;
        Lm[i * SG + a] = (on && a != i) ? r * skk * (s_r[i] * s_beta[i]) : 0.f;
        Cq[i * SG + a] = r * sqk * (s_r[NP + i] * isd);
    }
    if (tid < NP) {
        s_gk[tid] = s_G[tid] * s_r[tid];
        s_gq[tid] = s_G[tid] * s_r[NP + tid] * isd;
    }
    lds_barrier();

    // ---- waves 4..7: T = (I + Lm)^-1 by forward substitution.  Waves nt < CT: the KS and
    //      QS tiles of value columns j0 + 16nt.. from the unit partials, and rhs.
    v4f rhs[NT], qs[NT];
    // rhs from this wave's KS tile (v, beta and the decay-norm scales are in LDS)
    auto form_rhs = [&](int mt, int jj, const v4f &ks) {
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const int i = 16 * mt + 4 * g4 + v;
            rhs[mt][v] = s_beta[i] * (Vl[i * SV + jj] - s_gk[i] * ks[v]);
        }
    };
    if (wv_u < 4) {
        if constexpr (WIDE) write_log_header(tid);  // (these waves have nothing else here)
        else if (wave < CT) {
            const int nt = wave, jj = 16 * nt + l16;
#pragma unroll
            for (int mt = 0; mt < NT; ++mt) {
                v4f ks = {0.f, 0.f, 0.f, 0.f};
                qs[mt] = ks;
#pragma unroll
                for (int kp = 0; kp < KP; ++kp) {
                    const float *pp = scr + Ly::OFF_UNIT + (kp * CT + nt) * Ly::UNIT + lane * 4;
                    ks += *reinterpret_cast<const v4f *>(pp + mt * 256);
                    qs[mt] += *reinterpret_cast<const v4f *>(pp + (NT + mt) * 256);
                }
                form_rhs(mt, jj, ks);
            }
        }
    } else if constexpr (NP == 16) {
        // waves 4..7, four columns each: lane = (column a, row i) over rows of 16 lanes
        const int a = 4 * (wv_u - 4) + (lane >> 4), i = lane & 15;
        v4f Lr[4];
#pragma unroll
        for (int k4 = 0; k4 < 4; ++k4) Lr[k4] = *reinterpret_cast<const v4f *>(Lm + i * SG + 4 * k4);
        Tm[i * SG + a] = bcast_solve(i == a ? 1.f : 0.f, Lr, std::make_integer_sequence<int, 16>());
    } else {
        // 32 nodes, waves 4..7: the diagonal 16 x 16 blocks T11 = (I + L11)^-1 and
        // T22 = (I + L22)^-1 by the same substitution (block pb on pass pb), T12 = 0; then
        // T21 = -T22 L21 T11 below
#pragma unroll
        for (int pb = 0; pb < 2; ++pb) {
            const int a = 4 * (wv_u - 4) + (lane >> 4), i = lane & 15, o = 16 * pb;
            v4f Lr[4];
#pragma unroll
            for (int k4 = 0; k4 < 4; ++k4) Lr[k4] = *reinterpret_cast<const v4f *>(Lm + (o + i) * SG + o + 4 * k4);
            Tm[(o + i) * SG + o + a] = bcast_solve(i == a ? 1.f : 0.f, Lr, std::make_integer_sequence<int, 16>());
            if (pb == 0) Tm[i * SG + 16 + a] = 0.f;
        }
    }
    if constexpr (NP == 32) lds_barrier();  // the diagonal blocks of T are complete
    if constexpr (NP == 32) {
        // wave 4: M = L21 T11, then T21 = -T22 M (two 16 x 16 products; the accumulator of the
        // first is the right operand of the second)
        if (wv_u == 4) {
            v4f t11;
#pragma unroll
            for (int e = 0; e < 4; ++e) t11[e] = Tm[(4 * g4 + e) * SG + l16];
            const v4f zero = {0.f, 0.f, 0.f, 0.f};
            const v4f mm = mfma4(*reinterpret_cast<const v4f *>(Lm + (16 + l16) * SG + 4 * g4), t11, zero);
            const v4f t21 = mfma4(*reinterpret_cast<const v4f *>(Tm + (16 + l16) * SG + 16 + 4 * g4), mm, zero);
#pragma unroll
            for (int e = 0; e < 4; ++e) Tm[(16 + 4 * g4 + e) * SG + l16] = -t21[e];
        }
    }
    lds_barrier();

    // ---- epilogue: wave nt < CT owns value columns j0 + 16nt..: D = T rhs (delta rows,
    //      replay log), O = diag(gq) QS + Cq D (output).
    //      Column blocks: waves 4..7 write the replay-log header beside it.
    static_assert(WIDE || CT <= 4, "epilogue waves");
    static_assert(2 * NP * SV <= Ly::SCR, "output tiles fit the scratch");
    float *Ot = scr, *Dt = scr + NP * SV;  // output and delta rows of the block, [NP][SV] each
    if (wave < CT) {
        const int nt = wave, jj = 16 * nt + l16;
        if constexpr (WIDE) {  // KS and QS of this wave's column tile are its own tiles
#pragma unroll
            for (int mt = 0; mt < NT; ++mt) {
                form_rhs(mt, jj, sp[mt]);
                qs[mt] = sp[NT + mt];
            }
        }
        v4f dl[NT];
#pragma unroll
        for (int mt = 0; mt < NT; ++mt) {
            dl[mt] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kt = 0; kt < NT; ++kt)
                dl[mt] = mfma4(*reinterpret_cast<const v4f *>(Tm + (16 * mt + l16) * SG + 16 * kt + 4 * g4), rhs[kt],
                               dl[mt]);
        }
#pragma unroll
        for (int mt = 0; mt < NT; ++mt) {
            v4f o;
#pragma unroll
            for (int v = 0; v < 4; ++v) o[v] = s_gq[16 * mt + 4 * g4 + v] * qs[mt][v];
#pragma unroll
            for (int kt = 0; kt < NT; ++kt)
                o = mfma4(*reinterpret_cast<const v4f *>(Cq + (16 * mt + l16) * SG + 16 * kt + 4 * g4), dl[kt], o);
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int i = 16 * mt + 4 * g4 + v;
                Ot[i * SV + jj] = o[v];
                Dt[i * SV + jj] = dl[mt][v];
            }
        }
    }
    if (!WIDE && wv_u >= 4 && jb == 0) write_log_header(tid - 256);
    lds_barrier();
    // output rows and the log's delta rows of the block, in 16-byte chunks from consecutive
    // lanes (whole lines per store instruction; a log row is 1 + d_k + d_v floats, so its
    // chunks are only 4-byte aligned)
    for (int f = tid; f < 2 * nvc * Q4; f += kThreads) {
        const bool is_out = f < nvc * Q4;
        const int ff = is_out ? f : f - nvc * Q4;
        const int i = ff / Q4, q4 = ff - i * Q4;
        const int64_t row = ((int64_t)c * N + i) * Hv + h;
        if (is_out)
            __builtin_nontemporal_store(*reinterpret_cast<const v4f *>(Ot + i * SV + 4 * q4),
                                        reinterpret_cast<v4f *>(args.out + row * DV + j0 + 4 * q4));
        else
            __builtin_nontemporal_store(*reinterpret_cast<const v4f *>(Dt + i * SV + 4 * q4),
                                        reinterpret_cast<v4u *>(args.replay_log + row * R + 1 + DK + j0 + 4 * q4));
    }
}

template <int DK, int DV, int NP, bool RAGGED, bool WIDE>
__global__ __launch_bounds__(kThreads) void tree_verify_kernel(const VerifyArgs args) {
    verify_body<DK, DV, NP, false, RAGGED, WIDE, false>(args);
}

// Commit windows of the fused route, written by workgroups of their own that run beside
// the verify workgroups of the same launch, so that these stores drain while the verify
// workgroups compute.  Workgroup b covers lane b / blocks_per_lane and a block of
// 4 * (kThreads / NP) channels; thread t covers node t / (kThreads / NP) and one 4-channel
// group (NP = 8 for trees of at most 8 nodes, the pages' width-8 chains, else the verify's
// padded node count).  The window of node i is the last 3 sources of its extended sequence, oldest
// first: the tokens of its parent and grandparent, or the slot's newest history columns
// in their place past the root, then the node's own tokens ("perf(qwen35): fuse the
// DFlash2 concurrent verify Gated DeltaNet route", Optimizations, first bullet).
// A node's windows are 3 * (kThreads / NP) consecutive 16-byte chunks; they go through a
// wave-private transpose in LDS so that each store instruction writes consecutive chunks
// from consecutive lanes (whole lines), which drains faster than 16-byte pieces at a
// 48-byte lane stride.  Nothing is written for a padding or invalid lane (the verify
// workgroups report it).
template <int NP, bool RAGGED>
__device__ __forceinline__ void window_body(const VerifyArgs &args, int b) {
    constexpr int GPB = kThreads / NP;  // 4-channel groups per workgroup
    const Dims d = args.d;
    const int N = d.N;
    const int bpl = (d.Ch + 4 * GPB - 1) / (4 * GPB);
    const int c = b / bpl, ch0 = (b - c * bpl) * 4 * GPB;
    const int tid = threadIdx.x, lane = tid & 63;
    const int i = tid / GPB, ch = ch0 + 4 * (tid % GPB);
    const int s = args.slot_ids[c];
    const int par = args.parents[(int64_t)c * N + (lane < N ? lane : 0)];  // lane j: parent of node j
    const int nv = RAGGED ? args.lane_nodes[c] : N;
    // the lane's validity, as the verify workgroups decide it
    int bad = (s < -1 || s >= d.P || nv < 0 || nv > N) ? 1 : 0;
    for (int o = lane; o < d.C; o += 64)
        if (o != c && args.slot_ids[o] == s) bad = 1;
    if (lane < nv && lane < N && (par < -1 || par >= lane)) bad = 1;
    if (s == -1 || __builtin_amdgcn_ballot_w64(bad)) return;  // uniform over the wave
    // absent nodes' parents are not checked: treat those nodes as root children so that no
    // address is formed from them (present nodes' ancestors are present)
    const int parv = lane < nv ? par : -1;
    const int ic = i < N ? i : 0;
    const int a1 = __shfl(parv, ic);
    const int a2s = __shfl(parv, a1 >= 0 ? a1 : 0);
    const int a2 = a1 >= 0 ? a2s : -1;
    // threads past the node count or the channel count load in-range rows and store nothing
    const int chc = ch < d.Ch ? ch : 0;
    const float *xr = args.x + (int64_t)c * N * d.Ch + chc;
    const float *hr = args.conv_hist + ((int64_t)s * d.Ch + chc) * 3;
    const v4f t3 = *reinterpret_cast<const v4f *>(xr + (int64_t)ic * d.Ch);
    v4f hraw[3];
#pragma unroll
    for (int e = 0; e < 3; ++e) hraw[e] = reinterpret_cast<const v4f *>(hr)[e];
    v4f hc[3];
    hist_columns(hraw, hc);
    const v4f x1 = *reinterpret_cast<const v4f *>(xr + (int64_t)(a1 >= 0 ? a1 : 0) * d.Ch);
    const v4f x2 = *reinterpret_cast<const v4f *>(xr + (int64_t)(a2 >= 0 ? a2 : 0) * d.Ch);
    const v4f t2 = a1 >= 0 ? x1 : hc[2];
    const v4f t1 = a1 >= 0 ? (a2 >= 0 ? x2 : hc[2]) : hc[1];
    // this thread's 12 window floats in the history layout [ch][3], as 3 chunks in LDS; the
    // GPB threads of node i (within one wave) then store the node's 3 * GPB chunks in order
    extern __shared__ float lds[];
    v4f *chunks = reinterpret_cast<v4f *>(lds);
    chunks[3 * tid] = v4f{t1.x, t2.x, t3.x, t1.y};
    chunks[3 * tid + 1] = v4f{t2.y, t3.y, t1.z, t2.z};
    chunks[3 * tid + 2] = v4f{t3.z, t1.w, t2.w, t3.w};
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    const int gi = tid % GPB;
    // (a buffer resource that ends at the row's last channel: chunks of channel groups past it
    // are dropped by the range check; immediate offsets, no per-store address arithmetic)
    const __amdgpu_buffer_rsrc_t wr = __builtin_amdgcn_make_buffer_rsrc(
        args.commit_win + (((int64_t)c * N + ic) * d.Ch + ch0) * 3, 0, (d.Ch - ch0) * 12, kRsrcWord3);
#pragma unroll
    for (int u = 0; u < 3; ++u) {
        const int j = GPB * u + gi;  // chunk j holds part j % 3 of channel group j / 3
        const v4f v = chunks[3 * (tid - gi) + j];
        if (i < nv) __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(v4i, v), wr, 16 * j, 0, kNonTemporal);
    }
}

// (16-node trees: two workgroups side by side on a CU -- a verify and a window workgroup, or two
// wide verify workgroups -- so at least four waves per SIMD, at most 128 VGPRs)
template <int DK, int DV, int NP, bool RAGGED, bool WIDE, bool WINV>
__global__ __launch_bounds__(kThreads, NP == 16 ? 4 : 1) void conv_tree_verify_kernel(const VerifyArgs args) {
    constexpr int NB = VerifyLayout<DK, DV, NP, true, WIDE, WINV>::NB;
    static_assert(kThreads * 12 <= VerifyLayout<DK, DV, NP, true, WIDE, WINV>::LDS_FLOATS, "window chunks fit the LDS");
    const int n_verify = NB * args.d.Hv * args.d.C;
    if ((int)blockIdx.x < n_verify)
        verify_body<DK, DV, NP, true, RAGGED, WIDE, WINV>(args);
    else if (args.d.N <= 8)  // present only when the verify workgroups do not write the windows
        window_body<8, RAGGED>(args, blockIdx.x - n_verify);  // chains of 8: a wave per node
    else
        window_body<NP, RAGGED>(args, blockIdx.x - n_verify);
}

template <int DK, int DV, int NP, bool FUSED, bool RAGGED, bool WIDE, bool WINV>
hipError_t launch(const VerifyArgs &a, hipStream_t stream) {
    using Ly = VerifyLayout<DK, DV, NP, FUSED, WIDE, WINV>;
    const size_t lds = sizeof(float) * Ly::LDS_FLOATS;
    // the LDS limit is a property of the kernel, set once (also keeps stream capture clean)
    const void *kernel = FUSED ? reinterpret_cast<const void *>(&conv_tree_verify_kernel<DK, DV, NP, RAGGED, WIDE, WINV>)
                               : reinterpret_cast<const void *>(&tree_verify_kernel<DK, DV, NP, RAGGED, WIDE>);
    static const hipError_t attr = hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (attr != hipSuccess) return attr;
    // fused: the window workgroups follow the verify workgroups
    const bool window_wgs = FUSED && !(WIDE && WINV);
    const int gpb = kThreads / (a.d.N <= 8 ? 8 : NP);  // window workgroups: 4-channel groups per workgroup
    const int grid = Ly::NB * a.d.Hv * a.d.C + (window_wgs ? a.d.C * ((a.d.Ch + 4 * gpb - 1) / (4 * gpb)) : 0);
    if constexpr (FUSED)
        hipLaunchKernelGGL((conv_tree_verify_kernel<DK, DV, NP, RAGGED, WIDE, WINV>), dim3(grid), dim3(kThreads), lds,
                           stream, a);
    else
        hipLaunchKernelGGL((tree_verify_kernel<DK, DV, NP, RAGGED, WIDE>), dim3(grid), dim3(kThreads), lds, stream, a);
    return hipGetLastError();
}

// Fused wide launches whose grid spans two or more workgroups per CU have the verify
// workgroups write the commit windows (windows_in_verify); otherwise window workgroups do.
template <int DK, int DV, int NP, bool WIDE>
hipError_t launch_variant(const VerifyArgs &a, hipStream_t stream) {
    const bool fused = a.x != nullptr;
    const bool ragged = a.lane_nodes != nullptr;
    if (!fused)
        return ragged ? launch<DK, DV, NP, false, true, WIDE, false>(a, stream)
                      : launch<DK, DV, NP, false, false, WIDE, false>(a, stream);
    if constexpr (WIDE)
        if (windows_in_verify(a.d))
            return ragged ? launch<DK, DV, NP, true, true, true, true>(a, stream)
                          : launch<DK, DV, NP, true, false, true, true>(a, stream);
    return ragged ? launch<DK, DV, NP, true, true, WIDE, false>(a, stream)
                  : launch<DK, DV, NP, true, false, WIDE, false>(a, stream);
}

template <int DK, int DV, bool WIDE>
hipError_t launch_wide(const VerifyArgs &a, hipStream_t stream) {
    return a.d.N <= 16 ? launch_variant<DK, DV, 16, WIDE>(a, stream) : launch_variant<DK, DV, 32, WIDE>(a, stream);
}

// The q/k conv, norms, Gram products and tree algebra of a (lane, value head) are repeated by
// each of its column blocks.  While the grid fits the chip in one pass (C * H_v < 256) the
// 64-column blocks give the parallelism; beyond it the launch is bound by arithmetic and one
// workgroup per (lane, value head) over all 128 columns does a third less of it per byte.
// (Between 128 and 256, where some CUs run two 64-column workgroups, the wide workgroups were
// measured slower even with the split state product: 10.1 against 9.6 us on 5 lanes x 32 heads.)
template <int DK, int DV>
hipError_t launch_np(const VerifyArgs &a, hipStream_t stream) {
    if constexpr (DV == 128)
        if (a.d.C * a.d.Hv >= 256) return launch_wide<DK, DV, true>(a, stream);
    return launch_wide<DK, DV, false>(a, stream);
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
