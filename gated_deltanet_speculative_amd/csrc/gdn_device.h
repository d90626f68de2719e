// Device-side helpers shared by the gfx950 kernels: vector types, the LDS-only
// barrier and the fast transcendental forms of the norm and gate functions.
#pragma once

#include <hip/hip_runtime.h>

#include <utility>

#include "gdn_verify.h"

namespace gdn {

typedef float v4f __attribute__((ext_vector_type(4)));
// Four consecutive floats at a 4-byte-aligned address, one dwordx4 access (the HSA
// runtime runs in unaligned access mode): replay-log rows are 1 + d_k + d_v floats
// long, so their slices carry no 16-byte alignment.
typedef float v4u __attribute__((ext_vector_type(4), aligned(4)));

// Workgroup barrier for LDS communication only: waits for this wave's LDS operations,
// not for its outstanding global loads, so requested data keeps streaming in.
__device__ inline void lds_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0), vmcnt and expcnt left open
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

typedef __bf16 bf2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf8 __attribute__((ext_vector_type(8)));

// x = hi + lo + r with hi = bf16(x), lo = bf16(x - hi) (round to nearest even) and
// |r| <= 2^-18 |x|: three bf16 products hi.hi + hi.lo + lo.hi, accumulated in float32, give a
// product to about 2^-17 relative (the dropped lo.lo and r terms).  By pairs: one packed
// conversion gives both hi parts, whose float values are the packed word's halves moved to
// the top (a shift and a mask), so a pair costs six VALU instructions instead of eight.
template <int K>
__device__ inline void split_bf16(const float (&x)[K], __bf16 (&h)[K], __bf16 (&l)[K]) {
    static_assert(K % 2 == 0, "pairs");
#pragma unroll
    for (int e = 0; e < K; e += 2) {
        unsigned u = __builtin_bit_cast(unsigned, bf2{(__bf16)x[e], (__bf16)x[e + 1]});
        asm("" : "+v"(u));  // (opaque: otherwise u << 16 is folded into a second conversion of x[e])
        const bf2 hp = __builtin_bit_cast(bf2, u);
        const float h0 = __builtin_bit_cast(float, u << 16), h1 = __builtin_bit_cast(float, u & 0xffff0000u);
        const bf2 lp = {(__bf16)(x[e] - h0), (__bf16)(x[e + 1] - h1)};
        h[e] = hp[0];
        h[e + 1] = hp[1];
        l[e] = lp[0];
        l[e + 1] = lp[1];
    }
}

// 1 / max(|x|, 1e-6) from |x|^2, and the gate nonlinearities, on the hardware
// transcendental units (about 1 ulp each; the outputs they feed carry a 2e-4 tolerance)
__device__ inline float inv_norm(float sq) { return fminf(__builtin_amdgcn_rsqf(sq), 1e6f); }
__device__ inline float fast_exp(float x) { return __builtin_amdgcn_exp2f(x * 1.4426950408889634f); }
__device__ inline float fast_softplus(float x) {
    return fmaxf(x, 0.f) + 0.6931471805599453f * __builtin_amdgcn_logf(1.0f + fast_exp(-fabsf(x)));
}
__device__ inline float fast_sigmoid(float x) { return __builtin_amdgcn_rcpf(1.0f + fast_exp(-x)); }
__device__ inline float fast_silu(float z) { return z * __builtin_amdgcn_rcpf(1.0f + fast_exp(-z)); }

// Four steps of v_mfma_f32_16x16x4_f32 over one 16-wide chunk of a contraction.  Within the
// chunk, lane group g = lane / 16 supplies index 4g + s in step s (a permutation shared by
// both operands), so a 16 x 16 accumulator tile -- lane holding rows 4g..4g+3 of column
// lane % 16 -- is directly the right operand of a following product.
__device__ inline v4f mfma4(v4f a, v4f b, v4f acc) {
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[0], b[0], acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[1], b[1], acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[2], b[2], acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[3], b[3], acc, 0, 0, 0);
    return acc;
}

// x[lane] + x[lane - SH] within each row of 16 lanes (0 past the row start): DPP row_shr
template <int SH>
__device__ inline float add_row_shr(float x) {
    return x + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x110 + SH, 0xF, 0xF, true));
}

// the same for a double (both halves moved by DPP; lanes before the row start add 0.0)
template <int SH>
__device__ inline double add_row_shr(double x) {
    const long long b = __double_as_longlong(x);
    const int lo = __builtin_amdgcn_update_dpp(0, (int)b, 0x110 + SH, 0xF, 0xF, true);
    const int hi = __builtin_amdgcn_update_dpp(0, (int)(b >> 32), 0x110 + SH, 0xF, 0xF, true);
    return x + __longlong_as_double((long long)((unsigned long long)(unsigned)hi << 32 | (unsigned)lo));
}

// value of lane K of each row of 16 lanes, in every lane of the row (DPP row_newbcast)
template <int K>
__device__ inline float row_bcast(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x150 + K, 0xF, 0xF, false));
}

// Forward substitution of one column of (I + L) t = e_a over a row of 16 lanes, lane i
// holding t_i (initially [i == a]) and row i of the strictly lower L: at step k, t_k is
// final and is broadcast to the row; rows above k are unchanged since L[i][k] = 0 there.
template <int... K>
__device__ inline float bcast_solve(float t, const v4f *Lr, std::integer_sequence<int, K...>) {
    ((t = fmaf(-Lr[K / 4][K % 4], row_bcast<K>(t), t)), ...);
    return t;
}

// Sum over aligned groups of W consecutive lanes (W = 4, 8 or 16; W = 16 is a DPP row),
// left in the last lane of each group; with W = 16 also the inclusive prefix sum along
// each row of 16 lanes.
template <int W, typename F>
__device__ inline F group_sum_last(F x) {
    x = add_row_shr<1>(x);
    x = add_row_shr<2>(x);
    if constexpr (W >= 8) x = add_row_shr<4>(x);
    if constexpr (W >= 16) x = add_row_shr<8>(x);
    return x;
}

// ---- slot preflight of the calls that write the pools directly (plain decode step,
//      prefill): slot range and duplicate slots over every non-padding lane

constexpr int kBitmapSlots = 65536;  // duplicate-slot check via an LDS bitmap up to this pool size

// The slot ids of lanes tid, tid + THREADS, ... (for slot_preflight), loaded ahead of the
// bulk loads so the preflight does not wait behind them.
template <int THREADS>
struct LaneSlotsT {
    static constexpr int kPerThread = (GDN_MAX_SEQS + THREADS - 1) / THREADS;
    int v[kPerThread];
    __device__ LaneSlotsT(const int32_t *__restrict__ slot_ids, int C) {
#pragma unroll
        for (int k = 0; k < kPerThread; ++k)  // (a uniform test: no load issued past the lane count)
            v[k] = THREADS * k < C ? slot_ids[min((int)threadIdx.x + THREADS * k, C - 1)] : -1;
    }
};

// GDN_STATUS_SLOT_RANGE / GDN_STATUS_SLOT_DUP over every non-padding lane, with an LDS
// bitmap of kBitmapSlots / 32 words (or a scan for larger pools) and one LDS word.  Every
// thread of the workgroup must call it (it contains barriers); all receive the same bits.
template <int THREADS>
__device__ int slot_preflight(const LaneSlotsT<THREADS> &ls, const int32_t *__restrict__ slot_ids, int C, int P,
                              unsigned int *bitmap, int *word) {
    const bool use_bitmap = P <= kBitmapSlots;
    if (use_bitmap)
        for (int w = threadIdx.x; w < (P + 31) / 32; w += THREADS) bitmap[w] = 0u;
    if (threadIdx.x == 0) *word = 0;
    lds_barrier();
    int bits = 0;
#pragma unroll
    for (int k = 0; k < LaneSlotsT<THREADS>::kPerThread; ++k) {
        const int t = threadIdx.x + THREADS * k;
        const int st = ls.v[k];
        if (t >= C || st == -1) continue;
        if (st < -1 || st >= P) {
            bits |= GDN_STATUS_SLOT_RANGE;
        } else if (use_bitmap) {
            const unsigned int m = 1u << (st & 31);
            if (atomicOr(&bitmap[st >> 5], m) & m) bits |= GDN_STATUS_SLOT_DUP;
        } else {
            for (int o = 0; o < C; ++o)
                if (o != t && slot_ids[o] == st) bits |= GDN_STATUS_SLOT_DUP;
        }
    }
    if (bits) atomicOr(word, bits);
    lds_barrier();
    return *word;
}

}  // namespace gdn
