// Device-side helpers shared by the gfx950 kernels: vector types, the LDS-only
// barrier and the fast transcendental forms of the norm and gate functions.
#pragma once

#include <hip/hip_runtime.h>

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

// 1 / max(|x|, 1e-6) from |x|^2, and the gate nonlinearities, on the hardware
// transcendental units (about 1 ulp each; the outputs they feed carry a 2e-4 tolerance)
__device__ inline float inv_norm(float sq) { return fminf(__builtin_amdgcn_rsqf(sq), 1e6f); }
__device__ inline float fast_exp(float x) { return __builtin_amdgcn_exp2f(x * 1.4426950408889634f); }
__device__ inline float fast_softplus(float x) {
    return fmaxf(x, 0.f) + 0.6931471805599453f * __builtin_amdgcn_logf(1.0f + fast_exp(-fabsf(x)));
}
__device__ inline float fast_sigmoid(float x) { return __builtin_amdgcn_rcpf(1.0f + fast_exp(-x)); }
__device__ inline float fast_silu(float z) { return z * __builtin_amdgcn_rcpf(1.0f + fast_exp(-z)); }

}  // namespace gdn
