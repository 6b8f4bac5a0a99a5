// kda_common.h -- small device helpers shared by the KDA kernels (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kda {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half4 __attribute__((ext_vector_type(4)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef float float4v __attribute__((ext_vector_type(4)));
// 16-byte move unit.  A native vector type (unlike HIP's uint4 struct) keeps
// register arrays of it in VGPRs.
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// bf16 is carried as its raw 16-bit pattern.
struct bf16_t {
    uint16_t bits;
};

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16_t x) {
    return __builtin_bit_cast(float, (uint32_t)x.bits << 16);
}

// Workgroup barrier that orders LDS traffic only.  __syncthreads() also
// waits for every outstanding global load and store of the wave
// (vmcnt(0)), which would drain the prefetch queue and stall on store
// completion at every barrier.  No kernel here reads global data written by
// another thread of its workgroup, so waiting for LDS is sufficient.
__device__ __forceinline__ void lds_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Natural exponent through the hardware base-2 exponential.
__device__ __forceinline__ float exp_e(float x) {
    return __builtin_amdgcn_exp2f(x * 1.4426950408889634f);
}

// Input preparation helpers (see kda_prep in kda.h).
// softplus(x) = max(x, 0) + ln(1 + e^-|x|), the logarithm through the hardware
// base-2 log: 1 + e^-|x| lies in [1, 2], so the absolute error stays below
// 1e-7 (for very negative x the true value e^x may be lost below that).
__device__ __forceinline__ float softplus_f(float x) {
    return fmaxf(x, 0.f) + 0.6931471805599453f * __builtin_amdgcn_logf(1.f + exp_e(-fabsf(x)));
}
// 1 / (1 + e^-x) with the hardware reciprocal (about 1 ulp; 0 when e^-x
// overflows, 1 when it underflows).
__device__ __forceinline__ float sigmoid_f(float x) {
    return __builtin_amdgcn_rcpf(1.f + exp_e(-x));
}
// 1 / sqrt(s) for s > 0 and 0 for s == 0, so that a zero vector stays zero.
__device__ __forceinline__ float rnorm(float s) { return s > 0.f ? rsqrtf(s) : 0.f; }

// Lane permute within rows of 16 lanes (DPP), every lane active.
template <int CTRL>
__device__ __forceinline__ float dpp_f(float x) {
    return __builtin_bit_cast(
        float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false));
}
// Sum over aligned groups of W lanes (W a power of two, 2..64): pairs, quads,
// half rows and rows through DPP (after the quad steps every lane of a quad
// holds the quad sum, so the mirror permutes pair equal partial sums), then
// cross-row steps through lane shuffles.
template <int W>
__device__ __forceinline__ float group_sum(float x) {
    static_assert(W >= 2 && W <= 64 && (W & (W - 1)) == 0, "bad group");
    x += dpp_f<0xB1>(x);                     // quad_perm [1,0,3,2]: lane ^ 1
    if constexpr (W >= 4) x += dpp_f<0x4E>(x);   // quad_perm [2,3,0,1]: lane ^ 2
    if constexpr (W >= 8) x += dpp_f<0x141>(x);  // row_half_mirror
    if constexpr (W >= 16) x += dpp_f<0x140>(x); // row_mirror
    if constexpr (W >= 32) x += __shfl_xor(x, 16);
    if constexpr (W >= 64) x += __shfl_xor(x, 32);
    return x;
}

// Load 4 consecutive input elements (bf16 or fp32) as floats.
__device__ __forceinline__ float4v load4(const float* p) {
    return *reinterpret_cast<const float4v*>(p);
}
__device__ __forceinline__ float4v load4(const bf16_t* p) {
    uint2 u = *reinterpret_cast<const uint2*>(p);
    float4v r;
    r[0] = __builtin_bit_cast(float, u.x << 16);
    r[1] = __builtin_bit_cast(float, u.x & 0xffff0000u);
    r[2] = __builtin_bit_cast(float, u.y << 16);
    r[3] = __builtin_bit_cast(float, u.y & 0xffff0000u);
    return r;
}

}  // namespace kda
