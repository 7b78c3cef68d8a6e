// rgdr_common.h -- small device helpers shared by the library's kernels (not part of the
// C ABI). bf16 values travel as raw 16-bit patterns; fp32 is the arithmetic type.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "rgdr.h"

namespace rgdr {

// bf16 -> fp32 is exact: the bf16 pattern is the top half of the fp32 pattern.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
    return __uint_as_float(static_cast<uint32_t>(h) << 16);
}

// fp32 -> bf16, round to nearest even (gfx950 converts in hardware: v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint16_t f32_to_bf16(float x) {
    return __builtin_bit_cast(uint16_t, static_cast<__bf16>(x));
}
// Two values, one instruction (v_cvt_pk_bf16_f32 with both sources), lo in the low half.
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{lo, hi}, bf16x2_t));
}

// Gate arithmetic ("com.microsoft.LinearAttentionGate" README, Description), fp32:
// softplus(x) = ln(1 + e^x) in the overflow-safe form, sigmoid(x) = 1 / (1 + e^-x).
__device__ __forceinline__ float softplus_f32(float x) {
    return x > 0.f ? x + log1pf(expf(-x)) : log1pf(expf(x));
}
__device__ __forceinline__ float sigmoid_f32(float x) { return 1.0f / (1.0f + expf(-x)); }

// Short branch-free forms for the fused decode, where the gate of each item sits on the path
// between its state tile's arrival and its reduction. They use the hardware exp2/log2 (about
// 1 ulp each) and keep log1p accurate for small arguments by the correction
// log1p(e) = log(u) * e / (u - 1) with u = 1 + e rounded (Goldberg, "What Every Computer
// Scientist Should Know About Floating-Point Arithmetic", Theorem 4). Error: a few ulp of fp32,
// far below the bf16 state's rounding. Infinities and NaN pass as in the precise forms.
__device__ __forceinline__ float softplus_fast(float x) {
    const float e = __expf(-fabsf(x));  // (0, 1]
    const float u = 1.0f + e;
    const float d = u - 1.0f;
    const float l = d == 0.f ? e : __logf(u) * (e * __builtin_amdgcn_rcpf(d));
    return fmaxf(x, 0.f) + l;
}
__device__ __forceinline__ float sigmoid_fast(float x) {
    return __builtin_amdgcn_rcpf(1.0f + __expf(-x));
}

// A gate input element held as raw bits: fp32 (the bits themselves) or fp16 (low 16 bits).
template <bool F16>
__device__ __forceinline__ float gate_value(uint32_t bits) {
    if constexpr (F16)
        return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(bits)));
    else
        return __uint_as_float(bits);
}

__host__ __device__ __forceinline__ bool aligned(const void *p, uintptr_t a) {
    return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0;
}

}  // namespace rgdr
