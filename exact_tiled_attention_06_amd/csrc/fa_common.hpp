// fa_common.hpp -- vector types, MFMA wrappers and small device helpers for gfx950.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>
#include <utility>

namespace fa {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Element-type tags of the two matrix-core input formats.
struct F16 {};
struct BF16 {};

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_inff();
// Initial running reference: finite and far below any score, so that the first
// tile always takes the rescale path and exp2(m_init - m_new) is exactly 0.
constexpr float kMInit = -1.0e30f;

// D(32x32, fp32) += A(32x16) * B(16x32) on the matrix cores.  Per lane l of
// the wave: A holds row l%32, k = 8*(l/32) .. +7; B holds column l%32,
// k = 8*(l/32) .. +7; D holds column l%32, rows 8*(r/4) + 4*(l/32) + r%4 for
// r = 0..15.
template <typename T>
__device__ __forceinline__ f32x16 mfma32x32x16(u32x4 a, u32x4 b, f32x16 c);

template <>
__device__ __forceinline__ f32x16 mfma32x32x16<F16>(u32x4 a, u32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}

template <>
__device__ __forceinline__ f32x16 mfma32x32x16<BF16>(u32x4 a, u32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// Two fp32 values -> one dword of two 16-bit values (x in the low half),
// rounded to nearest even (v_cvt_pk_f16_f32 / v_cvt_pk_bf16_f32).
template <typename T>
__device__ __forceinline__ uint32_t pack2(float x, float y);

template <>
__device__ __forceinline__ uint32_t pack2<F16>(float x, float y) {
    f32x2 v = {x, y};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, f16x2));
}

template <>
__device__ __forceinline__ uint32_t pack2<BF16>(float x, float y) {
    f32x2 v = {x, y};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

// Base-2 exponential and logarithm on the transcendental unit (v_exp_f32,
// v_log_f32).  exp2(-inf) = 0.
__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float log2_fast(float x) { return __builtin_amdgcn_logf(x); }

// Combine the two 32-lane halves of the wave: every lane l receives
// op(x[l % 32], x[32 + l % 32]).  v_permlane32_swap exchanges the upper half
// of one operand with the lower half of the other, so its two results hold,
// in every lane, the lower-half and the upper-half value of the column.
__device__ __forceinline__ float halves_max(float x) {
    uint32_t u = __builtin_bit_cast(uint32_t, x);
    auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    return fmaxf(__builtin_bit_cast(float, (uint32_t)r[0]), __builtin_bit_cast(float, (uint32_t)r[1]));
}

__device__ __forceinline__ float halves_sum(float x) {
    uint32_t u = __builtin_bit_cast(uint32_t, x);
    auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    return __builtin_bit_cast(float, (uint32_t)r[0]) + __builtin_bit_cast(float, (uint32_t)r[1]);
}

// f(std::integral_constant<int, 0>{}) ... f(std::integral_constant<int, N - 1>{}):
// a loop whose index is a compile-time constant in every iteration.
template <typename F, int... I>
__device__ __forceinline__ void static_for_impl(F& f, std::integer_sequence<int, I...>) {
    (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
    static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// Instruction classes of __builtin_amdgcn_sched_group_barrier masks.
constexpr int kSchedValu = 0x2;
constexpr int kSchedMfma = 0x8;

// Make a loaded value opaque to the optimiser, so that it stays in registers
// rather than being re-loaded from memory later when registers are scarce.
__device__ __forceinline__ void pin(u32x4& v) {
    asm volatile("" : "+v"(v[0]), "+v"(v[1]), "+v"(v[2]), "+v"(v[3]));
}

}  // namespace fa
