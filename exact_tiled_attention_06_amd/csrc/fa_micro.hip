// fa_micro.hip -- issue-rate microbenchmarks of the gfx950 instructions the
// attention kernels are built from: the 32x32x16 fp16 matrix product, the
// base-2 exponential, fp32 multiply-add and the fp32 -> 2 x fp16 packing, each
// (and a few others a softmax could use: the fp16 exponential, packed fp16
// add, three-input max), each alone and interleaved in one wave or split
// across the two waves of a SIMD.
//
// The attention loop per attended (query, key) pair costs 4 * D matrix-core
// FLOPs and one exponential plus a few vector ALU operations ("Inside
// FlashAttention", section 4.1: the non-matmul work costs far more per FLOP
// than the matmuls; "从零训练语言模型（第二部分）", section "先做性能分析":
// profile where the time goes), so the rates measured here bound it from the
// vector side.  Every probe runs a fixed straight-line body of register-only
// instructions (inline assembly, so that the compiler keeps the written order)
// in a loop and reads the shader clock (s_memtime) around it.  No probe
// touches memory inside the timed loop; the only store is each wave's cycle
// count.  The values the instructions compute are never read: only the issue
// timing is of interest.
#include <stdint.h>

#include <hip/hip_runtime.h>

#include "../../include/fa_micro.h"

namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// One 32x32x16 fp16 product with the accumulator in arch VGPRs or in AGPRs.
template <bool AGPR>
__device__ __forceinline__ void mfma(f32x16& c, const u32x4& a, const u32x4& b) {
    if constexpr (AGPR)
        asm volatile("v_mfma_f32_32x32x16_f16 %0, %1, %2, %0" : "+a"(c) : "v"(a), "v"(b));
    else
        asm volatile("v_mfma_f32_32x32x16_f16 %0, %1, %2, %0" : "+v"(c) : "v"(a), "v"(b));
}

// One vector instruction of kind OP on register x (y, z: extra operands).
template <int OP>
__device__ __forceinline__ void valu(float& x, float y, float z) {
    if constexpr (OP == FA_MICRO_OP_EXP)
        asm volatile("v_exp_f32 %0, %0" : "+v"(x));
    else if constexpr (OP == FA_MICRO_OP_FMA)
        asm volatile("v_fma_f32 %0, %0, %1, %2" : "+v"(x) : "v"(y), "v"(z));
    else if constexpr (OP == FA_MICRO_OP_ADD)
        asm volatile("v_add_f32 %0, %0, %1" : "+v"(x) : "v"(y));
    else if constexpr (OP == FA_MICRO_OP_CVT)
        asm volatile("v_cvt_pk_f16_f32 %0, %0, %1" : "+v"(x) : "v"(y));
    else if constexpr (OP == FA_MICRO_OP_EXP16)
        asm volatile("v_exp_f16 %0, %0" : "+v"(x));
    else if constexpr (OP == FA_MICRO_OP_PKADD16)
        asm volatile("v_pk_add_f16 %0, %0, %1" : "+v"(x) : "v"(y));
    else
        asm volatile("v_max3_f32 %0, %0, %1, %2" : "+v"(x) : "v"(y), "v"(z));
}

// The bodies.  Products: 8 matrix products round-robin over 4 independent
// accumulators.  Vector: 8 * K vector instructions of kind OP (32 when K = 0)
// round-robin over 16 registers, so no vector instruction waits on the one
// before it.  Mixed: each of the 8 products followed by K vector instructions.
template <bool AGPR>
__device__ __forceinline__ void body_products(f32x16 (&acc)[4], const u32x4& a, const u32x4& b) {
#pragma unroll
    for (int m = 0; m < 8; ++m) mfma<AGPR>(acc[m & 3], a, b);
}

template <int OP, int K>
__device__ __forceinline__ void body_vector(float (&x)[16], float y, float z) {
    constexpr int N = K == 0 ? 32 : 8 * K;
#pragma unroll
    for (int i = 0; i < N; ++i) valu<OP>(x[i & 15], y, z);
}

template <bool AGPR, int OP, int K>
__device__ __forceinline__ void body_mixed(f32x16 (&acc)[4], const u32x4& a, const u32x4& b, float (&x)[16], float y,
                                           float z) {
#pragma unroll
    for (int m = 0; m < 8; ++m) {
        mfma<AGPR>(acc[m & 3], a, b);
#pragma unroll
        for (int i = 0; i < K; ++i) valu<OP>(x[(m * K + i) & 15], y, z);
    }
}

// What each wave of the workgroup runs (wave w sits on SIMD w % 4):
//   FA_MICRO_MIXED     the mixed body on every wave;
//   FA_MICRO_PRODUCTS  products only on every wave;
//   FA_MICRO_VECTOR    vector instructions only on every wave;
//   FA_MICRO_SPLIT     products on waves 0-3, vector work on waves 4-7 (eight
//                      waves: two per SIMD, with complementary work).
template <bool AGPR, int OP, int K>
__global__ __launch_bounds__(512) void micro_kernel(uint64_t* __restrict__ cycles, int mode, int iters, float seed) {
    const int wave = threadIdx.x >> 6;
    f32x16 acc[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[j][r] = seed * (float)(r + j);
    u32x4 a, b;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        a[r] = __float_as_uint(seed) ^ (uint32_t)(threadIdx.x + r);
        b[r] = __float_as_uint(seed) ^ (uint32_t)(threadIdx.x * 3 + r);
    }
    float x[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) x[i] = seed * (float)(i + 1);
    const float y = seed * 0.5f, z = seed * 0.25f;
    const int role = mode == FA_MICRO_SPLIT ? (wave < 4 ? FA_MICRO_PRODUCTS : FA_MICRO_VECTOR) : mode;
    __syncthreads();
    const uint64_t t0 = __builtin_amdgcn_s_memtime();
    if (role == FA_MICRO_MIXED) {
        for (int it = 0; it < iters; ++it) body_mixed<AGPR, OP, K>(acc, a, b, x, y, z);
    } else if (role == FA_MICRO_PRODUCTS) {
        for (int it = 0; it < iters; ++it) body_products<AGPR>(acc, a, b);
    } else {
        for (int it = 0; it < iters; ++it) body_vector<OP, K>(x, y, z);
    }
    const uint64_t t1 = __builtin_amdgcn_s_memtime();
    // keep the results live (never true for the seeds the host passes)
    float sink = 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j) sink += acc[j][0];
#pragma unroll
    for (int i = 0; i < 16; ++i) sink += x[i];
    if ((threadIdx.x & 63) == 0) cycles[blockIdx.x * (blockDim.x >> 6) + wave] = t1 - t0;
    if (sink == 12345.678f) cycles[0] = 0;
}

template <bool AGPR, int OP, int K>
int launch(int mode, int waves, int iters, uint64_t* cycles, hipStream_t s) {
    (void)hipGetLastError();
    hipLaunchKernelGGL((micro_kernel<AGPR, OP, K>), dim3(1), dim3(64 * waves), 0, s, cycles, mode, iters, 1.0e-3f);
    return hipGetLastError() == hipSuccess ? FA_MICRO_OK : FA_MICRO_ERR_LAUNCH;
}

template <bool AGPR, int OP>
int by_k(int k, int mode, int waves, int iters, uint64_t* cycles, hipStream_t s) {
    switch (k) {
        case 0: return launch<AGPR, OP, 0>(mode, waves, iters, cycles, s);
        case 1: return launch<AGPR, OP, 1>(mode, waves, iters, cycles, s);
        case 2: return launch<AGPR, OP, 2>(mode, waves, iters, cycles, s);
        case 4: return launch<AGPR, OP, 4>(mode, waves, iters, cycles, s);
        case 8: return launch<AGPR, OP, 8>(mode, waves, iters, cycles, s);
        default: return launch<AGPR, OP, 16>(mode, waves, iters, cycles, s);
    }
}

template <bool AGPR>
int by_op(int op, int k, int mode, int waves, int iters, uint64_t* cycles, hipStream_t s) {
    switch (op) {
        case FA_MICRO_OP_EXP: return by_k<AGPR, FA_MICRO_OP_EXP>(k, mode, waves, iters, cycles, s);
        case FA_MICRO_OP_FMA: return by_k<AGPR, FA_MICRO_OP_FMA>(k, mode, waves, iters, cycles, s);
        case FA_MICRO_OP_ADD: return by_k<AGPR, FA_MICRO_OP_ADD>(k, mode, waves, iters, cycles, s);
        case FA_MICRO_OP_CVT: return by_k<AGPR, FA_MICRO_OP_CVT>(k, mode, waves, iters, cycles, s);
        case FA_MICRO_OP_EXP16: return by_k<AGPR, FA_MICRO_OP_EXP16>(k, mode, waves, iters, cycles, s);
        case FA_MICRO_OP_PKADD16: return by_k<AGPR, FA_MICRO_OP_PKADD16>(k, mode, waves, iters, cycles, s);
        default: return by_k<AGPR, FA_MICRO_OP_MAX3>(k, mode, waves, iters, cycles, s);
    }
}

}  // namespace

extern "C" int fa_micro(int op, int k, int agpr, int mode, int waves, int iters, uint64_t* cycles, void* stream) {
    if (op < FA_MICRO_OP_EXP || op > FA_MICRO_OP_MAX3) return FA_MICRO_ERR_ARG;
    if (k != 0 && k != 1 && k != 2 && k != 4 && k != 8 && k != 16) return FA_MICRO_ERR_ARG;
    if (agpr != 0 && agpr != 1) return FA_MICRO_ERR_ARG;
    if (mode < FA_MICRO_MIXED || mode > FA_MICRO_SPLIT) return FA_MICRO_ERR_ARG;
    if (waves < 1 || waves > 8 || (mode == FA_MICRO_SPLIT && waves != 8)) return FA_MICRO_ERR_ARG;
    if (iters < 1 || iters > (1 << 20)) return FA_MICRO_ERR_ARG;
    if (!cycles) return FA_MICRO_ERR_ARG;
    hipStream_t s = (hipStream_t)stream;
    return agpr ? by_op<true>(op, k, mode, waves, iters, cycles, s) : by_op<false>(op, k, mode, waves, iters, cycles, s);
}
