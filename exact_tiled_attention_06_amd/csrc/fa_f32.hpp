// fa_f32.hpp -- FlashAttention-2 forward for fp32 inputs (all arithmetic in fp32).
//
// The same Q-outer / K,V-inner online softmax as the matrix-core kernel, on the
// vector ALUs: one thread owns one query row (its q, its fp32 accumulator and
// its running m, l stay in registers), a workgroup of 64 threads owns 64
// consecutive rows, and each key/value tile of 32 rows is staged once in LDS
// and read by all 64 threads as broadcasts.  The softmax weights stay fp32
// for the P*V product: there is no lower-precision matrix input to round to.
// Causal workgroups stop at their last row's diagonal and mask only the tiles
// that cross it ("Triton 实现", section "Causal Mask 的处理"; "T5 讲解",
// section ⑤).
#pragma once

#include "fa_common.hpp"

namespace fa {

constexpr int F32_BM = 64;  // query rows per workgroup (one wave)
constexpr int F32_BN = 32;  // keys per LDS tile

template <int D, bool CAUSAL>
__global__ __attribute__((amdgpu_flat_work_group_size(F32_BM, F32_BM)))
void fa_fwd_f32_kernel(const float* __restrict__ Q, const float* __restrict__ K,
                       const float* __restrict__ V, float* __restrict__ O, float* __restrict__ LSE,
                       int S, int BH, int n_qblk, float c) {
    __shared__ float ks[F32_BN][D];
    __shared__ float vs[F32_BN][D];

    const int tid = threadIdx.x;
    const int wg = blockIdx.x;
    const int bh = wg % BH;
    const int rank = wg / BH;
    const int qblk = CAUSAL ? (n_qblk - 1 - rank) : rank;
    const int q0 = qblk * F32_BM;
    const int qrow = q0 + tid;
    const int64_t head = (int64_t)bh * S * D;

    float q[D], acc[D];
#pragma unroll
    for (int d = 0; d < D; ++d) {
        q[d] = (qrow < S) ? Q[head + (int64_t)qrow * D + d] : 0.f;
        acc[d] = 0.f;
    }
    float m_run = kNegInf, l_run = 0.f;

    const int kend = CAUSAL ? min(q0 + F32_BM, S) : S;
    for (int k0 = 0; k0 < kend; k0 += F32_BN) {
        // stage K and V rows k0 .. k0+31 (zero beyond S); coalesced over d
        for (int e = tid; e < F32_BN * D; e += F32_BM) {
            const int r = e / D, d = e % D;
            const bool ok = k0 + r < S;
            ks[r][d] = ok ? K[head + (int64_t)(k0 + r) * D + d] : 0.f;
            vs[r][d] = ok ? V[head + (int64_t)(k0 + r) * D + d] : 0.f;
        }
        __syncthreads();

        float s[F32_BN];
        float mx = kNegInf;
#pragma unroll
        for (int j = 0; j < F32_BN; ++j) {
            float dot = 0.f;
#pragma unroll
            for (int d = 0; d < D; ++d) dot = __builtin_fmaf(q[d], ks[j][d], dot);
            const int key = k0 + j;
            const bool hidden = (key >= S) || (CAUSAL && key > qrow);
            s[j] = hidden ? kNegInf : dot;
            mx = fmaxf(mx, s[j]);
        }
        const float m_new = fmaxf(m_run, mx * c);
        const float m_use = (m_new == kNegInf) ? 0.f : m_new;
        const float alpha = exp2_fast(m_run - m_use);
        m_run = m_new;
        float rs = 0.f;
#pragma unroll
        for (int d = 0; d < D; ++d) acc[d] *= alpha;
#pragma unroll
        for (int j = 0; j < F32_BN; ++j) {
            const float p = exp2_fast(__builtin_fmaf(s[j], c, -m_use));
            rs += p;
#pragma unroll
            for (int d = 0; d < D; ++d) acc[d] = __builtin_fmaf(p, vs[j][d], acc[d]);
        }
        l_run = l_run * alpha + rs;
        __syncthreads();
    }

    if (qrow < S) {
        const float inv = 1.0f / l_run;
#pragma unroll
        for (int d = 0; d < D; ++d) O[head + (int64_t)qrow * D + d] = acc[d] * inv;
        LSE[(int64_t)bh * S + qrow] = kLn2 * (m_run + log2_fast(l_run));
    }
}

}  // namespace fa
