// fa_f32.hpp -- FlashAttention-2 forward for fp32 inputs (all arithmetic in fp32).
//
// The same Q-outer / K,V-inner online softmax as the matrix-core kernels, on the
// vector ALUs: a workgroup owns 64 query rows, one per lane, and its NW waves
// split the block's keys into contiguous slices.  Every lane of a wave needs the
// same key and value row at the same time, so K and V are read with wave-uniform
// addresses (scalar loads through the scalar cache) and enter the FMAs as
// scalar operands; each dot product runs as 8 independent partial sums.  Keys
// are taken BN at a time: scores, their maximum, one rescale of the running
// state, then the weighted sum of value rows ("从零训练语言模型（第二部分）",
// section "安全 / 在线 softmax").  The softmax weights stay fp32 for the P*V
// product: there is no lower-precision matrix input to round to.  The waves'
// partial results are merged with the log-sum-exp rule through LDS (the merge
// the saved lse enables: "T5 讲解", section ⑥), and wave 0 writes O and lse.
// Causal workgroups stop at their last row's diagonal and mask only the keys
// that cross it ("Triton 实现", section "Causal Mask 的处理"; "T5 讲解",
// section ⑤); a sliding window (left, right) narrows every row's keys to
// i - left .. i + right the same way, and grouped heads read K/V head bh / G
// ("Inside FlashAttention", section 6.1).
#pragma once

#include "fa_common.hpp"

namespace fa {

constexpr int F32_BM = 64;  // query rows per workgroup (one per lane)
// The running reference m moves only when a key's scaled score exceeds it by
// more than this (log2 units), so weights stay below 2^8 and the exact
// rescale runs a few times per row instead of at every key.
constexpr float kF32Margin = 8.0f;

// Waves per workgroup (key slices); the merge buffer, (NW-1) * (D+2) floats
// per lane, must fit in LDS.
template <int D>
struct F32Cfg {
    static constexpr int NW = D == 128 ? 4 : 8;
    static constexpr int NT = 64 * NW;
};

template <int D, bool CAUSAL>
__global__ __attribute__((amdgpu_flat_work_group_size(F32Cfg<D>::NT, F32Cfg<D>::NT)))
void fa_fwd_f32_kernel(const float* __restrict__ Q, const float* __restrict__ K,
                       const float* __restrict__ V, float* __restrict__ O, float* __restrict__ LSE,
                       int Sq, int Sk, int BH, int n_qblk, int G, int wl, int wr, float c) {
    constexpr int NW = F32Cfg<D>::NW;
    constexpr int XW = D + 2;  // floats per lane in the merge: acc, m, l
    __shared__ float xch[(NW - 1) * XW * 64];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wg = blockIdx.x;
    const int bh = wg % BH;
    const int rank = wg / BH;
    const int qblk = CAUSAL ? (n_qblk - 1 - rank) : rank;
    const int q0 = qblk * F32_BM;
    const int qrow = q0 + lane;
    const int64_t head = (int64_t)bh * Sq * D;
    const int64_t kvhead = (int64_t)(bh / G) * Sk * D;  // grouped heads: G query heads per K/V head
    const float* kh = K + kvhead;
    const float* vh = V + kvhead;

    float q[D], acc[D];
    const int qsrc = min(qrow, Sq - 1);
#pragma unroll
    for (int d = 0; d < D; ++d) {
        q[d] = Q[head + (int64_t)qsrc * D + d];
        acc[d] = 0.f;
    }
    float m_run = kMInit, l_run = 0.f;

    // Keys of row i: lo(i) .. hi(i) -- at most i when causal, i - wl .. i + wr
    // within a window (wl, wr = -1: no limit on that side), never past Sk - 1.
    // The block's rows together see klo .. khi; this wave takes the slice
    // [kb, ke) of it (empty when the range is: a window can leave rows no key
    // when there are fewer keys than queries).
    const int qlast = min(q0 + F32_BM, Sq) - 1;
    const int klo = wl >= 0 ? max(0, q0 - wl) : 0;
    const int khi = min(min(CAUSAL ? qlast : Sk - 1, wr >= 0 ? qlast + wr : Sk - 1), Sk - 1);
    const int nk = khi - klo + 1;
    const int kb = klo + wave * nk / NW;
    const int ke = klo + (wave + 1) * nk / NW;
    const int lo = wl >= 0 ? max(0, qrow - wl) : 0;
    const int hi = min(min(CAUSAL ? qrow : Sk - 1, wr >= 0 ? qrow + wr : Sk - 1), Sk - 1);
    for (int key = kb; key < ke; ++key) {
        const float* kr = kh + (int64_t)key * D;
        float part[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) part[i] = 0.f;
#pragma unroll
        for (int d = 0; d < D; ++d) part[d & 7] = __builtin_fmaf(q[d], kr[d], part[d & 7]);
        float sc = (((part[0] + part[1]) + (part[2] + part[3])) + ((part[4] + part[5]) + (part[6] + part[7]))) * c;
        if (key < lo || key > hi) sc = kNegInf;
        // move the reference only when a weight would exceed 2^kF32Margin
        if (__builtin_amdgcn_ballot_w64(sc > m_run + kF32Margin)) {
            const float m_new = fmaxf(m_run, sc);
            const float alpha = exp2_fast(m_run - m_new);
            m_run = m_new;
            l_run *= alpha;
#pragma unroll
            for (int d = 0; d < D; ++d) acc[d] *= alpha;
        }
        const float p = exp2_fast(sc - m_run);
        l_run += p;
        const float* vr = vh + (int64_t)key * D;
#pragma unroll
        for (int d = 0; d < D; ++d) acc[d] = __builtin_fmaf(p, vr[d], acc[d]);
    }

    // ---- merge the waves' slices: M = max m, l = sum 2^(m-M) l, acc likewise ----
    if (wave > 0) {
        float* x = xch + (wave - 1) * XW * 64 + lane;
#pragma unroll
        for (int d = 0; d < D; ++d) x[d * 64] = acc[d];
        x[D * 64] = m_run;
        x[(D + 1) * 64] = l_run;
    }
    __syncthreads();
    if (wave != 0) return;
    float mx = m_run;
#pragma unroll
    for (int w = 1; w < NW; ++w) mx = fmaxf(mx, xch[((w - 1) * XW + D) * 64 + lane]);
    const float a0 = exp2_fast(m_run - mx);
    float l = l_run * a0;
#pragma unroll
    for (int d = 0; d < D; ++d) acc[d] *= a0;
#pragma unroll
    for (int w = 1; w < NW; ++w) {
        const float* x = xch + (w - 1) * XW * 64 + lane;
        const float aw = exp2_fast(x[D * 64] - mx);
        l += aw * x[(D + 1) * 64];
#pragma unroll
        for (int d = 0; d < D; ++d) acc[d] = __builtin_fmaf(aw, x[d * 64], acc[d]);
    }

    if (qrow < Sq) {
        // (a row with no key has l = 0 and acc = 0: O = 0, lse = ln2 * log2 0 = -inf)
        const float inv = l > 0.f ? 1.0f / l : 0.f;
#pragma unroll
        for (int d = 0; d < D; ++d) O[head + (int64_t)qrow * D + d] = acc[d] * inv;
        LSE[(int64_t)bh * Sq + qrow] = kLn2 * (mx + log2_fast(l));
    }
}

}  // namespace fa
