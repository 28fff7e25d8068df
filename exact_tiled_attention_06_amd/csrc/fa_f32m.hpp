// fa_f32m.hpp -- FlashAttention-2 forward for fp32 inputs on the matrix cores
// (v_mfma_f32_32x32x2_f32: fp32 operands, fp32 accumulation; all arithmetic in
// fp32).
//
// The same Q-outer / K,V-inner online softmax as the fp16 / bf16 kernels
// ("Triton 实现", sections "Q-outer 主循环" and "内层循环"; "T5 讲解", sections
// ②-⑥), with a workgroup per block of 32 query rows whose NW waves split the
// block's key tiles into contiguous slices and merge their partial results
// with the log-sum-exp rule through LDS at the end (the merge the saved lse
// enables: "T5 讲解", section ⑥; "Inside FlashAttention", section 2.4).
//
// Per 32-key tile a wave computes S^T = K Q^T on the matrix cores, one query
// per lane column (lane n + 32h holds keys 8(r/4) + 4h + r%4, r = 0..15, of
// query n): the k-index of each 32x32x2 step pairs dim s of the lower half of
// the head dimension with dim D/2 + s of the upper half, so a lane's K and Q
// operands are D/2 contiguous floats of one row.  The weights P stay fp32
// (there is no narrower matrix input to round them to) and O^T += V^T P^T
// takes register r of P as the B operand of step r, with V at the matching
// key as the A operand.  The running reference m follows every tile's row
// maximum exactly (one rescale of O and l per tile: cheap beside the fp32
// MFMAs).  Masks follow each row's key range lo(i) .. hi(i) (causal: keys up
// to i; a window (left, right): i - left .. i + right; never past S_k - 1), so
// causal, windowed, grouped-head (K/V head bh / G) and S_q != S_k problems
// share one kernel.  K and V operands come straight from HBM / L2 into
// registers: no tile is shared between waves, which walk different keys.
#pragma once

#include "fa_common.hpp"

namespace fa {

__device__ __forceinline__ f32x16 mfma32x32x2f32(float a, float b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

// Waves per workgroup (key slices of a 32-row block) and the register budget:
// D = 128 needs more than 256 registers per lane, so it runs one wave per
// SIMD.
template <int D>
struct F32mCfg {
    static constexpr int NW = D == 128 ? 4 : 8;
    static constexpr int NT = 64 * NW;
    static constexpr int HD = D / 2;           // S^T steps (dims per lane half)
    static constexpr int DB = (D + 31) / 32;   // 32-dim blocks of O^T
    static constexpr int OCC = D == 128 ? 1 : 2;
    static constexpr int XW = DB * 16 + 2;     // floats per lane in the merge: O^T, m, l
};

template <int D, bool CAUSAL>
__global__ __attribute__((amdgpu_flat_work_group_size(F32mCfg<D>::NT, F32mCfg<D>::NT),
                          amdgpu_waves_per_eu(F32mCfg<D>::OCC, F32mCfg<D>::OCC)))
void fa_fwd_f32m_kernel(const float* __restrict__ Q, const float* __restrict__ K, const float* __restrict__ V,
                        float* __restrict__ O, float* __restrict__ LSE, int Sq, int Sk, int BH, int n_qblk, int G,
                        int wl, int wr, float c) {
    using C = F32mCfg<D>;
    constexpr int NW = C::NW, HD = C::HD, DB = C::DB, XW = C::XW;
    __shared__ float xch[(NW - 1) * XW * 64];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int n = lane & 31;
    const int h = lane >> 5;

    // heads vary fastest; causal blocks longest first
    const int wg = blockIdx.x;
    const int bh = wg % BH;
    const int rank = wg / BH;
    const int qblk = CAUSAL ? n_qblk - 1 - rank : rank;
    const int q0 = qblk * 32;
    const int64_t head = (int64_t)bh * Sq * D;
    const int64_t kvhead = (int64_t)(bh / G) * Sk * D;  // grouped heads: G query heads per K/V head
    const float* kh = K + kvhead;
    const float* vh = V + kvhead;

    // Keys of row i: lo(i) .. hi(i); both are nondecreasing in i, so the block
    // sees lo(q0) .. hi(last row), which its waves split by 32-key tiles.
    auto lo_of = [&](int i) { return wl >= 0 ? max(0, i - wl) : 0; };
    auto hi_of = [&](int i) { return min(min(CAUSAL ? i : Sk - 1, wr >= 0 ? i + wr : Sk - 1), Sk - 1); };
    const int qlast = min(q0 + 32, Sq) - 1;
    const int klo = lo_of(q0), khi = hi_of(qlast);
    const int t0 = klo / 32;
    const int ntiles = khi >= klo ? khi / 32 + 1 - t0 : 0;
    const int tb = t0 + wave * ntiles / NW;
    const int te = t0 + (wave + 1) * ntiles / NW;
    const int qrow = min(q0 + n, Sq - 1);
    const int lo = lo_of(qrow), hi = hi_of(qrow);

    // Q operand: dims h*D/2 .. +D/2-1 of this lane's query row
    float qf[HD];
    {
        const f32x4* src = reinterpret_cast<const f32x4*>(Q + head + (int64_t)qrow * D + h * HD);
#pragma unroll
        for (int i = 0; i < HD / 4; ++i) {
            const f32x4 x = src[i];
#pragma unroll
            for (int e = 0; e < 4; ++e) qf[4 * i + e] = x[e];
        }
    }

    float m_run = kMInit, l_run = 0.f;
    // two partial O^T sums (even and odd steps r) per 32-dim block, so that
    // consecutive P*V MFMAs never wait for each other
    f32x16 oacc[2][DB];
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int r = 0; r < 16; ++r) oacc[j][db][r] = 0.f;

    for (int t = tb; t < te; ++t) {
        const int k0 = t * 32;
        // operands: K row k0 + n (rows past S_k clamped: their scores are
        // masked), and V at the 16 keys of this lane's half, dim 32db + n (dims
        // past D wrap: those output rows are never stored)
        float kf[HD];
        {
            const f32x4* src = reinterpret_cast<const f32x4*>(kh + (int64_t)min(k0 + n, Sk - 1) * D + h * HD);
#pragma unroll
            for (int i = 0; i < HD / 4; ++i) {
                const f32x4 x = src[i];
#pragma unroll
                for (int e = 0; e < 4; ++e) kf[4 * i + e] = x[e];
            }
        }
        float vf[DB][16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const float* vrow = vh + (int64_t)min(k0 + 8 * (r >> 2) + 4 * h + (r & 3), Sk - 1) * D;
#pragma unroll
            for (int db = 0; db < DB; ++db) vf[db][r] = vrow[(32 * db + n) % D];
        }

        // S^T on two accumulators (even and odd steps), summed once
        f32x16 sa, sb;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            sa[r] = 0.f;
            sb[r] = 0.f;
        }
#pragma unroll
        for (int s = 0; s < HD; s += 2) {
            sa = mfma32x32x2f32(kf[s], qf[s], sa);
            sb = mfma32x32x2f32(kf[s + 1], qf[s + 1], sb);
        }

        // scores in the exp2 domain, masked outside lo .. hi; the exact online
        // softmax step: m to max(m, tile max), O and l rescaled by 2^(m_old - m)
        float p[16];
        float mx = kNegInf;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int key = k0 + 8 * (r >> 2) + 4 * h + (r & 3);
            float sc = (sa[r] + sb[r]) * c;
            if (key < lo || key > hi) sc = kNegInf;
            p[r] = sc;
            mx = fmaxf(mx, sc);
        }
        mx = halves_max(mx);
        const float m_new = fmaxf(m_run, mx);
        const float alpha = exp2_fast(m_run - m_new);
        m_run = m_new;
        float rs = 0.f;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            p[r] = exp2_fast(p[r] - m_new);
            rs += p[r];
        }
        l_run = l_run * alpha + rs;
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int db = 0; db < DB; ++db)
#pragma unroll
                for (int r = 0; r < 16; ++r) oacc[j][db][r] *= alpha;
#pragma unroll
        for (int r = 0; r < 16; ++r)
#pragma unroll
            for (int db = 0; db < DB; ++db) oacc[r & 1][db] = mfma32x32x2f32(vf[db][r], p[r], oacc[r & 1][db]);
    }

    // ---- merge the waves' slices: M = max m, l = sum 2^(m-M) l, O^T likewise ----
    f32x16 o[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) o[db] = oacc[0][db] + oacc[1][db];
    auto slot = [&](int w, int k) __attribute__((always_inline)) -> float& {
        return xch[((w - 1) * XW + k) * 64 + lane];
    };
    if (wave > 0) {
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int r = 0; r < 16; ++r) slot(wave, db * 16 + r) = o[db][r];
        slot(wave, DB * 16) = m_run;
        slot(wave, DB * 16 + 1) = l_run;
    }
    __syncthreads();
    if (wave != 0) return;
    float mw[NW];
    mw[0] = m_run;
    float mxw = m_run;
#pragma unroll
    for (int w = 1; w < NW; ++w) {
        mw[w] = slot(w, DB * 16);
        mxw = fmaxf(mxw, mw[w]);
    }
    const float a0 = exp2_fast(mw[0] - mxw);
    float l = l_run * a0;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[db][r] *= a0;
#pragma unroll
    for (int w = 1; w < NW; ++w) {
        const float aw = exp2_fast(mw[w] - mxw);
        l += aw * slot(w, DB * 16 + 1);
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int r = 0; r < 16; ++r) o[db][r] = __builtin_fmaf(aw, slot(w, db * 16 + r), o[db][r]);
    }
    l = halves_sum(l);

    const int orow = q0 + n;
    if (orow < Sq) {
        // (a row with no key has l = 0 and O = 0: O = 0, lse = ln2 * log2 0 = -inf)
        const float inv = l > 0.f ? 1.0f / l : 0.f;
        float* dst = O + head + (int64_t)orow * D;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int d = 32 * db + 8 * g + 4 * h;
                if (d < D) {
                    f32x4 x;
#pragma unroll
                    for (int e = 0; e < 4; ++e) x[e] = o[db][4 * g + e] * inv;
                    *reinterpret_cast<f32x4*>(dst + d) = x;
                }
            }
        if (h == 0) LSE[(int64_t)bh * Sq + orow] = kLn2 * (mxw + log2_fast(l));
    }
}

}  // namespace fa
