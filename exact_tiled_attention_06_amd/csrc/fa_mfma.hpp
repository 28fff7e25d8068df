// fa_mfma.hpp -- FlashAttention-2 forward for fp16 / bf16 inputs on the gfx950 matrix cores.
//
// One workgroup owns one block of BM = NW * 32 * QB query rows of one
// (batch, head) and streams that head's keys and values through LDS in tiles
// of BN rows (query blocks outer, key/value blocks inner: "Triton 实现",
// sections "Grid 与并行策略" and "Q-outer 主循环"; "T5 讲解", section ②).
// Each wave owns 32 * QB whole query rows, so no softmax statistics cross a
// wave ("Inside FlashAttention", section 4.3, split-Q).
//
// Per wave and key tile:
//   S^T = K_tile * Q^T        32x32x16 MFMAs, fp32 accumulators.  Computing the
//                             transpose puts one query per lane column, so a row
//                             maximum or sum is a reduction inside the lane plus
//                             one exchange between the two wave halves.
//   mask                      only on tiles that cross the causal diagonal or the
//                             end of the sequence; off-band tiles take no compare
//                             ("Triton 实现", section "Causal Mask 的处理";
//                             "T5 讲解", section ⑤).
//   online softmax            exp2 form with c = scale * log2(e) ("Triton 实现",
//                             section "内层循环"): the tile's row maximum m_t = c *
//                             rowmax(S); when m_t exceeds the running reference
//                             m by more than TAU (log2 units) for any row of the
//                             wave, every row moves to m_new = max(m, m_t) and
//                             rescales l and acc by alpha = exp2(m - m_new)
//                             ("从零训练语言模型（第二部分）", section "安全 / 在线
//                             softmax"); p = exp2(S*c - m), l += rowsum(p).
//                             Keeping m until the maximum has grown by TAU leaves
//                             every p <= 2^TAU, far inside fp16 / bf16 / fp32
//                             range, and saves the rescale on almost every tile.
//   O^T += V^T * P^T          P rounded (nearest-even) to the input type,
//                             fp32 accumulation.
// The epilogue divides by l once and writes O and lse = ln2 * (m + log2 l), the
// natural-log form ("Inside FlashAttention", sections 2.4 and 4.1).
//
// Data movement: Q fragments live in VGPRs for the whole loop ("T5 讲解",
// section ③).  K and V tiles go from HBM straight into LDS with 16-byte
// global_load_lds transfers (no VGPR staging), double-buffered in separately
// declared LDS arrays: tile t+1 is in flight while tile t is consumed, and one
// barrier per tile publishes it.  Both tiles are stored row-major with an XOR
// swizzle of 16-byte chunks per row (applied on the HBM side of the transfer),
// chosen so that the K operand reads (ds_read_b128, one 16-byte chunk of 32
// consecutive rows) and the V operand reads (ds_read_b64_tr_b16, 8-byte pieces
// of four consecutive rows, transposed across lanes) hit distinct banks.
#pragma once

#include "fa_common.hpp"

#define FA_LDS __attribute__((address_space(3)))

namespace fa {

typedef short s16x4 __attribute__((ext_vector_type(4)));

template <int D_, bool CAUSAL_, int QB_, int NW_, int BN_>
struct MfmaConfig {
    static constexpr int D = D_;
    static constexpr bool CAUSAL = CAUSAL_;
    static constexpr int QB = QB_;          // 32-query column blocks per wave
    static constexpr int NW = NW_;          // waves per workgroup
    static constexpr int BN = BN_;          // keys per LDS tile
    static constexpr int NT = NW * 64;      // threads per workgroup
    static constexpr int BMW = 32 * QB;     // query rows per wave
    static constexpr int BM = NW * BMW;     // query rows per workgroup
    static constexpr int KB = BN / 32;      // 32-key blocks per tile
    static constexpr int KS = D / 16;       // k-steps of S^T = K Q^T (16 dims each)
    static constexpr int DB = (D + 31) / 32;  // 32-row blocks of O^T
    static constexpr int RB = 2 * D;        // bytes per K / V row
    static constexpr int CPR = D / 8;       // 16-byte chunks per row
    static constexpr int TILE = BN * RB;    // bytes per K or V tile
    static constexpr int LOADS = TILE / 1024;            // 1 KiB wave transfers per tile
    static constexpr int LOADS_PER_WAVE = LOADS / NW;
    static_assert(D == 16 || D == 32 || D == 64 || D == 128, "head dim");
    static_assert(BN % 32 == 0, "BN must be a multiple of 32");
    static_assert(LOADS % NW == 0 && LOADS_PER_WAVE >= 1, "tile transfers must split evenly over waves");
    static_assert(2 * 2 * TILE <= 160 * 1024, "LDS");
};

// Rescale threshold (log2 units): p = exp2(S*c - m) stays <= 2^TAU.
constexpr float kTau = 8.0f;
// Initial running reference: finite and far below any score, so that
// exp2(m_init - m_new) underflows to exactly 0 and no inf - inf arises.
constexpr float kMInit = -1.0e30f;

// XOR swizzle of the 16-byte chunk index within a K row: one chunk read by 16
// consecutive rows lands in 16 distinct (row parity, chunk) bank groups.
template <int D>
__device__ __forceinline__ int swz_k(int row) {
    constexpr int SH = D == 16 ? 3 : D == 32 ? 2 : D == 64 ? 1 : 0;
    return (row >> SH) & (D / 8 - 1);
}

// XOR swizzle within a V row: the 8-byte pieces that four consecutive rows
// contribute to one transposed read cover distinct banks.
template <int D>
__device__ __forceinline__ int swz_v(int row) {
    if constexpr (D == 64) return ((row >> 1) & 1) * 4;
    else if constexpr (D == 128) return (row & 3) * 4;
    else return 0;
}

__device__ __forceinline__ void wait_vmcnt0() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Issue this wave's share of the HBM -> LDS transfers of one K or V tile
// (rows k0 .. k0+BN-1 of head `src`).  Rows at or beyond S repeat row S-1:
// their keys are masked to -inf, so their finite values only ever meet p = 0.
template <typename Cfg, bool ISV>
__device__ __forceinline__ void load_tile(FA_LDS char* dst, const uint16_t* __restrict__ src, int k0, int S,
                                          int wave, int lane) {
    constexpr int D = Cfg::D;
#pragma unroll
    for (int i = 0; i < Cfg::LOADS_PER_WAVE; ++i) {
        const int inst = wave * Cfg::LOADS_PER_WAVE + i;
        const int slot = inst * 64 + lane;
        const int row = slot / Cfg::CPR;
        const int p = slot % Cfg::CPR;
        const int c = p ^ (ISV ? swz_v<D>(row) : swz_k<D>(row));
        const int grow = min(k0 + row, S - 1);
        const uint16_t* g = src + (int64_t)grow * D + c * 8;
        __builtin_amdgcn_global_load_lds((const void*)g, (FA_LDS void*)(dst + inst * 1024), 16, 0, 0);
    }
}

template <typename T, typename Cfg>
__global__ __attribute__((amdgpu_flat_work_group_size(Cfg::NT, Cfg::NT), amdgpu_waves_per_eu(2)))
void fa_fwd_mfma_kernel(const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
                        const uint16_t* __restrict__ V, uint16_t* __restrict__ O, float* __restrict__ LSE,
                        int S, int BH, int n_qblk, float c) {
    constexpr int D = Cfg::D, QB = Cfg::QB, KB = Cfg::KB, KS = Cfg::KS, DB = Cfg::DB;
    constexpr int BN = Cfg::BN, BM = Cfg::BM, BMW = Cfg::BMW, RB = Cfg::RB;
    constexpr bool CAUSAL = Cfg::CAUSAL;

    __shared__ __attribute__((aligned(1024))) char k_lds0[Cfg::TILE];
    __shared__ __attribute__((aligned(1024))) char k_lds1[Cfg::TILE];
    __shared__ __attribute__((aligned(1024))) char v_lds0[Cfg::TILE];
    __shared__ __attribute__((aligned(1024))) char v_lds1[Cfg::TILE];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int n = lane & 31;  // MFMA output column = this lane's query within a 32-block
    const int h = lane >> 5;  // wave half

    // Workgroup -> (head, query block).  Heads vary fastest so that the
    // workgroups of one head land on one XCD (dispatch is round-robin over the
    // 8 XCDs) and share its K/V in that XCD's L2; causal blocks go longest first.
    const int wg = blockIdx.x;
    const int bh = wg % BH;
    const int rank = wg / BH;
    const int qblk = CAUSAL ? (n_qblk - 1 - rank) : rank;
    const int q0 = qblk * BM;
    const int qw = q0 + wave * BMW;

    const int64_t head = (int64_t)bh * S * D;
    const uint16_t* qh = Q + head;
    const uint16_t* kh = K + head;
    const uint16_t* vh = V + head;

    const int kend = CAUSAL ? min(q0 + BM, S) : S;
    const int ntiles = (kend + BN - 1) / BN;

    // Tile 0 in flight before anything else.
    load_tile<Cfg, false>((FA_LDS char*)k_lds0, kh, 0, S, wave, lane);
    load_tile<Cfg, true>((FA_LDS char*)v_lds0, vh, 0, S, wave, lane);

    // Q^T operand fragments: lane holds Q[query][16ks + 8h .. +7].  Rows beyond
    // S repeat row S-1; their outputs are never stored.
    u32x4 qf[QB][KS];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        const int qrow = min(qw + qb * 32 + n, S - 1);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
            qf[qb][ks] = *reinterpret_cast<const u32x4*>(qh + (int64_t)qrow * D + ks * 16 + h * 8);
    }

    // Per-lane LDS byte offsets of the operand reads (constant over tiles).
    // K: row n of each 32-key block, logical chunk 2ks + h.
    int offk[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) offk[ks] = n * RB + (((2 * ks + h) ^ swz_k<D>(n)) * 16);
    // V (transposed reads): within a 16-lane group g = lane/16, lane r reads row
    // 4h + r/4 (+ block offsets) at dims 32db + 16(g&1) + 4(r&3) .. +3; after the
    // transpose, lane r holds dim 32db + 16(g&1) + r of four consecutive keys.
    const int r16 = lane & 15;
    const int g16 = lane >> 4;
    const int vrow = 4 * h + (r16 >> 2);
    int offv[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) {
        const int dim = (32 * db + 16 * (g16 & 1) + 4 * (r16 & 3)) % D;
        offv[db] = vrow * RB + (((dim >> 3) ^ swz_v<D>(vrow)) * 16) + (dim & 7) * 2;
    }

    float m_run[QB], l_run[QB];
    f32x16 oacc[QB][DB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        m_run[qb] = kMInit;
        l_run[qb] = 0.f;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int r = 0; r < 16; ++r) oacc[qb][db][r] = 0.f;
    }
    const f32x16 zero = {};

    auto step = [&](int t, FA_LDS char* kcur, FA_LDS char* vcur, FA_LDS char* knext, FA_LDS char* vnext) {
        const int k0 = t * BN;
        wait_vmcnt0();
        __syncthreads();
        if (t + 1 < ntiles) {
            load_tile<Cfg, false>(knext, kh, k0 + BN, S, wave, lane);
            load_tile<Cfg, true>(vnext, vh, k0 + BN, S, wave, lane);
        }
        // A wave whose last query precedes the tile's first key has nothing to do here.
        if (CAUSAL && k0 > qw + BMW - 1) return;

        // ---- S^T = K Q^T --------------------------------------------------------
        f32x16 s[QB][KB];
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                const u32x4 kf = *reinterpret_cast<const FA_LDS u32x4*>(kcur + kb * 32 * RB + offk[ks]);
#pragma unroll
                for (int qb = 0; qb < QB; ++qb)
                    s[qb][kb] = mfma32x32x16<T>(kf, qf[qb][ks], ks == 0 ? zero : s[qb][kb]);
            }
        }

        // ---- mask: only tiles that cross the diagonal or the end of the sequence --
        if ((CAUSAL && k0 + BN - 1 > qw) || k0 + BN > S) {
#pragma unroll
            for (int qb = 0; qb < QB; ++qb) {
                const int last = CAUSAL ? min(qw + qb * 32 + n, S - 1) : S - 1;
#pragma unroll
                for (int kb = 0; kb < KB; ++kb) {
                    // key of register r = k0 + 32kb + 4h + 8(r/4) + r%4; visible iff key <= last
                    const int lim = last - (k0 + kb * 32 + 4 * h);
#pragma unroll
                    for (int r = 0; r < 16; ++r)
                        if (8 * (r >> 2) + (r & 3) > lim) s[qb][kb][r] = kNegInf;
                }
            }
        }

        // ---- online softmax --------------------------------------------------------
        bool grow = false;
        float m_tile[QB];
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
            float a = s[qb][0][0], b = s[qb][0][1];
#pragma unroll
            for (int kb = 0; kb < KB; ++kb)
#pragma unroll
                for (int r = (kb == 0 ? 2 : 0); r < 16; r += 4) {
                    a = fmaxf(fmaxf(a, s[qb][kb][r]), s[qb][kb][r + 1]);
                    b = fmaxf(fmaxf(b, s[qb][kb][r + 2]), s[qb][kb][r + 3]);
                }
            m_tile[qb] = halves_max(fmaxf(a, b)) * c;
            grow |= m_tile[qb] > m_run[qb] + kTau;
        }
        if (__builtin_amdgcn_ballot_w64(grow) != 0) {
#pragma unroll
            for (int qb = 0; qb < QB; ++qb) {
                const float m_new = fmaxf(m_run[qb], m_tile[qb]);
                const float alpha = exp2_fast(m_run[qb] - m_new);
                m_run[qb] = m_new;
                l_run[qb] *= alpha;
#pragma unroll
                for (int db = 0; db < DB; ++db)
#pragma unroll
                    for (int r = 0; r < 16; ++r) oacc[qb][db][r] *= alpha;
            }
        }

        u32x4 pk[QB][KB][2];
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
            const float neg_m = -m_run[qb];
            float rs0 = 0.f, rs1 = 0.f;
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) {
#pragma unroll
                for (int r = 0; r < 16; r += 4) {
                    const float p0 = exp2_fast(__builtin_fmaf(s[qb][kb][r + 0], c, neg_m));
                    const float p1 = exp2_fast(__builtin_fmaf(s[qb][kb][r + 1], c, neg_m));
                    const float p2 = exp2_fast(__builtin_fmaf(s[qb][kb][r + 2], c, neg_m));
                    const float p3 = exp2_fast(__builtin_fmaf(s[qb][kb][r + 3], c, neg_m));
                    rs0 += p0 + p1;
                    rs1 += p2 + p3;
                    // B operand of P*V: slot i of MFMA j holds register 8j + i
                    const int j = r >> 3, w = (r & 7) >> 1;
                    pk[qb][kb][j][w] = pack2<T>(p0, p1);
                    pk[qb][kb][j][w + 1] = pack2<T>(p2, p3);
                }
            }
            l_run[qb] += rs0 + rs1;
        }

        // ---- O^T += V^T P^T ---------------------------------------------------------
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
#pragma unroll
            for (int j = 0; j < 2; ++j) {
#pragma unroll
                for (int db = 0; db < DB; ++db) {
                    // A operand: V[keys 32kb + 16j + {4h..4h+3, 8+4h..8+4h+3}][dim 32db + n]
                    FA_LDS char* base = vcur + (kb * 32 + 16 * j) * RB + offv[db];
                    const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((FA_LDS s16x4*)base);
                    const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((FA_LDS s16x4*)(base + 8 * RB));
                    const u32x2 lo2 = __builtin_bit_cast(u32x2, lo), hi2 = __builtin_bit_cast(u32x2, hi);
                    const u32x4 vf = {lo2[0], lo2[1], hi2[0], hi2[1]};
#pragma unroll
                    for (int qb = 0; qb < QB; ++qb)
                        oacc[qb][db] = mfma32x32x16<T>(vf, pk[qb][kb][j], oacc[qb][db]);
                }
            }
        }
    };

    for (int t = 0; t < ntiles; t += 2) {
        step(t, (FA_LDS char*)k_lds0, (FA_LDS char*)v_lds0, (FA_LDS char*)k_lds1, (FA_LDS char*)v_lds1);
        if (t + 1 < ntiles)
            step(t + 1, (FA_LDS char*)k_lds1, (FA_LDS char*)v_lds1, (FA_LDS char*)k_lds0, (FA_LDS char*)v_lds0);
    }

    // ---- epilogue: O = acc / l, lse = ln2 * (m + log2 l) ---------------------------
    uint16_t* oh = O + head;
    float* lh = LSE + (int64_t)bh * S;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        const float l = halves_sum(l_run[qb]);
        const float inv = 1.0f / l;
        const int qrow = qw + qb * 32 + n;
        if (qrow < S) {
#pragma unroll
            for (int db = 0; db < DB; ++db)
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const int d = db * 32 + 8 * g + 4 * h;
                    if (d < D) {
                        u32x2 w;
                        w[0] = pack2<T>(oacc[qb][db][4 * g + 0] * inv, oacc[qb][db][4 * g + 1] * inv);
                        w[1] = pack2<T>(oacc[qb][db][4 * g + 2] * inv, oacc[qb][db][4 * g + 3] * inv);
                        *reinterpret_cast<u32x2*>(oh + (int64_t)qrow * D + d) = w;
                    }
                }
            if (h == 0) lh[qrow] = kLn2 * (m_run[qb] + log2_fast(l));
        }
    }
}

}  // namespace fa
