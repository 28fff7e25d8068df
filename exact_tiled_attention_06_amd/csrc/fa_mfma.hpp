// fa_mfma.hpp -- FlashAttention-2 forward for fp16 / bf16 inputs on the gfx950 matrix cores.
//
// One workgroup owns one block of BM = NW * 32 * QB query rows of one
// (batch, head) and streams that head's keys and values through LDS in tiles
// of BN rows (query blocks outer, key/value blocks inner: "Triton 实现",
// sections "Grid 与并行策略" and "Q-outer 主循环"; "T5 讲解", section ②).
// Each wave owns 32 * QB whole query rows, so no softmax statistics cross a
// wave ("Inside FlashAttention", section 4.3, split-Q).
//
// Per wave and key tile the hot loop is
//   S^T = K_tile * Q^T        32x32x16 MFMAs, fp32 accumulators; computing the
//                             transpose puts one query per lane column, so a
//                             row maximum / sum is a reduction inside the lane
//                             plus one exchange between the two wave halves;
//   mask                      only on tiles that cross the causal diagonal or
//                             the end of the sequence (off-band tiles take no
//                             compare: "Triton 实现", section "Causal Mask 的
//                             处理"; "T5 讲解", section ⑤);
//   online softmax            m_new = max(m, rowmax(S) * c), p = exp2(S*c - m_new),
//                             alpha = exp2(m - m_new), l = alpha*l + rowsum(p),
//                             with c = scale * log2(e) ("Triton 实现", section
//                             "内层循环", the exp2 form; "T5 讲解", section ④);
//   O^T = alpha * O^T + V^T * P^T   P rounded to the input type, fp32 accumulate.
// The epilogue divides by l once and writes O and lse = ln2 * (m + log2 l),
// the natural-log form ("Inside FlashAttention", sections 2.4 and 4.1).
//
// Data movement: Q fragments live in VGPRs for the whole loop (read once,
// "T5 讲解", section ③).  K and V tiles are double-buffered in LDS: every
// thread loads its share of tile t+1 from HBM with 16-byte loads before the
// MFMAs of tile t and stores it to the other LDS buffer afterwards, so one
// barrier per tile suffices.  K is stored row-major (each MFMA operand read is
// one 16-byte LDS read); V is stored transposed (V^T[d][key]) with the keys of
// each 16-key group permuted so that the eight keys one lane contributes to a
// P*V MFMA are contiguous, again one 16-byte read.  LDS rows are padded by 16
// bytes so that reads of one 16-byte column across consecutive rows hit
// distinct banks.
#pragma once

#include "fa_common.hpp"

namespace fa {

template <typename T, int D_, bool CAUSAL_, int QB_, int NW_, int BN_>
struct MfmaConfig {
    static constexpr int D = D_;
    static constexpr bool CAUSAL = CAUSAL_;
    static constexpr int QB = QB_;                // 32-query column blocks per wave
    static constexpr int NW = NW_;                // waves per workgroup
    static constexpr int BN = BN_;                // keys per LDS tile
    static constexpr int NT = NW * 64;            // threads per workgroup
    static constexpr int BMW = 32 * QB;           // query rows per wave
    static constexpr int BM = NW * BMW;           // query rows per workgroup
    static constexpr int KB = BN / 32;            // 32-key blocks per tile
    static constexpr int KS = (D + 15) / 16;      // k-steps of S^T = K Q^T
    static constexpr int DB = (D + 31) / 32;      // 32-row blocks of O^T
    static constexpr int KROW = 2 * D + 16;       // bytes per padded K row in LDS
    static constexpr int VROW = 2 * BN + 16;      // bytes per padded V^T row in LDS
    static constexpr int KTILE = BN * KROW;       // bytes of one K tile
    static constexpr int VTILE = D * VROW;        // bytes of one V^T tile
    static constexpr int BUF = KTILE + VTILE;     // one LDS buffer
    static constexpr int LDS_BYTES = 2 * BUF;
    static constexpr int KCPR = D / 8;            // 16-byte chunks per K / V row in HBM
    static constexpr int K_UNITS = BN * KCPR;     // 16-byte K loads per tile
    static constexpr int K_PER_THREAD = (K_UNITS + NT - 1) / NT;
    static constexpr int V_UNITS = (BN / 2) * KCPR;   // (key pair, chunk) V loads per tile
    static constexpr int V_PER_THREAD = (V_UNITS + NT - 1) / NT;
    static_assert(D == 16 || D == 32 || D == 64 || D == 128, "head dim");
    static_assert(BN % 32 == 0, "BN must be a multiple of 32");
};

// Position of tile-local key k inside the permuted V^T row: bits 2 and 3 of k
// are exchanged, so that keys {4h..4h+3, 8+4h..8+4h+3} of every 16-key group
// occupy positions 8h..8h+7.
__device__ __forceinline__ int vt_pos(int k) {
    return (k & ~12) | ((k & 4) << 1) | ((k & 8) >> 1);
}

template <typename Cfg>
struct TileStage {
    u32x4 k[Cfg::K_PER_THREAD];
    u32x4 v[Cfg::V_PER_THREAD][2];
};

// HBM -> registers for key tile starting at key k0 of head base pointers kh, vh.
// Rows at or beyond S are zero-filled so that padded keys contribute exact zeros.
template <typename Cfg>
__device__ __forceinline__ void stage_load(TileStage<Cfg>& st, const uint16_t* __restrict__ kh,
                                           const uint16_t* __restrict__ vh, int k0, int S, int tid) {
    constexpr int D = Cfg::D;
#pragma unroll
    for (int i = 0; i < Cfg::K_PER_THREAD; ++i) {
        const int u = tid + i * Cfg::NT;
        const int row = u / Cfg::KCPR, ch = u % Cfg::KCPR;
        u32x4 val = {0u, 0u, 0u, 0u};
        if (u < Cfg::K_UNITS && k0 + row < S)
            val = *reinterpret_cast<const u32x4*>(kh + (int64_t)(k0 + row) * D + ch * 8);
        st.k[i] = val;
    }
#pragma unroll
    for (int i = 0; i < Cfg::V_PER_THREAD; ++i) {
        const int u = tid + i * Cfg::NT;
        const int pr = u / Cfg::KCPR, ch = u % Cfg::KCPR;
        const int row = 2 * pr;
        u32x4 a = {0u, 0u, 0u, 0u}, b = {0u, 0u, 0u, 0u};
        if (u < Cfg::V_UNITS) {
            if (k0 + row < S)
                a = *reinterpret_cast<const u32x4*>(vh + (int64_t)(k0 + row) * D + ch * 8);
            if (k0 + row + 1 < S)
                b = *reinterpret_cast<const u32x4*>(vh + (int64_t)(k0 + row + 1) * D + ch * 8);
        }
        st.v[i][0] = a;
        st.v[i][1] = b;
    }
}

// registers -> LDS buffer: K row-major (padded rows), V transposed and key-permuted.
template <typename Cfg>
__device__ __forceinline__ void stage_store(const TileStage<Cfg>& st, char* buf, int tid) {
#pragma unroll
    for (int i = 0; i < Cfg::K_PER_THREAD; ++i) {
        const int u = tid + i * Cfg::NT;
        if (u < Cfg::K_UNITS) {
            const int row = u / Cfg::KCPR, ch = u % Cfg::KCPR;
            *reinterpret_cast<u32x4*>(buf + row * Cfg::KROW + ch * 16) = st.k[i];
        }
    }
    char* vt = buf + Cfg::KTILE;
#pragma unroll
    for (int i = 0; i < Cfg::V_PER_THREAD; ++i) {
        const int u = tid + i * Cfg::NT;
        if (u < Cfg::V_UNITS) {
            const int pr = u / Cfg::KCPR, ch = u % Cfg::KCPR;
            const int pos = vt_pos(2 * pr);  // even; key 2*pr+1 lands at pos+1
            const u32x4 a = st.v[i][0], b = st.v[i][1];
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                // a[w] = (V[k][d], V[k][d+1]), b[w] = (V[k+1][d], V[k+1][d+1]) with d = 8ch + 2w
                const uint32_t lo = (a[w] & 0xffffu) | (b[w] << 16);          // (V[k][d],   V[k+1][d])
                const uint32_t hi = (a[w] >> 16) | (b[w] & 0xffff0000u);      // (V[k][d+1], V[k+1][d+1])
                const int d = ch * 8 + 2 * w;
                *reinterpret_cast<uint32_t*>(vt + d * Cfg::VROW + pos * 2) = lo;
                *reinterpret_cast<uint32_t*>(vt + (d + 1) * Cfg::VROW + pos * 2) = hi;
            }
        }
    }
}

template <typename T, typename Cfg>
__global__ __attribute__((amdgpu_flat_work_group_size(Cfg::NT, Cfg::NT), amdgpu_waves_per_eu(2)))
void fa_fwd_mfma_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    uint16_t* __restrict__ O, float* __restrict__ LSE, int S, int BH, int n_qblk, float c) {
    constexpr int D = Cfg::D, QB = Cfg::QB, KB = Cfg::KB, KS = Cfg::KS, DB = Cfg::DB;
    constexpr int BN = Cfg::BN, BM = Cfg::BM, BMW = Cfg::BMW;
    constexpr bool CAUSAL = Cfg::CAUSAL;

    __shared__ __attribute__((aligned(16))) char smem[Cfg::LDS_BYTES];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int n = lane & 31;  // column of the MFMA output = this lane's query within a 32-block
    const int h = lane >> 5;  // wave half

    // Workgroup -> (head, query block).  Heads vary fastest so that the
    // workgroups of one head land on the same XCD (dispatch is round-robin over
    // the 8 XCDs) and share its K/V in that XCD's L2; causal query blocks are
    // issued longest first.
    const int wg = blockIdx.x;
    const int bh = wg % BH;
    const int rank = wg / BH;
    const int qblk = CAUSAL ? (n_qblk - 1 - rank) : rank;
    const int q0 = qblk * BM;
    const int qw = q0 + wave * BMW;  // first query row of this wave

    const int64_t head = (int64_t)bh * S * D;
    const uint16_t* qh = Q + head;
    const uint16_t* kh = K + head;
    const uint16_t* vh = V + head;

    // Q^T operand fragments: lane holds Q[query][16ks + 8h .. +7].
    u32x4 qf[QB][KS];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        const int qrow = qw + qb * 32 + n;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            u32x4 val = {0u, 0u, 0u, 0u};
            if (qrow < S) val = *reinterpret_cast<const u32x4*>(qh + (int64_t)qrow * D + ks * 16 + h * 8);
            qf[qb][ks] = val;
        }
    }

    float m_run[QB], l_run[QB];
    f32x16 oacc[QB][DB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        m_run[qb] = kNegInf;
        l_run[qb] = 0.f;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int r = 0; r < 16; ++r) oacc[qb][db][r] = 0.f;
    }

    // Causal: keys beyond the block's last query are never visible.
    const int kend = CAUSAL ? min(q0 + BM, S) : S;
    const int ntiles = (kend + BN - 1) / BN;

    TileStage<Cfg> st;
    stage_load<Cfg>(st, kh, vh, 0, S, tid);
    stage_store<Cfg>(st, smem, tid);
    __syncthreads();

    for (int t = 0; t < ntiles; ++t) {
        const int k0 = t * BN;
        const bool more = t + 1 < ntiles;
        if (more) stage_load<Cfg>(st, kh, vh, k0 + BN, S, tid);

        const char* kt = smem + (t & 1) * Cfg::BUF;
        const char* vt = kt + Cfg::KTILE;

        // A wave whose last query precedes the tile's first key has nothing to do here.
        const bool active = (qw < S) && (!CAUSAL || (k0 <= qw + BMW - 1));
        if (active) {
            // ---- S^T = K Q^T -------------------------------------------------
            f32x16 s[QB][KB];
#pragma unroll
            for (int qb = 0; qb < QB; ++qb)
#pragma unroll
                for (int kb = 0; kb < KB; ++kb)
#pragma unroll
                    for (int r = 0; r < 16; ++r) s[qb][kb][r] = 0.f;
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) {
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) {
                    // A operand: K[kb*32 + n][16ks + 8h .. +7]
                    const u32x4 kf = *reinterpret_cast<const u32x4*>(
                        kt + (kb * 32 + n) * Cfg::KROW + (ks * 2 + h) * 16);
#pragma unroll
                    for (int qb = 0; qb < QB; ++qb) s[qb][kb] = mfma32x32x16<T>(kf, qf[qb][ks], s[qb][kb]);
                }
            }

            // ---- mask: only tiles crossing the diagonal or the sequence end ---
            const bool needs_mask = (CAUSAL && (k0 + BN - 1 > qw)) || (k0 + BN > S);
            if (needs_mask) {
#pragma unroll
                for (int qb = 0; qb < QB; ++qb) {
                    const int qrow = qw + qb * 32 + n;
#pragma unroll
                    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
                        for (int r = 0; r < 16; ++r) {
                            const int key = k0 + kb * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
                            const bool hidden = (key >= S) || (CAUSAL && key > qrow);
                            if (hidden) s[qb][kb][r] = kNegInf;
                        }
                }
            }

            // ---- online softmax ---------------------------------------------
            u32x4 pk[QB][KB][2];
#pragma unroll
            for (int qb = 0; qb < QB; ++qb) {
                float mx = kNegInf;
#pragma unroll
                for (int kb = 0; kb < KB; ++kb)
#pragma unroll
                    for (int r = 0; r < 16; r += 2) mx = fmaxf(mx, fmaxf(s[qb][kb][r], s[qb][kb][r + 1]));
                mx = halves_max(mx);
                const float m_new = fmaxf(m_run[qb], mx * c);
                // A row with no visible key so far keeps m = -inf; subtracting 0
                // instead keeps exp2 at exactly 0 rather than NaN.
                const float m_use = (m_new == kNegInf) ? 0.f : m_new;
                const float alpha = exp2_fast(m_run[qb] - m_use);
                m_run[qb] = m_new;
                float rs0 = 0.f, rs1 = 0.f, rs2 = 0.f, rs3 = 0.f;
#pragma unroll
                for (int kb = 0; kb < KB; ++kb) {
#pragma unroll
                    for (int r = 0; r < 16; r += 4) {
                        const float p0 = exp2_fast(__builtin_fmaf(s[qb][kb][r + 0], c, -m_use));
                        const float p1 = exp2_fast(__builtin_fmaf(s[qb][kb][r + 1], c, -m_use));
                        const float p2 = exp2_fast(__builtin_fmaf(s[qb][kb][r + 2], c, -m_use));
                        const float p3 = exp2_fast(__builtin_fmaf(s[qb][kb][r + 3], c, -m_use));
                        rs0 += p0;
                        rs1 += p1;
                        rs2 += p2;
                        rs3 += p3;
                        // B operand of P*V: slot i of MFMA j holds register 8j + i
                        const int j = r >> 3, w = (r & 7) >> 1;
                        pk[qb][kb][j][w] = pack2<T>(p0, p1);
                        pk[qb][kb][j][w + 1] = pack2<T>(p2, p3);
                    }
                }
                l_run[qb] = l_run[qb] * alpha + ((rs0 + rs1) + (rs2 + rs3));
#pragma unroll
                for (int db = 0; db < DB; ++db)
#pragma unroll
                    for (int r = 0; r < 16; ++r) oacc[qb][db][r] *= alpha;
            }

            // ---- O^T += V^T P^T ---------------------------------------------
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) {
#pragma unroll
                for (int j = 0; j < 2; ++j) {
#pragma unroll
                    for (int db = 0; db < DB; ++db) {
                        // A operand: V^T[d][keys kb*32 + 16j + {4h..4h+3, 8+4h..8+4h+3}]
                        const int d = (db * 32 + n) % D;
                        const u32x4 vf = *reinterpret_cast<const u32x4*>(
                            vt + d * Cfg::VROW + (kb * 32 + 16 * j + 8 * h) * 2);
#pragma unroll
                        for (int qb = 0; qb < QB; ++qb)
                            oacc[qb][db] = mfma32x32x16<T>(vf, pk[qb][kb][j], oacc[qb][db]);
                    }
                }
            }
        }

        if (more) stage_store<Cfg>(st, smem + ((t + 1) & 1) * Cfg::BUF, tid);
        __syncthreads();
    }

    // ---- epilogue: O = acc / l, lse = ln2 * (m + log2 l) ---------------------
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
