// fa_ksplit.hpp -- the matrix-core forward kernel for grids too small to fill
// the GPU (few batch*head pairs): the waves of a workgroup share one block of
// query rows and split its key range.
//
// A query block's rows are independent of every other block's, and so are
// disjoint key ranges of one row, as long as the partial results are merged
// with the log-sum-exp rule the saved lse exists for ("T5 讲解", section ⑥;
// "Inside FlashAttention", section 2.4): over key ranges r with running
// reference m_r, sum l_r and unnormalised output acc_r,
//     M = max_r m_r,   l = sum_r 2^(m_r - M) l_r,   O = sum_r 2^(m_r - M) acc_r / l
// (m in the exp2 domain of the kernel).  Wave w of the workgroup runs the same
// Q-outer / K,V-inner online softmax as fa_mfma.hpp over the w-th contiguous
// slice of the block's key tiles, streaming its own K/V tiles HBM -> LDS into
// LDS buffers of its own, so the loop needs no barrier; at the end the waves
// exchange (m, l, acc) through LDS and wave 0 merges and writes O and lse.
// With NW waves per block, a thin grid gets NW times the waves and each row's
// serial chain of tiles is NW times shorter, at the same HBM traffic (every
// block still reads its key range once).  With two 32-row blocks per wave
// (D = 32, 64) a wave walks its slice with the half-step loop of fa_split.hpp;
// the arithmetic, and so every output bit, is that of the plain loop.
#pragma once

#include "fa_mfma.hpp"
#include "fa_split.hpp"

namespace fa {

// Lane offsets for a wave that issues every transfer of a tile itself: the
// swizzles repeat every 16 rows, i.e. every PER = RB / 64 transfers (at least 1),
// so transfer i uses offset[i % PER] + (i / PER) * PER KiB.
template <typename Cfg>
struct WaveLoader {
    static constexpr int PER = Cfg::RB >= 64 ? Cfg::RB / 64 : 1;
    static constexpr int LOADS = Cfg::TILE / 1024;  // transfers per tile
    static_assert(LOADS % PER == 0, "whole swizzle periods per tile");
    template <bool ISV>
    static __device__ __forceinline__ void offsets(int lane, uint32_t (&off)[PER]) {
#pragma unroll
        for (int i = 0; i < PER; ++i) off[i] = tile_lane_offset<Cfg, ISV>(i, lane);
    }
    template <typename T>
    static __device__ __forceinline__ void load(FA_LDS char* dst, __amdgpu_buffer_rsrc_t rsrc,
                                                const uint32_t (&off)[PER], int k0) {
#pragma unroll
        for (int i = 0; i < LOADS; ++i)
            load_part<T, Cfg>(dst + i * 1024, rsrc, off[i % PER] + (uint32_t)((i / PER) * PER * 1024), k0);
    }
};

// LDS of one workgroup: four arrays (K and V, two buffers each) that hold one
// tile per wave, declared apart so that the compiler's tracking of the
// LDS-direct transfers sees which array each one writes (a fragment read then
// waits only for transfers into its own array).  After the loop the first
// three arrays hold the accumulators of waves 1..3 (QB*DB*16 per lane) and a
// small array their m and l.
template <typename Cfg>
constexpr int ksplit_arr_bytes() {
    return Cfg::NW * Cfg::TILE > Cfg::QB * Cfg::DB * 16 * 64 * 4 ? Cfg::NW * Cfg::TILE
                                                                  : Cfg::QB * Cfg::DB * 16 * 64 * 4;
}
template <typename Cfg>
constexpr int ksplit_lds_bytes() {
    return 4 * ksplit_arr_bytes<Cfg>() + (Cfg::NW - 1) * 2 * Cfg::QB * 64 * 4;
}

template <typename T, typename Cfg>
__global__ __attribute__((amdgpu_flat_work_group_size(Cfg::NT, Cfg::NT), amdgpu_waves_per_eu(Cfg::OCC, Cfg::OCC)))
void fa_fwd_ksplit_kernel(const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
                          const uint16_t* __restrict__ V, uint16_t* __restrict__ O, float* __restrict__ LSE,
                          int Sq, int Sk, int BH, int n_qblk, int G, float c, int round) {
    using W = WaveTile<T, Cfg>;
    using L = WaveLoader<Cfg>;
    constexpr int D = Cfg::D, QB = Cfg::QB, KB = Cfg::KB, KS = Cfg::KS, DB = Cfg::DB;
    constexpr int NW = Cfg::NW, BN = Cfg::BN, BMW = Cfg::BMW, RB = Cfg::RB, TILE = Cfg::TILE;
    constexpr bool CAUSAL = Cfg::CAUSAL;
    static_assert(Cfg::PIPE && Cfg::TBN == BN, "pipelined loop, one compute tile per LDS tile");

    static_assert(NW == 4, "the exchange uses three of the four arrays");
    constexpr int ARR = ksplit_arr_bytes<Cfg>();
    __shared__ __attribute__((aligned(1024))) char lk0[ARR];
    __shared__ __attribute__((aligned(1024))) char lk1[ARR];
    __shared__ __attribute__((aligned(1024))) char lv0[ARR];
    __shared__ __attribute__((aligned(1024))) char lv1[ARR];
    __shared__ __attribute__((aligned(16))) float xml[(NW - 1) * 2 * QB * 64];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int n = lane & 31;
    const int h = lane >> 5;
    FA_LDS char* const kbuf[2] = {(FA_LDS char*)lk0 + wave * TILE, (FA_LDS char*)lk1 + wave * TILE};
    FA_LDS char* const vbuf[2] = {(FA_LDS char*)lv0 + wave * TILE, (FA_LDS char*)lv1 + wave * TILE};

    // Workgroup -> (head, query block): heads vary fastest, causal blocks
    // longest first.  Every wave holds the block's BMW rows.
    const int lin = CAUSAL ? causal_work_index(round, BH) : (int)blockIdx.x;
    const int bh = lin % BH;
    const int rank = lin / BH;
    const int qblk = CAUSAL ? (n_qblk - 1 - rank) : rank;
    const int q0 = qblk * BMW;

    const int64_t head = (int64_t)bh * Sq * D;
    const int64_t kvhead = (int64_t)(bh / G) * Sk * D;  // grouped heads: G query heads per K/V head
    const uint16_t* qh = Q + head;
    const __amdgpu_buffer_rsrc_t krs = head_rsrc<T>(K + kvhead, Sk * RB);
    const __amdgpu_buffer_rsrc_t vrs = head_rsrc<T>(V + kvhead, Sk * RB);
    uint32_t koff[L::PER], voff[L::PER];
    L::template offsets<false>(lane, koff);
    L::template offsets<true>(lane, voff);

    // This wave's slice [tb, te) of the block's key tiles.
    const int kend = CAUSAL ? min(q0 + BMW, Sk) : Sk;
    const int ntiles = (kend + BN - 1) / BN;
    const int tb = wave * ntiles / NW;
    const int te = (wave + 1) * ntiles / NW;
    const int nt = te - tb;

    u32x4 qf[QB][KS];
    int last[QB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        const int qrow = min(q0 + qb * 32 + n, Sq - 1);
        last[qb] = CAUSAL ? min(qrow, Sk - 1) : Sk - 1;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
            qf[qb][ks] = *reinterpret_cast<const u32x4*>(qh + (int64_t)qrow * D + ks * 16 + h * 8);
    }
    // (pinned once every load is in flight, so that their round trips overlap)
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) pin(qf[qb][ks]);

    int offk[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) offk[ks] = n * RB + (((2 * ks + h) ^ swz_k<D>(n)) * 16);
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

    constexpr bool kHalf = QB == 2 && KB == 1 && KS >= 2;
    if constexpr (kHalf) {
        // Two 32-row blocks per wave (D = 32, 64): the half-step loop of
        // fa_split.hpp (softmax of one block beside the other block's MFMAs)
        // over this wave's slice.  Relative tile u = t - tb: LDS tile u, in
        // buffers u & 1, holds K(t+1) and V(t); K(tb) waits in the second K
        // buffer, which LDS tile 1 refills after K(tb)'s fragments were
        // consumed.  The wave is the only reader of its buffers, so a refill
        // needs no barrier: the fragments of the tile it replaces fed MFMAs
        // issued before it.
        using ST = SplitTile<T, Cfg>;
        // per block a: na = its tiles in the slice, ua = the slice's leading
        // tiles that need no mask for any of its rows (may be <= 0)
        int na[2], ua[2];
#pragma unroll
        for (int a = 0; a < 2; ++a) {
            const int r0 = q0 + 32 * a;
            const int rend = CAUSAL ? min(r0 + 32, Sk) : Sk;
            const int wt = r0 < Sq ? min(ntiles, (rend + BN - 1) / BN) : 0;
            na[a] = max(0, min(te, wt) - tb);
            ua[a] = min(CAUSAL ? (r0 + 1) / BN : ntiles, Sk / BN) - tb;
        }
        const int nw = max(na[0], na[1]);  // = na[1] unless block 1 has no rows
        if (nw > 0) {
            f32x16 s[2];
            u32x4 p[2][2];
            u32x4 kfr[KS], vfr[2][DB];
            L::template load<T>(kbuf[1], krs, koff, tb * BN);
            if (nw > 1) L::template load<T>(kbuf[0], krs, koff, (tb + 1) * BN);
            L::template load<T>(vbuf[0], vrs, voff, tb * BN);
            wait_vmcnt0();
            ST::read_k(kbuf[1], offk, kfr);
            if (na[0] > 0) ST::qk(kfr, qf[0], s[0]);

            // generic half-step (first tile, masked tiles, a block's last tiles)
            auto half_any = [&](auto blk, int u) __attribute__((always_inline)) {
                constexpr int A = decltype(blk)::value, B = 1 - A;
                const int upv = A == 0 ? u - 1 : u;  // block B's P*V tile
                const int uqk = A == 0 ? u : u + 1;  // block B's S tile
                if (upv >= 0 && upv < na[B]) ST::pv(vfr, p[B], oacc[B]);
                if (uqk < na[B]) ST::qk(kfr, qf[B], s[B]);
                if (u < na[A]) {
                    if (u >= ua[A]) ST::mask(s[A], last[A], (tb + u) * BN, h);
                    if (u == 0) {
                        m_run[A] = fmaxf(m_run[A], ST::rmax(s[A]) * c);
                        ST::expo(s[A], m_run[A], c, p[A], l_run[A]);
                    } else {
                        float rs;
                        ST::expo(s[A], m_run[A], c, p[A], rs);
                        if (ST::needs_rescale(rs)) ST::rescale(s[A], m_run[A], l_run[A], oacc[A], c, p[A], rs);
                        l_run[A] += rs;
                    }
                }
            };
            auto steady_half = [&](auto blk) __attribute__((always_inline)) {
                constexpr int A = decltype(blk)::value, B = 1 - A;
                float rs;
                ST::half(kfr, vfr, qf[B], s[A], s[B], p[A], p[B], oacc[B], m_run[A], c, rs);
                if (ST::needs_rescale(rs)) ST::rescale(s[A], m_run[A], l_run[A], oacc[A], c, p[A], rs);
                l_run[A] += rs;
            };
            // between the half-steps of tile u: wait for LDS tile u, read the
            // fragments of K(t+1) and V(t), then start LDS tile u+1 into the
            // other buffers (fenced, as in fa_split.hpp, so that no fragment
            // read moves across the transfers or into another half-step)
            auto sync_with = [&](int u, FA_LDS char* kc, FA_LDS char* vc, FA_LDS char* kn, FA_LDS char* vn)
                                 __attribute__((always_inline)) {
                wait_vmcnt0();
                __builtin_amdgcn_sched_barrier(0);
                ST::read_k(kc, offk, kfr);
                ST::read_v(vc, offv, vfr);
                __builtin_amdgcn_sched_barrier(0);
                if (u + 1 < nw) {
                    if (u + 2 < nw) L::template load<T>(kn, krs, koff, (tb + u + 2) * BN);
                    L::template load<T>(vn, vrs, voff, (tb + u + 1) * BN);
                }
            };
            auto sync = [&](auto par, int u) __attribute__((always_inline)) {
                constexpr int P = decltype(par)::value;
                sync_with(u, kbuf[P], vbuf[P], kbuf[1 - P], vbuf[1 - P]);
            };
            auto sync_rt = [&](int u) __attribute__((always_inline)) {
                const bool odd = u & 1;
                sync_with(u, odd ? kbuf[1] : kbuf[0], odd ? vbuf[1] : vbuf[0], odd ? kbuf[0] : kbuf[1],
                          odd ? vbuf[0] : vbuf[1]);
            };
            using A0 = std::integral_constant<int, 0>;
            using A1 = std::integral_constant<int, 1>;
            // steady for 1 <= u < us: both blocks unmasked, every MFMA present
            const int us = min(min(ua[0], ua[1]), min(na[1], na[0] - 1));
            half_any(A0{}, 0);
            sync_rt(0);
            half_any(A1{}, 0);
            int u = 1;
            for (; u + 1 < us; u += 2) {
                steady_half(A0{});
                sync(A1{}, u);
                steady_half(A1{});
                steady_half(A0{});
                sync(A0{}, u + 1);
                steady_half(A1{});
            }
            if (u < us) {
                steady_half(A0{});
                sync(A1{}, u);
                steady_half(A1{});
                ++u;
            }
            for (; u < nw; ++u) {
                half_any(A0{}, u);
                sync_rt(u);
                half_any(A1{}, u);
            }
            // P*V of block 1's last tile (its V is still in vfr)
            if (na[1] == nw) ST::pv(vfr, p[1], oacc[1]);
        }
    } else if (nt > 0) {
        // Relative tile u = t - tb lives in buffers u & 1.  Iteration u: S(u) in
        // s_cur, S(u+1) to s_nxt, P(u-1) in p_prv, P(u) to p_cur; K(u+2) and V(u)
        // start into the buffers K(u) and V(u-2) left (their reads ended in
        // iteration u-1: this wave is their only reader, so no barrier).
        f32x16 sA[QB][KB], sB[QB][KB];
        u32x4 pA[QB][KB][2], pB[QB][KB][2];
        L::template load<T>(kbuf[0], krs, koff, tb * BN);
        if (nt > 1) L::template load<T>(kbuf[1], krs, koff, (tb + 1) * BN);
        wait_vmcnt0();
        W::qk(kbuf[0], offk, qf, sA);

        // rows whose tiles need no mask: tiles before the block's first row
        // and before the end of the sequence
        const int unmasked = min(CAUSAL ? (q0 + 1) / BN : ntiles, Sk / BN);
        auto iter = [&](auto kind, int u, FA_LDS char* kc, FA_LDS char* kn, FA_LDS char* vc, FA_LDS char* vp,
                        f32x16 (&s_cur)[QB][KB], f32x16 (&s_nxt)[QB][KB], u32x4 (&p_prv)[QB][KB][2],
                        u32x4 (&p_cur)[QB][KB][2]) __attribute__((always_inline)) {
            constexpr int KIND = decltype(kind)::value;  // 0 first, 1 steady, 2 edge
            const int t = tb + u;
            const int k0 = t * BN;
            wait_vmcnt0();  // K(u+1) and V(u-1) landed
            if (KIND == 1 || u + 2 < nt) L::template load<T>(kc, krs, koff, k0 + 2 * BN);
            L::template load<T>(vc, vrs, voff, k0);
            if constexpr (KIND == 0) {
                if (u + 1 < nt) W::qk(kn, offk, qf, s_nxt);
                if ((CAUSAL && k0 + BN - 1 > q0) || k0 + BN > Sk) W::mask(s_cur, last, k0, h);
                W::first(s_cur, m_run, l_run, c, p_cur);
                return;
            }
            float rs[QB];
            if constexpr (KIND == 1) {
                W::step(kn, vp, offk, offv, qf, s_cur, s_nxt, p_prv, p_cur, oacc, m_run, c, rs);
            } else {
                if (u + 1 < nt) W::qk(kn, offk, qf, s_nxt);
                W::pv(vp, offv, p_prv, oacc);
                if ((CAUSAL && k0 + BN - 1 > q0) || k0 + BN > Sk) W::mask(s_cur, last, k0, h);
                W::expo(s_cur, m_run, c, p_cur, rs);
            }
            if (W::needs_rescale(rs)) W::rescale(s_cur, m_run, l_run, oacc, c, p_cur, rs);
#pragma unroll
            for (int qb = 0; qb < QB; ++qb) l_run[qb] += rs[qb];
        };
        using First = std::integral_constant<int, 0>;
        using Steady = std::integral_constant<int, 1>;
        using Edge = std::integral_constant<int, 2>;
        // steady for 1 <= u < u_steady: a next tile exists and this tile needs no mask
        const int u_steady = min(nt - 1, unmasked - tb);
        iter(First{}, 0, kbuf[0], kbuf[1], vbuf[0], vbuf[1], sA, sB, pA, pB);
        int u = 1;
        for (; u + 1 < u_steady; u += 2) {
            iter(Steady{}, u, kbuf[1], kbuf[0], vbuf[1], vbuf[0], sB, sA, pB, pA);
            iter(Steady{}, u + 1, kbuf[0], kbuf[1], vbuf[0], vbuf[1], sA, sB, pA, pB);
        }
        for (; u < nt; u += 2) {
            iter(Edge{}, u, kbuf[1], kbuf[0], vbuf[1], vbuf[0], sB, sA, pB, pA);
            if (u + 1 < nt) iter(Edge{}, u + 1, kbuf[0], kbuf[1], vbuf[0], vbuf[1], sA, sB, pA, pB);
        }
        // P*V of the last tile, whose V is in buffer (nt-1) & 1
        wait_vmcnt0();
        if ((nt - 1) & 1) W::pv(vbuf[1], offv, pA, oacc);
        else W::pv(vbuf[0], offv, pB, oacc);
    }

    // ---- merge the waves' partial results, then the epilogue ------------------------
    __syncthreads();  // every wave is done with its K/V buffers
    // wave w's accumulators in array w - 1, its m and l in xml
    auto acc_slot = [&](int w, int k) __attribute__((always_inline)) -> float& {
        float* const a = (float*)(w == 1 ? lk0 : w == 2 ? lk1 : lv0);
        return a[k * 64 + lane];
    };
    auto ml_slot = [&](int w, int k) __attribute__((always_inline)) -> float& {
        return xml[((w - 1) * 2 * QB + k) * 64 + lane];
    };
    if (wave > 0) {
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
#pragma unroll
            for (int db = 0; db < DB; ++db)
#pragma unroll
                for (int r = 0; r < 16; ++r) acc_slot(wave, (qb * DB + db) * 16 + r) = oacc[qb][db][r];
            ml_slot(wave, qb) = m_run[qb];
            ml_slot(wave, QB + qb) = l_run[qb];
        }
    }
    __syncthreads();
    if (wave != 0) return;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        float mw[NW];
        mw[0] = m_run[qb];
        float mx = mw[0];
#pragma unroll
        for (int w = 1; w < NW; ++w) {
            mw[w] = ml_slot(w, qb);
            mx = fmaxf(mx, mw[w]);
        }
        const float a0 = exp2_fast(mw[0] - mx);
        float l = l_run[qb] * a0;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int r = 0; r < 16; ++r) oacc[qb][db][r] *= a0;
#pragma unroll
        for (int w = 1; w < NW; ++w) {
            const float aw = exp2_fast(mw[w] - mx);
            l += aw * ml_slot(w, QB + qb);
#pragma unroll
            for (int db = 0; db < DB; ++db)
#pragma unroll
                for (int r = 0; r < 16; ++r) oacc[qb][db][r] += aw * acc_slot(w, (qb * DB + db) * 16 + r);
        }
        m_run[qb] = mx;
        l_run[qb] = l;
    }

    uint16_t* oh = O + head;
    float* lh = LSE + (int64_t)bh * Sq;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        const float l = halves_sum(l_run[qb]);
        const float inv = 1.0f / l;
        const int qrow = q0 + qb * 32 + n;
        if (qrow < Sq) {
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
