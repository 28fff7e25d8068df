// fa_split.hpp -- the matrix-core forward kernel for waves that own two 32-query
// column blocks (64 query rows) and walk the keys in tiles of 32.
//
// Same method as fa_mfma.hpp (query blocks outer, key/value tiles inner, online
// softmax with a running reference m and sum l, one normalisation at the end:
// "Triton 实现", sections "Q-outer 主循环" and "内层循环"; "T5 讲解", sections
// ②-⑥), with a different software pipeline.  The two column blocks a = 0, 1 of a
// wave are offset by half a tile: every half-step runs the softmax of one block
// while the matrix cores compute, for the other block, O^T += V^T P^T of the tile
// it finished and S^T = K Q^T of the tile it starts:
//
//   H(t,0):  softmax(t, 0)   |  P*V(t-1, 1),  S(t, 1)
//   H(t,1):  softmax(t, 1)   |  P*V(t, 0),    S(t+1, 0)
//
// Each block's scores and probabilities live in one register set that is
// consumed and refilled on alternate half-steps, so a wave holds one score tile
// and one P tile per block instead of two of each.  The K and V operand
// fragments read from LDS at the start of H(t,1) (K of tile t+1, V of tile t)
// serve that half-step and the next, so every fragment still feeds two MFMAs.
// K and V tiles stream HBM -> LDS with one barrier per tile, two buffers each.
// A block's rescale (threshold rule of fa_mfma.hpp) touches only its own
// accumulator, which the other block's MFMAs of the same half-step never write.
#pragma once

#include "fa_mfma.hpp"

namespace fa {

template <typename T, typename Cfg>
struct SplitTile {
    static_assert(Cfg::QB == 2 && Cfg::KB == 1 && Cfg::PIPE, "two column blocks, 32-key tiles");
    using W = WaveTile<T, Cfg>;
    using Pair = typename W::Pair;
    static constexpr int KS = Cfg::KS, DB = Cfg::DB;
    static constexpr int NPV = 2 * DB;  // O^T MFMAs of one block per tile
    static constexpr int NQK = KS;      // S^T MFMAs of one block per tile
    static constexpr int NM = NPV + NQK;

    // Pair i of a block's scores: registers 2i, 2i+1, packed into slot i % 4 of
    // P operand i / 4 (operand j holds keys 16j + {4h..4h+3, 8+4h..8+4h+3}).
    static __device__ __forceinline__ Pair pexp(const f32x16& s, float m, float c, int i) {
        return {exp2_fast(__builtin_fmaf(s[2 * i], c, -m)), exp2_fast(__builtin_fmaf(s[2 * i + 1], c, -m))};
    }
    static __device__ __forceinline__ void ppack(Pair x, int i, u32x4 (&p)[2], float& rs) {
        p[i >> 2][i & 3] = pack2<T>(x.p0, x.p1);
        rs = pair_sum(rs, x.p0, x.p1, i == 0);
    }
    static __device__ __forceinline__ void expo(const f32x16& s, float m, float c, u32x4 (&p)[2], float& rs) {
#pragma unroll
        for (int i = 0; i < 8; ++i) ppack(pexp(s, m, c, i), i, p, rs);
        pin(p[0]);
        pin(p[1]);
    }

    static __device__ __forceinline__ float rmax(const f32x16& s) {
        float a = fmaxf(s[0], s[1]), b = fmaxf(s[2], s[3]);
#pragma unroll
        for (int r = 4; r < 16; r += 4) {
            a = fmaxf(fmaxf(a, s[r]), s[r + 1]);
            b = fmaxf(fmaxf(b, s[r + 2]), s[r + 3]);
        }
        return halves_max(fmaxf(a, b));
    }

    // key of register r is k0 + 4h + 8(r/4) + r%4; visible iff key <= last
    static __device__ __forceinline__ void mask(f32x16& s, int last, int k0, int h) {
        const int lim = last - (k0 + 4 * h);
#pragma unroll
        for (int r = 0; r < 16; ++r)
            if (8 * (r >> 2) + (r & 3) > lim) s[r] = kNegInf;
    }

    static __device__ __forceinline__ void read_k(const FA_LDS char* kt, const int (&offk)[KS], u32x4 (&kfr)[KS]) {
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) kfr[ks] = *reinterpret_cast<const FA_LDS u32x4*>(kt + offk[ks]);
    }
    static __device__ __forceinline__ void read_v(const FA_LDS char* vt, const int (&offv)[DB], u32x4 (&vfr)[2][DB]) {
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int db = 0; db < DB; ++db) vfr[j][db] = W::v_frag(vt, offv, 0, j, db);
    }

    static __device__ __forceinline__ void qk(const u32x4 (&kfr)[KS], const u32x4 (&qfb)[KS], f32x16& s) {
        const f32x16 zero = {};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) s = mfma32x32x16<T>(kfr[ks], qfb[ks], ks == 0 ? zero : s);
    }
    static __device__ __forceinline__ void pv(const u32x4 (&vfr)[2][DB], const u32x4 (&p)[2], f32x16 (&o)[DB]) {
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int db = 0; db < DB; ++db) o[db] = mfma32x32x16<T>(vfr[j][db], p[j], o[db]);
    }

    // Steady half-step: softmax of block a (sa -> pa, partial sums rsa) with the
    // other block's P*V (pb, ob) and S^T (sb) on the matrix cores, in issue
    // order: the P*V MFMAs, then the S^T ones, each followed by its share of the
    // softmax.  A wave issues its own independent vector instructions while its
    // MFMA runs (one 32x32x16 MFMA hides two exponentials or four FMAs), so the
    // order is pinned with scheduling groups at D = 64: eight vector
    // instructions first (they wait for no LDS read), then every MFMA followed
    // by six of them; measured 3 % faster on B=4 H=16 S=4096 than the
    // compiler's own order, which bunches the MFMAs at the end of the
    // half-step.  The packed P is materialised before the rescale check, so
    // that its conversions count among those groups.
    static __device__ __forceinline__ void half(const u32x4 (&kfr)[KS], const u32x4 (&vfr)[2][DB],
                                                const u32x4 (&qfb)[KS], const f32x16& sa, f32x16& sb,
                                                u32x4 (&pa)[2], const u32x4 (&pb)[2], f32x16 (&ob)[DB], float ma,
                                                float c, float& rsa) {
        constexpr int NP = 8, LEAD = 1;
        const f32x16 zero = {};
        Pair x[NP];
        int nf = 0, nc = 0, ipv = 0, iqk = 0;
#pragma unroll
        for (; nf < LEAD; ++nf) x[nf] = pexp(sa, ma, c, nf);
#pragma unroll
        for (int i = 0; i < NM; ++i) {
            if (ipv < NPV) {
                const int j = ipv / DB, db = ipv % DB;
                ob[db] = mfma32x32x16<T>(vfr[j][db], pb[j], ob[db]);
                ++ipv;
            } else {
                sb = mfma32x32x16<T>(kfr[iqk], qfb[iqk], iqk == 0 ? zero : sb);
                ++iqk;
            }
            const int nf0 = nf;
            const int f_end = i == NM - 1 ? NP : LEAD + ((i + 1) * (NP - LEAD) + NM / 2) / NM;
            const int c_end = i == NM - 1 ? NP : min(((i + 1) * NP + NM / 2) / NM, nf0);
#pragma unroll
            for (; nf < f_end; ++nf) x[nf] = pexp(sa, ma, c, nf);
#pragma unroll
            for (; nc < c_end; ++nc) ppack(x[nc], nc, pa, rsa);
        }
        if constexpr (KS == 4) {  // D = 64, where the pattern was measured
            pin(pa[0]);
            pin(pa[1]);
            __builtin_amdgcn_sched_group_barrier(kSchedValu, 8, 0);
#pragma unroll
            for (int i = 0; i < NM; ++i) {
                __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
                __builtin_amdgcn_sched_group_barrier(kSchedValu, 6, 0);
            }
        }
    }

    // The exact path for block a: m to max(m, c * rowmax), l and acc rescaled by
    // alpha = exp2(m_old - m_new), the tile exponentiated again.
    static __device__ __forceinline__ void rescale(const f32x16& s, float& m, float& l, f32x16 (&o)[DB], float c,
                                                   u32x4 (&p)[2], float& rs) {
        const float m_new = fmaxf(m, rmax(s) * c);
        const float alpha = exp2_fast(m - m_new);
        m = m_new;
        l *= alpha;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int r = 0; r < 16; ++r) o[db][r] *= alpha;
        expo(s, m, c, p, rs);
    }

    static __device__ __forceinline__ bool needs_rescale(float rs) {
        return __builtin_amdgcn_ballot_w64(!(rs <= kSumLimit)) != 0;
    }
};

// SINGLE = true is the race check of the double-buffered staging: one K and one
// V buffer, the next tile's transfers issued only after a barrier that follows
// every wave's last fragment read of the current one.  The arithmetic and its
// order are the same, so its O and lse must equal the double-buffered kernel's
// bit for bit; a difference would expose a read of a buffer still being
// refilled.
template <typename T, typename Cfg, bool SINGLE = false, bool KSPLIT = false>
__global__ __attribute__((amdgpu_flat_work_group_size(Cfg::NT, Cfg::NT), amdgpu_waves_per_eu(Cfg::OCC, Cfg::OCC)))
void fa_fwd_split_kernel(const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
                         const uint16_t* __restrict__ V, uint16_t* __restrict__ O, float* __restrict__ LSE, int Sq, int Sk,
                         int BH, int n_qblk, int G, float c, int round, float* __restrict__ PO,
                         float* __restrict__ PL, int nsplit) {
    using ST = SplitTile<T, Cfg>;
    constexpr int D = Cfg::D, KS = Cfg::KS, DB = Cfg::DB;
    constexpr int BN = Cfg::BN, BM = Cfg::BM, BMW = Cfg::BMW, RB = Cfg::RB;
    constexpr int SUB = Cfg::TBN / BN;  // compute tiles per LDS tile
    constexpr bool CAUSAL = Cfg::CAUSAL;

    // K and V stream through LDS in tiles of TBN = SUB * BN keys, two buffers
    // each (declared apart so the compiler's tracking of the LDS-direct
    // transfers sees which buffer each one writes).  V tile j holds keys
    // j*TBN .. +TBN-1; K tile j is staged one compute tile ahead, keys
    // j*TBN + BN .. +TBN-1 + BN, because the sync of compute tile t reads K(t+1)
    // and V(t): tile t = j*SUB + u finds both in slot u of LDS tile j, so one
    // barrier (at u = 0) covers SUB compute tiles.  K(0) sits in the last slot of
    // the other K buffer ("K tile -1").
    __shared__ __attribute__((aligned(1024))) char k_lds0[Cfg::TILE];
    __shared__ __attribute__((aligned(1024))) char k_lds1[Cfg::TILE];
    __shared__ __attribute__((aligned(1024))) char v_lds0[Cfg::TILE];
    __shared__ __attribute__((aligned(1024))) char v_lds1[Cfg::TILE];
    FA_LDS char* const kbuf[2] = {(FA_LDS char*)k_lds0, SINGLE ? (FA_LDS char*)k_lds0 : (FA_LDS char*)k_lds1};
    FA_LDS char* const vbuf[2] = {(FA_LDS char*)v_lds0, SINGLE ? (FA_LDS char*)v_lds0 : (FA_LDS char*)v_lds1};
    // K(0): the last slot of the second K array in either mode
    FA_LDS char* const k0slot = (FA_LDS char*)k_lds1 + (SUB - 1) * BN * RB;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int n = lane & 31;
    const int h = lane >> 5;

    // Workgroup -> (head, query block): heads vary fastest (one head's blocks
    // share an XCD's L2), causal blocks longest first.  With KSPLIT (causal, a
    // workspace PO / PL): the nsplit longest blocks of every head are split
    // at a key-tile boundary into two halves, each a workgroup of its own, and
    // every head's items run longest first (split_work_item); a half
    // writes its fp32 partial result (O normalised by its own l, and its lse)
    // to the workspace, and fa_fwd_merge_kernel combines the two by the
    // log-sum-exp rule ("T5 讲解", section ⑥; "Inside FlashAttention",
    // section 2.4).  This shortens the longest serial chains of tiles when the
    // whole grid is resident at once.
    int bh, qblk;
    int part = -1;  // -1: the whole block; 0, 1: its first or second key half
    if constexpr (KSPLIT) {
        static_assert(CAUSAL && !SINGLE, "the key split serves causal problems");
        bh = blockIdx.x % BH;
        split_work_item(blockIdx.x / BH, n_qblk, nsplit, qblk, part);
    } else {
        const int wg = CAUSAL ? causal_work_index(round, BH) : (int)blockIdx.x;
        bh = wg % BH;
        const int rank = wg / BH;
        qblk = CAUSAL ? (n_qblk - 1 - rank) : rank;
    }
    const int q0 = qblk * BM;
    const int qw = q0 + wave * BMW;

    // The block's key tiles and this workgroup's range [tb, te) of them (all,
    // for a whole block; halves split at a multiple of the LDS tile).  The K/V
    // resources start at key kb = tb * BN, so tile indices and the key limits
    // below are relative to it, and a whole block (kb = 0) runs unchanged.
    const int ntiles_blk = ((CAUSAL ? min(q0 + BM, Sk) : Sk) + BN - 1) / BN;
    const int tsplit = (ntiles_blk / 2) / SUB * SUB;
    const int tb = part == 1 ? tsplit : 0;
    const int te = part == 0 ? tsplit : ntiles_blk;
    const int kb = tb * BN;

    const int64_t head = (int64_t)bh * Sq * D;
    const int64_t kvhead = (int64_t)(bh / G) * Sk * D + (int64_t)kb * D;  // grouped heads: G query heads per K/V head
    const uint16_t* qh = Q + head;
    const __amdgpu_buffer_rsrc_t krs = head_rsrc<T>(K + kvhead, (Sk - kb) * RB);
    const __amdgpu_buffer_rsrc_t vrs = head_rsrc<T>(V + kvhead, (Sk - kb) * RB);
    const uint32_t koff = tile_lane_offset<Cfg, false>(wave, lane);
    const uint32_t voff = tile_lane_offset<Cfg, true>(wave, lane);

    const int ntiles = te - tb;
    const int nlds = (ntiles + SUB - 1) / SUB;

    // Per column block a (rows qw + 32a ..): wt = tiles of the range it attends
    // to, um = leading tiles that need no mask for any of its rows, last = the
    // last key each row sees (relative to kb).
    int wt[2], um[2], last[2];
#pragma unroll
    for (int a = 0; a < 2; ++a) {
        const int r0 = qw + 32 * a;
        const int rend = CAUSAL ? min(r0 + 32, Sk) : Sk;
        const int wt_blk = r0 < Sq ? min(ntiles_blk, (rend + BN - 1) / BN) : 0;
        wt[a] = max(0, min(te, wt_blk) - tb);
        um[a] = min(CAUSAL ? (r0 + 1) / BN : ntiles_blk, Sk / BN) - tb;
        last[a] = (CAUSAL ? min(r0 + n, Sk - 1) : Sk - 1) - kb;
    }

    // Prologue transfers: K(0) (this wave's share of its BN rows), K tile 0, V tile 0.
    {
        constexpr int K0_LOADS = BN * RB / 1024;  // 1 KiB transfers of K(0)
        static_assert(K0_LOADS <= Cfg::NW, "K(0) in one transfer per wave");
        if (wave < K0_LOADS)
            load_part<T, Cfg>(k0slot + wave * 1024, krs, koff, 0);
    }
    load_tile<T, Cfg, false>(kbuf[0], krs, koff, BN, wave, lane);
    load_tile<T, Cfg, true>(vbuf[0], vrs, voff, 0, wave, lane);

    // Q^T operand fragments, resident for the whole loop ("T5 讲解", section ③).
    // Every load is issued before the first pin: a pin right after its load
    // makes the wave wait out each load's round trip in turn.
    u32x4 qf[2][KS];
#pragma unroll
    for (int a = 0; a < 2; ++a) {
        const int qrow = min(qw + 32 * a + n, Sq - 1);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
            qf[a][ks] = *reinterpret_cast<const u32x4*>(qh + (int64_t)qrow * D + ks * 16 + h * 8);
    }
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) pin(qf[a][ks]);

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

    float m_run[2] = {kMInit, kMInit}, l_run[2] = {0.f, 0.f};
    f32x16 oacc[2][DB];
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int r = 0; r < 16; ++r) oacc[a][db][r] = 0.f;
    f32x16 s[2];
    u32x4 p[2][2];
    u32x4 kfr[KS], vfr[2][DB];

    wait_vmcnt0();
    __syncthreads();
    ST::read_k(k0slot, offk, kfr);
    if (wt[0] > 0) ST::qk(kfr, qf[0], s[0]);

    // Generic half-step (first tile, masked tiles, a block's last tiles): the
    // same work as ST::half under wave-uniform conditions, compiler-scheduled.
    auto half_any = [&](auto blk, int t) __attribute__((always_inline)) {
        constexpr int A = decltype(blk)::value, B = 1 - A;
        const int tb = A == 0 ? t - 1 : t;  // the P*V tile of block B
        const int tq = A == 0 ? t : t + 1;  // the S tile of block B
        if (tb >= 0 && tb < wt[B]) ST::pv(vfr, p[B], oacc[B]);
        if (tq < wt[B]) ST::qk(kfr, qf[B], s[B]);
        if (t < wt[A]) {
            if (t >= um[A]) ST::mask(s[A], last[A], t * BN, h);
            if (t == 0) {
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
    using A0 = std::integral_constant<int, 0>;
    using A1 = std::integral_constant<int, 1>;

    // Between the half-steps of compute tile t = j*SUB + u (LDS tile j, in
    // buffers of parity j % 2): at u = 0 wait for LDS tile j and barrier; read the
    // fragments of K(t+1) and V(t) from slot u; at u = 0 then start LDS tile j+1
    // into the other buffers (their last fragments were read before the
    // barrier).  The fragment reads come before the new transfers, so that the
    // compiler, which tracks the transfers' LDS targets, never makes them wait
    // for a transfer in flight; `kc`, `vc` are the buffers of parity j % 2.  The
    // slot u is a compile-time constant (its offset folds into the reads'
    // immediate offsets: no per-lane address arithmetic).
    auto sync_with = [&](int j, auto ucst, FA_LDS char* kc, FA_LDS char* vc, FA_LDS char* kn, FA_LDS char* vn)
                         __attribute__((always_inline)) {
        constexpr int U = decltype(ucst)::value;
        if constexpr (U == 0) {
            wait_vmcnt0();
            __syncthreads();
        }
        // (fenced, so that the scheduler cannot hoist later tiles' fragment
        // reads into earlier half-steps and run out of registers)
        __builtin_amdgcn_sched_barrier(0);
        ST::read_k(kc + U * BN * RB, offk, kfr);
        ST::read_v(vc + U * BN * RB, offv, vfr);
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (SINGLE) {
            // one buffer: refill it only once every wave has read its last slot
            if constexpr (U == SUB - 1) {
                __syncthreads();
                if (j + 1 < nlds) {
                    load_tile<T, Cfg, false>(kn, krs, koff, (j + 1) * Cfg::TBN + BN, wave, lane);
                    load_tile<T, Cfg, true>(vn, vrs, voff, (j + 1) * Cfg::TBN, wave, lane);
                }
            }
        } else if constexpr (U == 0) {
            if (j + 1 < nlds) {
                load_tile<T, Cfg, false>(kn, krs, koff, (j + 1) * Cfg::TBN + BN, wave, lane);
                load_tile<T, Cfg, true>(vn, vrs, voff, (j + 1) * Cfg::TBN, wave, lane);
            }
        }
    };
    // buffers known at compile time (steady tiles) ...
    auto sync = [&](auto par, int j, auto ucst) __attribute__((always_inline)) {
        constexpr int P = decltype(par)::value;
        sync_with(j, ucst, kbuf[P], vbuf[P], kbuf[1 - P], vbuf[1 - P]);
    };
    // ... or chosen at run time (generic tiles: fewer code copies)
    auto sync_rt = [&](int j, auto ucst) __attribute__((always_inline)) {
        const bool odd = j & 1;
        sync_with(j, ucst, odd ? kbuf[1] : kbuf[0], odd ? vbuf[1] : vbuf[0], odd ? kbuf[0] : kbuf[1],
                  odd ? vbuf[0] : vbuf[1]);
    };
    // steady for 1 <= t < t_steady: both blocks unmasked, every MFMA present
    const int t_steady = min(min(um[0], um[1]), min(wt[1], wt[0] - 1));
    // The SUB compute tiles of LDS tile j (buffers of parity P), all steady ...
    auto lds_steady = [&](auto par, int j) __attribute__((always_inline)) {
        static_for<SUB>([&](auto ucst) __attribute__((always_inline)) {
            steady_half(A0{});
            sync(par, j, ucst);
            steady_half(A1{});
        });
    };
    // ... or under the generic conditions.
    auto lds_generic = [&](int j) __attribute__((always_inline)) {
        static_for<SUB>([&](auto ucst) __attribute__((always_inline)) {
            constexpr int U = decltype(ucst)::value;
            const int t = j * SUB + U;
            if (t < ntiles) {
                half_any(A0{}, t);
                sync_rt(j, ucst);
                half_any(A1{}, t);
            }
        });
    };
    using P0 = std::integral_constant<int, 0>;
    using P1 = std::integral_constant<int, 1>;
    // LDS tile 0 (it holds the first compute tile), then LDS tiles 1 .. js-1,
    // which hold steady compute tiles only, then the rest; separate loops keep
    // the steady code free of the generic path's registers.
    const int js = t_steady / SUB;
    if (nlds > 0) lds_generic(0);
    int j = 1;
    for (; j + 1 < js; j += 2) {
        lds_steady(P1{}, j);
        lds_steady(P0{}, j + 1);
    }
    if (j < js) lds_steady(P1{}, j++);
    for (; j < nlds; ++j) lds_generic(j);
    // P*V of block 1's last tile (V of tile ntiles-1 is still in vfr)
    if (wt[1] == ntiles && ntiles > 0) ST::pv(vfr, p[1], oacc[1]);

    // ---- epilogue: O = acc / l, lse = ln2 * (m + log2 l) ---------------------------
    if (KSPLIT && part >= 0) {
        // a key half: its fp32 partial, item (2j + part) * BH + bh of BM rows
        // (j: the block's rank among the split ones), rows in block order
        const int64_t item = ((int64_t)(2 * (n_qblk - 1 - qblk) + part) * BH + bh) * BM;
#pragma unroll
        for (int a = 0; a < 2; ++a)
            store_partial<D, DB>(PO, PL, item + (qw - q0) + 32 * a, oacc[a], l_run[a], m_run[a], n, h);
        return;
    }
    uint16_t* oh = O + head;
    float* lh = LSE + (int64_t)bh * Sq;
#pragma unroll
    for (int a = 0; a < 2; ++a) {
        const float l = halves_sum(l_run[a]);
        const float inv = 1.0f / l;
        const int qrow = qw + 32 * a + n;
        if (qrow < Sq) {
#pragma unroll
            for (int db = 0; db < DB; ++db)
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const int d = db * 32 + 8 * g + 4 * h;
                    if (d < D) {
                        u32x2 w;
                        w[0] = pack2<T>(oacc[a][db][4 * g + 0] * inv, oacc[a][db][4 * g + 1] * inv);
                        w[1] = pack2<T>(oacc[a][db][4 * g + 2] * inv, oacc[a][db][4 * g + 3] * inv);
                        *reinterpret_cast<u32x2*>(oh + (int64_t)qrow * D + d) = w;
                    }
                }
            if (h == 0) lh[qrow] = kLn2 * (m_run[a] + log2_fast(l));
        }
    }
}

}  // namespace fa
