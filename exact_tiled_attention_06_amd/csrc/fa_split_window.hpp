// fa_split_window.hpp -- the two-block forward kernel of fa_split.hpp for
// sliding windows (fp16 / bf16, D = 32 and 64).
//
// window_size = (left, right) limits query i to keys lo(i) .. hi(i),
// lo = max(0, i - left), hi = min(i (causal), i + right, S_k - 1), and whole
// tiles outside a block's window are skipped like the tiles above the causal
// diagonal ("Inside FlashAttention", section 6.1).  A wave owns two 32-query
// column blocks a = 0, 1 offset by half a tile, exactly as in fa_split.hpp:
//
//   H(t,0):  softmax(t, 0)   |  P*V(t-1, 1),  S(t, 1)
//   H(t,1):  softmax(t, 1)   |  P*V(t, 0),    S(t+1, 0)
//
// but each block walks its own tile range [wb, we) (lo and hi are
// non-decreasing in i, so a block's rows see one contiguous range, and the
// tiles inside every row's window form one interval [ml, mu) that needs no
// mask).  The workgroup stages the union [tbeg, tend) of its rows' ranges,
// one 32-key tile per barrier; the half-steps in the middle, where both
// blocks are past their first tile and unmasked, are SplitTile::half with
// compile-time buffers, the rest run under the range conditions.  A row whose
// window holds no key (possible only with fewer keys than queries) keeps the
// initial reference m and l = 0, and is written as O = 0, lse = -inf.
#pragma once

#include "fa_split.hpp"

namespace fa {

template <typename T, typename Cfg>
__global__ __attribute__((amdgpu_flat_work_group_size(Cfg::NT, Cfg::NT), amdgpu_waves_per_eu(Cfg::OCC, Cfg::OCC)))
void fa_fwd_split_window_kernel(const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
                                const uint16_t* __restrict__ V, uint16_t* __restrict__ O, float* __restrict__ LSE,
                                int Sq, int Sk, int BH, int n_qblk, int G, int wl, int wr, float c) {
    using ST = SplitTile<T, Cfg>;
    constexpr int D = Cfg::D, KS = Cfg::KS, DB = Cfg::DB;
    constexpr int BN = Cfg::BN, BM = Cfg::BM, BMW = Cfg::BMW, RB = Cfg::RB;
    constexpr bool CAUSAL = Cfg::CAUSAL;
    static_assert(Cfg::TBN == BN, "one compute tile per LDS tile");

    // LDS tile j (buffers j % 2) holds K of compute tile tbeg + j + 1 and V of
    // tile tbeg + j; K(tbeg) sits in the other K buffer before the loop.
    __shared__ __attribute__((aligned(1024))) char k_lds0[Cfg::TILE];
    __shared__ __attribute__((aligned(1024))) char k_lds1[Cfg::TILE];
    __shared__ __attribute__((aligned(1024))) char v_lds0[Cfg::TILE];
    __shared__ __attribute__((aligned(1024))) char v_lds1[Cfg::TILE];
    FA_LDS char* const kbuf[2] = {(FA_LDS char*)k_lds0, (FA_LDS char*)k_lds1};
    FA_LDS char* const vbuf[2] = {(FA_LDS char*)v_lds0, (FA_LDS char*)v_lds1};

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int n = lane & 31;
    const int h = lane >> 5;

    const int wg = blockIdx.x;
    const int bh = wg % BH;
    const int q0 = (wg / BH) * BM;
    const int qw = q0 + wave * BMW;

    const int64_t head = (int64_t)bh * Sq * D;
    const int64_t kvhead = (int64_t)(bh / G) * Sk * D;  // grouped heads: G query heads per K/V head
    const __amdgpu_buffer_rsrc_t krs = head_rsrc<T>(K + kvhead, Sk * RB);
    const __amdgpu_buffer_rsrc_t vrs = head_rsrc<T>(V + kvhead, Sk * RB);
    const uint32_t koff = tile_lane_offset<Cfg, false>(wave, lane);
    const uint32_t voff = tile_lane_offset<Cfg, true>(wave, lane);

    // keys of row i: lo(i) .. hi(i) (hi >= 0 since S_k >= 1)
    auto lo_of = [&](int i) { return wl >= 0 ? max(0, i - wl) : 0; };
    auto hi_of = [&](int i) { return min(min(CAUSAL ? i : Sk - 1, wr >= 0 ? i + wr : Sk - 1), Sk - 1); };
    const int qlast = min(q0 + BM, Sq) - 1;
    const int tbeg = lo_of(q0) / BN;      // the workgroup's tiles [tbeg, tend)
    const int tend = hi_of(qlast) / BN + 1;

    // per block a (rows qw + 32a ..): tiles [wb, we), unmasked tiles [ml, mu),
    // and the lane's row's key range first .. last
    int wb[2], we[2], ml[2], mu[2], first[2], last[2];
#pragma unroll
    for (int a = 0; a < 2; ++a) {
        const int r0 = qw + 32 * a;
        const int rl = min(r0 + 31, Sq - 1);
        const bool live = r0 < Sq;
        wb[a] = live ? lo_of(r0) / BN : tend;
        we[a] = live ? hi_of(rl) / BN + 1 : tend;
        ml[a] = (lo_of(rl) + BN - 1) / BN;
        mu[a] = (hi_of(r0) + 1) / BN;
        const int qrow = min(r0 + n, Sq - 1);
        first[a] = lo_of(qrow);
        last[a] = hi_of(qrow);
    }

    // prologue transfers: K(tbeg) (this wave's share), K(tbeg+1) and V(tbeg)
    {
        constexpr int K0_LOADS = BN * RB / 1024;
        static_assert(K0_LOADS <= Cfg::NW, "K(tbeg) in one transfer per wave");
        if (wave < K0_LOADS) load_part<T, Cfg>(kbuf[1] + wave * 1024, krs, koff, tbeg * BN);
    }
    load_tile<T, Cfg, false>(kbuf[0], krs, koff, (tbeg + 1) * BN, wave, lane);
    load_tile<T, Cfg, true>(vbuf[0], vrs, voff, tbeg * BN, wave, lane);

    // Q^T operand fragments, resident for the whole loop ("T5 讲解", section ③)
    u32x4 qf[2][KS];
#pragma unroll
    for (int a = 0; a < 2; ++a) {
        const int qrow = min(qw + 32 * a + n, Sq - 1);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
            qf[a][ks] = *reinterpret_cast<const u32x4*>(Q + head + (int64_t)qrow * D + ks * 16 + h * 8);
    }
    // (pinned once every load is in flight, so that their round trips overlap)
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
    ST::read_k(kbuf[1], offk, kfr);
    if (tbeg >= wb[0] && tbeg < we[0]) ST::qk(kfr, qf[0], s[0]);

    auto in = [](int t, int b, int e) { return t >= b && t < e; };
    // Generic half-step: the pipeline's work for the blocks whose ranges hold
    // it, the two-sided mask outside [ml, mu), the first tile's reference.
    auto half_any = [&](auto blk, int t) __attribute__((always_inline)) {
        constexpr int A = decltype(blk)::value, B = 1 - A;
        const int tb = A == 0 ? t - 1 : t;  // the P*V tile of block B
        const int tq = A == 0 ? t : t + 1;  // the S tile of block B
        if (in(tb, wb[B], we[B])) ST::pv(vfr, p[B], oacc[B]);
        if (in(tq, wb[B], we[B])) ST::qk(kfr, qf[B], s[B]);
        if (in(t, wb[A], we[A])) {
            if (t < ml[A] || t >= mu[A]) {
                // key of register r: 32t + 8(r/4) + 4h + r%4, visible iff first <= key <= last
                const int k0 = t * BN + 4 * h;
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int key = k0 + 8 * (r >> 2) + (r & 3);
                    if (key < first[A] || key > last[A]) s[A][r] = kNegInf;
                }
            }
            if (t == wb[A]) {
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

    // Between the half-steps of tile t (LDS tile j = t - tbeg, buffers j % 2):
    // wait for it and barrier, read K(t+1) and V(t), then stage LDS tile j+1
    // into the other buffers (their fragments were read before the barrier).
    auto sync_with = [&](int t, FA_LDS char* kc, FA_LDS char* vc, FA_LDS char* kn, FA_LDS char* vn)
                         __attribute__((always_inline)) {
        wait_vmcnt0();
        __syncthreads();
        __builtin_amdgcn_sched_barrier(0);
        ST::read_k(kc, offk, kfr);
        ST::read_v(vc, offv, vfr);
        __builtin_amdgcn_sched_barrier(0);
        if (t + 1 < tend) {
            load_tile<T, Cfg, false>(kn, krs, koff, (t + 2) * BN, wave, lane);
            load_tile<T, Cfg, true>(vn, vrs, voff, (t + 1) * BN, wave, lane);
        }
    };
    auto sync = [&](auto par, int t) __attribute__((always_inline)) {
        constexpr int P = decltype(par)::value;
        sync_with(t, kbuf[P], vbuf[P], kbuf[1 - P], vbuf[1 - P]);
    };
    auto sync_rt = [&](int t) __attribute__((always_inline)) {
        const bool odd = (t - tbeg) & 1;
        sync_with(t, odd ? kbuf[1] : kbuf[0], odd ? vbuf[1] : vbuf[0], odd ? kbuf[0] : kbuf[1],
                  odd ? vbuf[0] : vbuf[1]);
    };
    auto generic = [&](int t) __attribute__((always_inline)) {
        half_any(A0{}, t);
        sync_rt(t);
        half_any(A1{}, t);
    };
    auto steady = [&](auto par, int t) __attribute__((always_inline)) {
        steady_half(A0{});
        sync(par, t);
        steady_half(A1{});
    };
    using P0 = std::integral_constant<int, 0>;
    using P1 = std::integral_constant<int, 1>;

    // steady for ts0 <= t < ts1: both blocks past their first tile, unmasked,
    // every MFMA of both half-steps present (block 1's P*V of t-1 and S of t,
    // block 0's S of t+1)
    const int ts0 = max(max(wb[0], wb[1]) + 1, max(ml[0], ml[1]));
    const int ts1 = min(min(we[1], we[0] - 1), min(mu[0], mu[1]));
    int t = tbeg;
    for (; t < tend && t < ts0; ++t) generic(t);
    if (t < ts1 && ((t - tbeg) & 1)) steady(P1{}, t++);
    for (; t + 1 < ts1; t += 2) {
        steady(P0{}, t);
        steady(P1{}, t + 1);
    }
    if (t < ts1) steady(P0{}, t++);
    for (; t < tend; ++t) generic(t);
    // P*V of block 1's last tile when it is the workgroup's last (V still in vfr)
    if (in(tend - 1, wb[1], we[1])) ST::pv(vfr, p[1], oacc[1]);

    // ---- epilogue: O = acc / l, lse = ln2 * (m + log2 l) ---------------------------
    // (a row with no key has l = 0 and acc = 0: O = 0 and lse = ln2 * log2 0 = -inf)
    uint16_t* oh = O + head;
    float* lh = LSE + (int64_t)bh * Sq;
#pragma unroll
    for (int a = 0; a < 2; ++a) {
        const float l = halves_sum(l_run[a]);
        const float inv = l > 0.f ? 1.0f / l : 0.f;
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
