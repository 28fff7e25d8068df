// fa_window.hpp -- matrix-core forward for a sliding window (fp16 / bf16).
//
// window_size = (left, right) ("Inside FlashAttention", section 6.1): query i
// attends to keys i - left .. i + right (a side of -1 is unlimited), and to no
// key past i when causal.  Like the causal split into off-band and on-band
// blocks ("Triton 实现", section "Causal Mask 的处理"; "T5 讲解", section ⑤), a
// workgroup visits only the key tiles its rows' window touches, and only tiles
// that cross a window edge (or the end of the sequence) take a mask; tiles
// inside every row's window take none.  Grouped heads read K/V head bh / G.
//
// The loop is the plain one of fa_mfma.hpp (one 32-key tile per barrier: S,
// mask, online softmax with the threshold rescale, P*V), with the tile range
// and the two-sided mask added: each wave owns 32 query rows, NW waves share
// the K/V tiles streamed HBM -> LDS.  A row whose keys start later than its
// wave's first tile sees only -inf there; its reference m stays at the initial
// value until its first visible key, which takes the rescale path.
#pragma once

#include "fa_mfma.hpp"

namespace fa {

template <typename T, typename Cfg>
__global__ __attribute__((amdgpu_flat_work_group_size(Cfg::NT, Cfg::NT), amdgpu_waves_per_eu(2, 2)))
void fa_fwd_window_kernel(const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
                          const uint16_t* __restrict__ V, uint16_t* __restrict__ O, float* __restrict__ LSE,
                          int Sq, int Sk, int BH, int n_qblk, int G, int wl, int wr, float c) {
    using W = WaveTile<T, Cfg>;
    constexpr int D = Cfg::D, KS = Cfg::KS, DB = Cfg::DB, RB = Cfg::RB, BM = Cfg::BM, BN = Cfg::BN;
    constexpr bool CAUSAL = Cfg::CAUSAL;
    static_assert(Cfg::QB == 1 && Cfg::KB == 1 && !Cfg::PIPE && Cfg::TBN == BN, "one 32-row block, 32-key tiles");

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
    const int qblk = wg / BH;
    const int q0 = qblk * BM;
    const int qw = q0 + 32 * wave;

    const int64_t head = (int64_t)bh * Sq * D;
    const int64_t kvhead = (int64_t)(bh / G) * Sk * D;
    const __amdgpu_buffer_rsrc_t krs = head_rsrc<T>(K + kvhead, Sk * RB);
    const __amdgpu_buffer_rsrc_t vrs = head_rsrc<T>(V + kvhead, Sk * RB);
    const uint32_t koff = tile_lane_offset<Cfg, false>(wave, lane);
    const uint32_t voff = tile_lane_offset<Cfg, true>(wave, lane);

    // keys of row i: lo(i) .. hi(i), an empty range when a window leaves the
    // row no key (only possible with fewer keys than queries)
    auto lo_of = [&](int i) { return wl >= 0 ? max(0, i - wl) : 0; };
    auto hi_of = [&](int i) { return min(min(CAUSAL ? i : Sk - 1, wr >= 0 ? i + wr : Sk - 1), Sk - 1); };
    const int qlast = min(q0 + BM, Sq) - 1;
    const int tb = lo_of(q0) / BN;              // the workgroup's key tiles [tb, te)
    const int te = hi_of(qlast) / BN + 1;
    const bool live = qw < Sq;
    const int wlast = min(qw + 31, Sq - 1);
    const int wb = live ? lo_of(qw) / BN : te;   // this wave's tiles [wb, we)
    const int we = live ? hi_of(wlast) / BN + 1 : te;
    // tiles in [ml, mu) lie inside every row's window: no mask
    const int ml = (lo_of(wlast) + BN - 1) / BN;
    const int mu = (hi_of(qw) + 1) / BN;
    const int qrow = min(qw + n, Sq - 1);
    const int first = lo_of(qrow), last = hi_of(qrow);

    load_tile<T, Cfg, false>(kbuf[0], krs, koff, tb * BN, wave, lane);
    load_tile<T, Cfg, true>(vbuf[0], vrs, voff, tb * BN, wave, lane);

    u32x4 qf[1][KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
        qf[0][ks] = *reinterpret_cast<const u32x4*>(Q + head + (int64_t)qrow * D + ks * 16 + h * 8);
    // (pinned once every load is in flight, so that their round trips overlap)
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) pin(qf[0][ks]);
    int offk[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) offk[ks] = n * RB + (((2 * ks + h) ^ swz_k<D>(n)) * 16);
    const int r16 = lane & 15, g16 = lane >> 4;
    const int vrow = 4 * h + (r16 >> 2);
    int offv[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) {
        const int dim = (32 * db + 16 * (g16 & 1) + 4 * (r16 & 3)) % D;
        offv[db] = vrow * RB + (((dim >> 3) ^ swz_v<D>(vrow)) * 16) + (dim & 7) * 2;
    }

    float m_run[1] = {kMInit}, l_run[1] = {0.f};
    f32x16 oacc[1][DB];
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[0][db][r] = 0.f;
    f32x16 s[1][1];
    u32x4 p[1][1][2];

    auto step = [&](auto par, int t) __attribute__((always_inline)) {
        constexpr int P = decltype(par)::value;
        wait_vmcnt0();
        __syncthreads();
        if (t + 1 < te) {
            load_tile<T, Cfg, false>(kbuf[1 - P], krs, koff, (t + 1) * BN, wave, lane);
            load_tile<T, Cfg, true>(vbuf[1 - P], vrs, voff, (t + 1) * BN, wave, lane);
        }
        if (t < wb || t >= we) return;  // wave-uniform
        W::qk(kbuf[P], offk, qf, s);
        if (t < ml || t >= mu) {
            // key of register r: 32t + 8(r/4) + 4h + r%4, visible iff first <= key <= last
            const int k0 = t * BN + 4 * h;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int key = k0 + 8 * (r >> 2) + (r & 3);
                if (key < first || key > last) s[0][0][r] = kNegInf;
            }
        }
        if (t == wb) {
            W::first(s, m_run, l_run, c, p);
        } else {
            float rs[1];
            W::expo(s, m_run, c, p, rs);
            if (W::needs_rescale(rs)) W::rescale(s, m_run, l_run, oacc, c, p, rs);
            l_run[0] += rs[0];
        }
        W::pv(vbuf[P], offv, p, oacc);
    };
    using P0 = std::integral_constant<int, 0>;
    using P1 = std::integral_constant<int, 1>;
    int t = tb;
    for (; t + 1 < te; t += 2) {
        step(P0{}, t);
        step(P1{}, t + 1);
    }
    if (t < te) step(P0{}, t);

    // ---- epilogue: O = acc / l, lse = ln2 * (m + log2 l) ---------------------------
    // (a row with no key has l = 0 and acc = 0: O = 0 and lse = ln2 * log2 0 = -inf)
    const float l = halves_sum(l_run[0]);
    const float inv = l > 0.f ? 1.0f / l : 0.f;
    if (qw + n < Sq) {
        uint16_t* oh = O + head;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int d = db * 32 + 8 * g + 4 * h;
                if (d < D) {
                    u32x2 w;
                    w[0] = pack2<T>(oacc[0][db][4 * g + 0] * inv, oacc[0][db][4 * g + 1] * inv);
                    w[1] = pack2<T>(oacc[0][db][4 * g + 2] * inv, oacc[0][db][4 * g + 3] * inv);
                    *reinterpret_cast<u32x2*>(oh + (int64_t)(qw + n) * D + d) = w;
                }
            }
        if (h == 0) LSE[(int64_t)bh * Sq + qw + n] = kLn2 * (m_run[0] + log2_fast(l));
    }
}

}  // namespace fa
