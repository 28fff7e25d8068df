// fa_bwd.hpp -- FlashAttention-2 backward for fp16 / bf16 inputs on the gfx950
// matrix cores.
//
// Gradients of O = softmax(scale * Q K^T) V for an upstream gradient dO, with
// the probabilities recomputed block by block from the saved natural-log lse
// instead of stored ("从零训练语言模型（第二部分）", sections "使用 LSE 连接正向和
// 反向传播" and "反向传播"):
//     P   = exp(scale * Q K^T - lse)        (masked keys: 0)
//     dV  = P^T dO          dP = dO V^T
//     dS  = P o (dP - D),   D_i = rowsum(dO_i o O_i)
//     dQ  = scale * dS K    dK = scale * dS^T Q
// Two kernels, no atomics:
//   fa_bwd_dq_kernel    query blocks outer, K/V tiles inner (the forward's
//                       schedule): dQ stays in registers.  It also forms D for
//                       its rows from O and dO and writes it to a workspace.
//   fa_bwd_dkdv_kernel  key blocks outer, Q/dO tiles inner (the schedule the
//                       page gives for dK and dV): dK and dV stay in registers.
// S and dP are recomputed by both, so the pair runs 7 tile products instead of
// the 5 of a single pass that scatters dQ with atomics; in exchange every
// output is written once, deterministically, in its input type.
//
// Layout conventions are the forward's (fa_mfma.hpp): 32x32x16 MFMAs; a wave
// owns 32 rows (queries in the dQ kernel, keys in the dK/dV kernel) whose
// operand fragments stay in VGPRs; the streamed tiles (32 rows) go HBM -> LDS by
// buffer_load ... lds, stored once per way they are read: "row" layout for
// ds_read_b128 fragments whose k index is the head dimension, "transposed"
// layout for ds_read_b64_tr_b16 fragments whose k index is the row.
//   dQ kernel, per K/V tile:   S^T = K Q^T, dP^T = V dO^T  (lane = query)
//                              dQ^T += K^T dS^T
//   dK/dV kernel, per Q tile:  S = Q K^T, dP = dO V^T      (lane = key)
//                              dV^T += dO^T P,  dK^T += Q^T dS
// P and dS are rounded (nearest-even) to the input type for the MFMAs that
// consume them, as the forward rounds P.
#pragma once

#include "fa_mfma.hpp"

namespace fa {

template <int D_, bool CAUSAL_, int NW_, int QBQ_ = (D_ == 128 ? 1 : 2), int QS_ = 1, int KSQ_ = 1>
struct BwdConfig {
    using L = MfmaConfig<D_, CAUSAL_, 1, NW_, 32>;  // staging of 32-row tiles, fragment offsets
    static constexpr int D = D_, NW = NW_;
    static constexpr bool CAUSAL = CAUSAL_;
    static constexpr int KS = L::KS, DB = L::DB, RB = L::RB, TILE = L::TILE;
    static constexpr int NT = 64 * NW;
    // dK/dV kernel: QS groups of NW waves share a key block and split its
    // query steps (QS = 2 doubles the waves of a thin grid)
    static constexpr int QS = QS_;
    static constexpr int NT_KV = 64 * NW * QS;
    static_assert(QS == 1 || (QS == 2 && (D == 32 || D == 64)), "query split of the dK/dV kernel");
    // dQ kernel: KSQ groups of NW waves share a query block and split its
    // key tiles (KSQ = 2 doubles the waves of a thin grid)
    static constexpr int KSQ = KSQ_;
    static constexpr int NT_Q = 64 * NW * KSQ;
    static_assert(KSQ == 1 || (KSQ == 2 && QBQ_ == 1 && D >= 32), "key split of the dQ kernel");
    static constexpr int BM = 32 * NW;  // keys per dK/dV workgroup
    // dQ kernel: 32-query blocks per wave (two halve its LDS reads per MFMA;
    // D = 128 has no registers for a second set; one doubles the waves of a
    // thin grid) and queries per workgroup
    static constexpr int QBQ = QBQ_;
    static_assert(QBQ == 1 || (QBQ == 2 && D <= 64), "query blocks per dQ wave");
    static constexpr int BMQ = 32 * QBQ * NW;
    // D = 128 keeps two accumulators of 64 registers each in the dK/dV kernel
    static constexpr int OCC_DQ = 2;
    static constexpr int OCC_KV = D == 128 ? 1 : 2;
};

// Sum over the eight element products of two packed operands, in fp32.
template <typename T>
__device__ __forceinline__ float dot8(u32x4 a, u32x4 b);

template <>
__device__ __forceinline__ float dot8<F16>(u32x4 a, u32x4 b) {
    const f16x8 x = __builtin_bit_cast(f16x8, a), y = __builtin_bit_cast(f16x8, b);
    float s = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) s = __builtin_fmaf((float)x[e], (float)y[e], s);
    return s;
}

template <>
__device__ __forceinline__ float dot8<BF16>(u32x4 a, u32x4 b) {
    const bf16x8 x = __builtin_bit_cast(bf16x8, a), y = __builtin_bit_cast(bf16x8, b);
    float s = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) s = __builtin_fmaf((float)x[e], (float)y[e], s);
    return s;
}

// Operand fragments of one row of a [S,D] head: lane (n, h) gets
// X[row][16ks + 8h .. +7] for every k-step ks (row clamped to S-1).  The
// loads are only issued here; pin_frags, called once every load is in flight,
// keeps them resident.
template <int KS>
__device__ __forceinline__ void row_frags(const uint16_t* xh, int row, int D, int h, u32x4 (&f)[KS]) {
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) f[ks] = *reinterpret_cast<const u32x4*>(xh + (int64_t)row * D + ks * 16 + h * 8);
}

template <int KS>
__device__ __forceinline__ void pin_frags(u32x4 (&f)[KS]) {
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) pin(f[ks]);
}

// Compiler-only barrier: memory accesses are not moved across it, so loads
// before it are issued before those after it.
__device__ __forceinline__ void issue_order() { asm volatile("" ::: "memory"); }

// LDS byte offsets of a lane's fragment reads (the forward's formulas): row
// reads of chunk (2ks + h), and the transposed reads of dims 32db + ...
template <typename Cfg>
__device__ __forceinline__ void frag_offsets(int lane, int (&offk)[Cfg::KS], int (&offv)[Cfg::DB]) {
    constexpr int D = Cfg::D, RB = Cfg::RB;
    const int n = lane & 31, h = lane >> 5;
#pragma unroll
    for (int ks = 0; ks < Cfg::KS; ++ks) offk[ks] = n * RB + (((2 * ks + h) ^ swz_k<D>(n)) * 16);
    const int r16 = lane & 15, g16 = lane >> 4;
    const int vrow = 4 * h + (r16 >> 2);
#pragma unroll
    for (int db = 0; db < Cfg::DB; ++db) {
        const int dim = (32 * db + 16 * (g16 & 1) + 4 * (r16 & 3)) % D;
        offv[db] = vrow * RB + (((dim >> 3) ^ swz_v<D>(vrow)) * 16) + (dim & 7) * 2;
    }
}

// Store a 32-row block held as X^T accumulators (rows = dims 32db + 8g + 4h +
// 0..3, lane column = row of X), times `mul`, rounded to T.
template <typename T, int D, int DB>
__device__ __forceinline__ void store_t(uint16_t* xh, int row, int h, const f32x16 (&acc)[DB], float mul) {
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const int d = db * 32 + 8 * g + 4 * h;
            if (d < D) {
                u32x2 w;
                w[0] = pack2<T>(acc[db][4 * g + 0] * mul, acc[db][4 * g + 1] * mul);
                w[1] = pack2<T>(acc[db][4 * g + 2] * mul, acc[db][4 * g + 3] * mul);
                *reinterpret_cast<u32x2*>(xh + (int64_t)row * D + d) = w;
            }
        }
}

// ------------------------------------------------------------------ dQ kernel

template <typename T, typename Cfg>
__global__ __attribute__((amdgpu_flat_work_group_size(Cfg::NT_Q, Cfg::NT_Q), amdgpu_waves_per_eu(Cfg::OCC_DQ, Cfg::OCC_DQ)))
void fa_bwd_dq_kernel(const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
                      const uint16_t* __restrict__ V, const uint16_t* __restrict__ O,
                      const uint16_t* __restrict__ dO, const float* __restrict__ LSE,
                      uint16_t* __restrict__ dQ, float* __restrict__ DELTA, int Sq, int Sk, int BH, int n_blk, int G,
                      int wl, int wr, float c, float scale) {
    using L = typename Cfg::L;
    using W = WaveTile<T, L>;
    constexpr int D = Cfg::D, KS = Cfg::KS, DB = Cfg::DB, RB = Cfg::RB;
    constexpr bool CAUSAL = Cfg::CAUSAL;

    constexpr int KSQ = Cfg::KSQ;

    // per K/V tile: K row layout (S^T operand), K transposed layout (dQ^T
    // operand), V row layout (dP^T operand); two buffers each, one slice of
    // each per wave group
    __shared__ __attribute__((aligned(1024))) char kr0[KSQ * Cfg::TILE];
    __shared__ __attribute__((aligned(1024))) char kr1[KSQ * Cfg::TILE];
    __shared__ __attribute__((aligned(1024))) char kt0[KSQ * Cfg::TILE];
    __shared__ __attribute__((aligned(1024))) char kt1[KSQ * Cfg::TILE];
    __shared__ __attribute__((aligned(1024))) char vr0[KSQ * Cfg::TILE];
    __shared__ __attribute__((aligned(1024))) char vr1[KSQ * Cfg::TILE];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    // Wave group grp (of KSQ) walks its share of the query block's key tiles;
    // `wave` is the wave's index in its group, which fixes its queries and
    // its share of the staging.
    const int grp = KSQ == 1 ? 0 : __builtin_amdgcn_readfirstlane(tid >> 6) / Cfg::NW;
    const int wave = KSQ == 1 ? __builtin_amdgcn_readfirstlane(tid >> 6) : __builtin_amdgcn_readfirstlane(tid >> 6) % Cfg::NW;
    const int gt = grp * Cfg::TILE;
    FA_LDS char* const krb[2] = {(FA_LDS char*)kr0 + gt, (FA_LDS char*)kr1 + gt};
    FA_LDS char* const ktb[2] = {(FA_LDS char*)kt0 + gt, (FA_LDS char*)kt1 + gt};
    FA_LDS char* const vrb[2] = {(FA_LDS char*)vr0 + gt, (FA_LDS char*)vr1 + gt};
    const int n = lane & 31;
    const int h = lane >> 5;

    // heads vary fastest; causal query blocks longest first.  A wave owns QB
    // blocks of 32 queries (rows qw + 32a ..), so each K, V and K^T fragment
    // read from LDS feeds QB MFMAs.
    constexpr int QB = Cfg::QBQ;
    constexpr int BMQ = Cfg::BMQ;
    const int wg = blockIdx.x;
    const int bh = wg % BH;
    const int rank = wg / BH;
    const int qblk = CAUSAL ? (n_blk - 1 - rank) : rank;
    const int q0 = qblk * BMQ;
    const int qw = q0 + 32 * QB * wave;

    const int64_t head = (int64_t)bh * Sq * D;
    const int64_t kvhead = (int64_t)(bh / G) * Sk * D;  // grouped heads: G query heads per K/V head
    const __amdgpu_buffer_rsrc_t krs = head_rsrc<T>(K + kvhead, Sk * RB);
    const __amdgpu_buffer_rsrc_t vrs = head_rsrc<T>(V + kvhead, Sk * RB);
    const uint32_t roff = tile_lane_offset<L, false>(wave, lane);
    const uint32_t toff = tile_lane_offset<L, true>(wave, lane);

    // keys of query i: lo(i) .. hi(i) (causal: up to i; window: i - wl .. i + wr)
    auto lo_of = [&](int i) { return wl >= 0 ? max(0, i - wl) : 0; };
    auto hi_of = [&](int i) { return min(min(CAUSAL ? i : Sk - 1, wr >= 0 ? i + wr : Sk - 1), Sk - 1); };
    const int qlast = min(q0 + BMQ, Sq) - 1;
    const int tb = lo_of(q0) / 32;                 // the workgroup's key tiles [tb, te)
    const int te = hi_of(qlast) / 32 + 1;
    // group grp takes tiles [tgb, tge); every group runs nth steps, a group
    // with fewer tiles as padding (staging nothing, computing nothing)
    const int nth = KSQ == 1 ? te - tb : max(0, (te - tb + KSQ - 1) / KSQ);
    const int tgb = KSQ == 1 ? tb : tb + grp * nth;
    const int tge = KSQ == 1 ? te : min(te, tgb + nth);
    // per block a: tiles in [ml, mu) need no mask; the wave computes tiles
    // [wb, we), the union over its blocks (a block masks the tiles outside its
    // own range entirely)
    int ml[QB], mu[QB], first[QB], last[QB], qrow[QB];
    int wb = te, we = te;
#pragma unroll
    for (int a = 0; a < QB; ++a) {
        const int r0 = qw + 32 * a;
        const int rl = min(r0 + 31, Sq - 1);
        ml[a] = r0 < Sq ? (lo_of(rl) + 31) / 32 : te;
        mu[a] = r0 < Sq ? (hi_of(r0) + 1) / 32 : 0;
        if (r0 < Sq) {
            wb = min(wb, lo_of(r0) / 32);
            we = a == 0 ? hi_of(rl) / 32 + 1 : max(we, hi_of(rl) / 32 + 1);
        }
        qrow[a] = min(r0 + n, Sq - 1);
        first[a] = lo_of(qrow[a]);
        last[a] = hi_of(qrow[a]);
    }

    auto stage = [&](auto par, int t) __attribute__((always_inline)) {
        constexpr int P = decltype(par)::value;
        load_tile<T, L, false>(krb[P], krs, roff, t * 32, wave, lane);
        load_tile<T, L, true>(ktb[P], krs, toff, t * 32, wave, lane);
        load_tile<T, L, false>(vrb[P], vrs, roff, t * 32, wave, lane);
    };
    using P0 = std::integral_constant<int, 0>;
    using P1 = std::integral_constant<int, 1>;

    // resident: Q and dO fragments of the wave's queries; D = rowsum(dO o O).
    // Every fragment load is issued before the first tile's staging, and the
    // values are waited for after it, so the two overlap.
    u32x4 qf[QB][KS], df[QB][KS], of[QB][KS];
    float lsev[QB];  // the rows' lse, loaded with the fragments
#pragma unroll
    for (int a = 0; a < QB; ++a) {
        row_frags<KS>(Q + head, qrow[a], D, h, qf[a]);
        row_frags<KS>(dO + head, qrow[a], D, h, df[a]);
        row_frags<KS>(O + head, qrow[a], D, h, of[a]);
        lsev[a] = LSE[(int64_t)bh * Sq + qrow[a]];
    }
    issue_order();
    // a block with no key tile (a window that leaves its rows no key, S_k < S_q)
    // stages nothing: no LDS transfer may outlive the workgroup
    if (tgb < tge) stage(P0{}, tgb);
    float delta[QB], lse2[QB];
#pragma unroll
    for (int a = 0; a < QB; ++a) {
        pin_frags<KS>(qf[a]);
        pin_frags<KS>(df[a]);
        float part = 0.f;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) part += dot8<T>(df[a][ks], of[a][ks]);
        delta[a] = halves_sum(part);
        if (grp == 0 && h == 0 && qw + 32 * a + n < Sq) DELTA[(int64_t)bh * Sq + qw + 32 * a + n] = delta[a];
        // a row with no key (lse = -inf; all its scores are masked to -inf)
        // takes +inf, so that its masked scores give exp2(-inf) = 0
        lse2[a] = first[a] <= last[a] ? lsev[a] * kLog2e : __builtin_inff();
    }

    int offk[KS], offv[DB];
    frag_offsets<L>(lane, offk, offv);

    f32x16 dqacc[QB][DB];
#pragma unroll
    for (int a = 0; a < QB; ++a)
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int r = 0; r < 16; ++r) dqacc[a][db][r] = 0.f;

    auto step = [&](auto par, int t) __attribute__((always_inline)) {
        constexpr int P = decltype(par)::value;
        wait_vmcnt0();
        __syncthreads();
        if (t + 1 < tge) stage(std::integral_constant<int, 1 - P>{}, t + 1);
        if ((KSQ > 1 && t >= tge) || t < wb || t >= we) return;  // wave-uniform
        const f32x16 zero = {};
        f32x16 st[QB], dpt[QB];
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const u32x4 kfr = W::k_frag(krb[P], offk, 0, ks);
            const u32x4 vfr = W::k_frag(vrb[P], offk, 0, ks);
#pragma unroll
            for (int a = 0; a < QB; ++a) {
                st[a] = mfma32x32x16<T>(kfr, qf[a][ks], ks == 0 ? zero : st[a]);
                // the dP^T chain starts from -D, so that it ends at dP^T - D
                f32x16 nd;
#pragma unroll
                for (int r = 0; r < 16; ++r) nd[r] = -delta[a];
                dpt[a] = mfma32x32x16<T>(vfr, df[a][ks], ks == 0 ? nd : dpt[a]);
            }
        }
        u32x4 dsp[QB][2];
#pragma unroll
        for (int a = 0; a < QB; ++a) {
            if (t < ml[a] || t >= mu[a]) {
                // key of register r: 32t + 8(r/4) + 4h + r%4, visible iff first <= key <= last
                const int k0 = t * 32 + 4 * h;
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int key = k0 + 8 * (r >> 2) + (r & 3);
                    if (key < first[a] || key > last[a]) st[a][r] = kNegInf;
                }
            }
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const float p0 = exp2_fast(__builtin_fmaf(st[a][2 * i], c, -lse2[a]));
                const float p1 = exp2_fast(__builtin_fmaf(st[a][2 * i + 1], c, -lse2[a]));
                dsp[a][i >> 2][i & 3] = pack2<T>(p0 * dpt[a][2 * i], p1 * dpt[a][2 * i + 1]);
            }
        }
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int db = 0; db < DB; ++db) {
                const u32x4 ktf = W::v_frag(ktb[P], offv, 0, j, db);
#pragma unroll
                for (int a = 0; a < QB; ++a) dqacc[a][db] = mfma32x32x16<T>(ktf, dsp[a][j], dqacc[a][db]);
            }
    };
    int i = 0;
    for (; i + 1 < nth; i += 2) {
        step(P0{}, tgb + i);
        step(P1{}, tgb + i + 1);
    }
    if (i < nth) step(P0{}, tgb + i);

    if constexpr (KSQ == 2) {
        // group 1 hands its fp32 partial dQ to group 0 through LDS (one
        // staging array per wave, free once every wave is past the loop)
        static_assert(Cfg::NW <= 4 && QB == 1 && DB * 16 * 64 * 4 <= KSQ * Cfg::TILE, "exchange fits");
        wait_vmcnt0();
        __syncthreads();
        float* const x = (float*)(wave == 0 ? kr0 : wave == 1 ? kr1 : wave == 2 ? kt0 : kt1);
        if (grp == 1) {
#pragma unroll
            for (int db = 0; db < DB; ++db)
#pragma unroll
                for (int r = 0; r < 16; ++r) x[(db * 16 + r) * 64 + lane] = dqacc[0][db][r];
        }
        __syncthreads();
        if (grp == 1) return;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int r = 0; r < 16; ++r) dqacc[0][db][r] += x[(db * 16 + r) * 64 + lane];
    }

#pragma unroll
    for (int a = 0; a < QB; ++a)
        if (qw + 32 * a + n < Sq) store_t<T, D, DB>(dQ + head, qw + 32 * a + n, h, dqacc[a], scale);
}

// ---------------------------------------------------------------- dK/dV kernel

template <typename T, typename Cfg>
__global__ __attribute__((amdgpu_flat_work_group_size(Cfg::NT_KV, Cfg::NT_KV),
                          amdgpu_waves_per_eu(Cfg::OCC_KV, Cfg::OCC_KV)))
void fa_bwd_dkdv_kernel(const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
                        const uint16_t* __restrict__ V, const uint16_t* __restrict__ dO,
                        const float* __restrict__ LSE, const float* __restrict__ DELTA,
                        uint16_t* __restrict__ dK, uint16_t* __restrict__ dV, int Sq, int Sk, int BHkv, int n_blk, int G,
                        int wl, int wr, float c, float scale) {
    using L = typename Cfg::L;
    using W = WaveTile<T, L>;
    constexpr int D = Cfg::D, KS = Cfg::KS, DB = Cfg::DB, RB = Cfg::RB, BM = Cfg::BM;
    constexpr bool CAUSAL = Cfg::CAUSAL;

    constexpr int QS = Cfg::QS;

    // per Q/dO tile: Q row layout (S operand), Q transposed layout (dK^T
    // operand), dO row layout (dP operand), dO transposed layout (dV^T
    // operand), and the tile's 32 lse and D values; three buffers each, so
    // that tiles are staged two steps ahead; one slice of each per wave group
    __shared__ __attribute__((aligned(1024))) char qr0[QS * Cfg::TILE];
    __shared__ __attribute__((aligned(1024))) char qr1[QS * Cfg::TILE];
    __shared__ __attribute__((aligned(1024))) char qr2[QS * Cfg::TILE];
    __shared__ __attribute__((aligned(1024))) char qt0[QS * Cfg::TILE];
    __shared__ __attribute__((aligned(1024))) char qt1[QS * Cfg::TILE];
    __shared__ __attribute__((aligned(1024))) char qt2[QS * Cfg::TILE];
    __shared__ __attribute__((aligned(1024))) char or0[QS * Cfg::TILE];
    __shared__ __attribute__((aligned(1024))) char or1[QS * Cfg::TILE];
    __shared__ __attribute__((aligned(1024))) char or2[QS * Cfg::TILE];
    __shared__ __attribute__((aligned(1024))) char ot0[QS * Cfg::TILE];
    __shared__ __attribute__((aligned(1024))) char ot1[QS * Cfg::TILE];
    __shared__ __attribute__((aligned(1024))) char ot2[QS * Cfg::TILE];
    __shared__ __attribute__((aligned(16))) float ls0[QS * 32];
    __shared__ __attribute__((aligned(16))) float ls1[QS * 32];
    __shared__ __attribute__((aligned(16))) float ls2[QS * 32];
    __shared__ __attribute__((aligned(16))) float dl0[QS * 32];
    __shared__ __attribute__((aligned(16))) float dl1[QS * 32];
    __shared__ __attribute__((aligned(16))) float dl2[QS * 32];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    // Wave group grp (of QS) walks its share of the key block's query steps;
    // `wave` is the wave's index in its group, which fixes its keys and its
    // share of the staging.
    const int grp = QS == 1 ? 0 : __builtin_amdgcn_readfirstlane(tid >> 6) / Cfg::NW;
    const int wave = QS == 1 ? __builtin_amdgcn_readfirstlane(tid >> 6) : __builtin_amdgcn_readfirstlane(tid >> 6) % Cfg::NW;
    const int gt = grp * Cfg::TILE, gs = grp * 32;
    FA_LDS char* const qrb[3] = {(FA_LDS char*)qr0 + gt, (FA_LDS char*)qr1 + gt, (FA_LDS char*)qr2 + gt};
    FA_LDS char* const qtb[3] = {(FA_LDS char*)qt0 + gt, (FA_LDS char*)qt1 + gt, (FA_LDS char*)qt2 + gt};
    FA_LDS char* const orb[3] = {(FA_LDS char*)or0 + gt, (FA_LDS char*)or1 + gt, (FA_LDS char*)or2 + gt};
    FA_LDS char* const otb[3] = {(FA_LDS char*)ot0 + gt, (FA_LDS char*)ot1 + gt, (FA_LDS char*)ot2 + gt};
    FA_LDS float* const lsb[3] = {(FA_LDS float*)ls0 + gs, (FA_LDS float*)ls1 + gs, (FA_LDS float*)ls2 + gs};
    FA_LDS float* const dlb[3] = {(FA_LDS float*)dl0 + gs, (FA_LDS float*)dl1 + gs, (FA_LDS float*)dl2 + gs};

    const int n = lane & 31;
    const int h = lane >> 5;

    // K/V heads vary fastest; causal key blocks with the most queries (lowest
    // keys) first.  The workgroup owns keys k0 .. k0+BM-1 of K/V head kvbh and
    // walks, for each of the G query heads that read it, the query tiles that
    // can see any of its keys.
    const int wg = blockIdx.x;
    const int kvbh = wg % BHkv;
    const int kblk = wg / BHkv;
    const int k0 = kblk * BM;
    const int kw = k0 + 32 * wave;

    const int64_t kvhead = (int64_t)kvbh * Sk * D;
    const uint32_t roff = tile_lane_offset<L, false>(wave, lane);
    const uint32_t toff = tile_lane_offset<L, true>(wave, lane);

    // queries that see key j: ilo(j) .. ihi(j) (causal: from j; window: j - wr .. j + wl)
    auto ilo_of = [&](int j) { return max(CAUSAL ? j : 0, wr >= 0 ? j - wr : 0); };
    auto ihi_of = [&](int j) { return min(Sq - 1, wl >= 0 ? j + wl : Sq - 1); };
    const int klast = min(k0 + BM, Sk) - 1;
    const int t0 = ilo_of(k0) / 32;                  // query tiles [t0, t1) of each head
    const int t1 = ihi_of(klast) / 32 + 1;
    const int nt = t1 - t0;
    const int nsteps = G * nt;
    const bool live = kw < Sk;                       // the wave has keys
    const int kwlast = min(kw + 31, Sk - 1);
    const int tw0 = live ? ilo_of(kw) / 32 : t1;     // this wave's query tiles [tw0, tw1)
    const int tw1 = live ? ihi_of(kwlast) / 32 + 1 : t1;
    const int ml = (ilo_of(kwlast) + 31) / 32;       // query tiles in [ml, mu) need no mask
    const int mu = (ihi_of(kw) + 1) / 32;
    const int krow = min(kw + n, Sk - 1);
    const int qlo = ilo_of(krow), qhi = ihi_of(krow);  // this lane's key is seen by qlo .. qhi
    if (nsteps <= 0) {
        // no query sees a key of this block (keys past the queries' causal
        // reach, or a window, with fewer queries than keys): dK = dV = 0
        f32x16 zero[DB];
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int r = 0; r < 16; ++r) zero[db][r] = 0.f;
        if (grp == 0 && live && kw + n < Sk) {
            store_t<T, D, DB>(dK + kvhead, kw + n, h, zero, 1.0f);
            store_t<T, D, DB>(dV + kvhead, kw + n, h, zero, 1.0f);
        }
        return;
    }
    // group grp takes steps ub .. ub + nmine - 1 (nmine may be 0 for the
    // last group); every group runs nsh steps, the extra ones as padding
    const int nsh = (nsteps + QS - 1) / QS;
    const int ub = grp * nsh;
    const int nmine = min(nsh, nsteps - ub);
    // the step whose tiles a group stages at its local step u: clamped to
    // the group's last real step (or, for a group without steps, to the step
    // before its range), so every staging reads a valid tile
    auto ug = [&](int u) { return ub + min(u, nmine - 1); };

    // step u: query head kvbh*G + u / nt, query tile t0 + u % nt
    auto stage = [&](auto par, int u) __attribute__((always_inline)) {
        constexpr int P = decltype(par)::value;
        const int64_t qhead = (int64_t)(kvbh * G + u / nt) * Sq * D;
        const int t = t0 + u % nt;
        const __amdgpu_buffer_rsrc_t qrs = head_rsrc<T>(Q + qhead, Sq * RB);
        const __amdgpu_buffer_rsrc_t ors = head_rsrc<T>(dO + qhead, Sq * RB);
        load_tile<T, L, false>(qrb[P], qrs, roff, t * 32, wave, lane);
        load_tile<T, L, true>(qtb[P], qrs, toff, t * 32, wave, lane);
        load_tile<T, L, false>(orb[P], ors, roff, t * 32, wave, lane);
        load_tile<T, L, true>(otb[P], ors, toff, t * 32, wave, lane);
    };
    // A tile's 32 lse and D values go through lanes 0..31 of wave 0: loaded
    // into registers (three rotating pairs) with the tile's staging, two
    // steps ahead, and written to LDS (plain stores: lse times log2 e, and -D)
    // before the barrier that publishes the tile.  Every lane loads, so that
    // no branch or merge needs a loaded value early, through buffer loads
    // (which the compiler keeps in issue order with the staging); rows past S
    // read as 0 and occur only in tiles outside [ml, mu), where the mask sets
    // their P to 0.
    float lreg[3], dreg[3];
    const bool ld_lane = wave == 0 && lane < 32;
    auto fetch_ld = [&](auto par, int u) __attribute__((always_inline)) {
        constexpr int P = decltype(par)::value;
        const int64_t qrow0 = (int64_t)(kvbh * G + u / nt) * Sq;
        const __amdgpu_buffer_rsrc_t lrs = __builtin_amdgcn_make_buffer_rsrc((void*)(LSE + qrow0), 0, Sq * 4, kBufferFlags);
        const __amdgpu_buffer_rsrc_t drs = __builtin_amdgcn_make_buffer_rsrc((void*)(DELTA + qrow0), 0, Sq * 4, kBufferFlags);
        const int row = (t0 + u % nt) * 32 + n;
        lreg[P] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(lrs, row * 4, 0, 0));
        dreg[P] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(drs, row * 4, 0, 0));
    };
    using P0 = std::integral_constant<int, 0>;
    using P1 = std::integral_constant<int, 1>;
    using P2 = std::integral_constant<int, 2>;
    // This wave's vector-memory operations per step: the lse and D loads, and
    // the tile transfers (spread over the first LOADS waves).  Every step
    // issues them (steps past the last repeat the last tile into a buffer that
    // is not read again, and the step count is padded to the unroll of 3), so
    // the loop body is straight-line in its loads and one wait count holds.
    constexpr int kStepOps = 2 + 4 * L::LOADS_PER_WAVE;
    const bool stages = L::LOADS >= L::NW || wave < L::LOADS;  // wave-uniform

    // resident: K and V fragments of the wave's 32 keys, loaded together with
    // the first two steps' loads; the prologue ends with all of them complete
    // (the loop's wait counts then hold from its first step)
    u32x4 kf[KS], vf[KS];
    row_frags<KS>(K + kvhead, krow, D, h, kf);
    row_frags<KS>(V + kvhead, krow, D, h, vf);
    fetch_ld(P0{}, ug(0));
    stage(P0{}, ug(0));
    fetch_ld(P1{}, ug(1));
    stage(P1{}, ug(1));
    // (the asm operands make the compiler complete these loads here rather
    // than sink them into the loop, where their waits would land in every
    // iteration)
    asm volatile("" : "+v"(lreg[0]), "+v"(dreg[0]), "+v"(lreg[1]), "+v"(dreg[1]));
    wait_vmcnt0();
    pin_frags<KS>(kf);
    pin_frags<KS>(vf);

    int offk[KS], offv[DB];
    frag_offsets<L>(lane, offk, offv);

    f32x16 dkacc[DB], dvacc[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            dkacc[db][r] = 0.f;
            dvacc[db][r] = 0.f;
        }

    // step u, buffers u % 3: tile u and its lse and D were loaded two steps
    // earlier; the loads issued last step may still be in flight
    auto step = [&](auto par, int u) __attribute__((always_inline)) {
        constexpr int P = decltype(par)::value;
        if (stages)
            wait_vmcnt<kStepOps>();
        else
            wait_vmcnt<2>();
        if (ld_lane) {
            lsb[P][lane] = lreg[P] * kLog2e;
            dlb[P][lane] = -dreg[P];
        }
        lds_barrier();
        fetch_ld(std::integral_constant<int, (P + 2) % 3>{}, ug(u + 2));
        stage(std::integral_constant<int, (P + 2) % 3>{}, ug(u + 2));
        if (u >= nmine) return;  // padding step
        const int t = t0 + (ub + u) % nt;
        if (t < tw0 || t >= tw1) return;  // wave-uniform
        // query of register r: 32t + 8(r/4) + 4h + r%4; lse and -D for the
        // four consecutive queries of each register group come in one 16-byte
        // read.  dP starts from -D, so its accumulator ends as dP - D.
        float lse[16];
        f32x16 ndd;
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            // (read as a float vector: a bit_cast of a vector-element lvalue
            // yields element 0 with this compiler)
            const f32x4 a = *reinterpret_cast<const FA_LDS f32x4*>(lsb[P] + 8 * g + 4 * h);
            const f32x4 b = *reinterpret_cast<const FA_LDS f32x4*>(dlb[P] + 8 * g + 4 * h);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                lse[4 * g + e] = a[e];
                ndd[4 * g + e] = b[e];
            }
        }
        const f32x16 zero = {};
        f32x16 s = zero, dp = ndd;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            s = mfma32x32x16<T>(W::k_frag(qrb[P], offk, 0, ks), kf[ks], ks == 0 ? zero : s);
            dp = mfma32x32x16<T>(W::k_frag(orb[P], offk, 0, ks), vf[ks], dp);
        }
        // P = exp2(S c - lse log2 e) and dS = P o (dP - D), packed for the
        // MFMAs.  Queries outside qlo .. qhi (which ends before S) do not see
        // this lane's key; only tiles outside [ml, mu) have any, so the mask
        // is compiled into a second copy taken by a wave-uniform branch.
        u32x4 pp[2], dsp[2];
        auto probs = [&](auto masked) __attribute__((always_inline)) {
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                float pv[2], dv[2];
#pragma unroll
                for (int e = 0; e < 2; ++e) {
                    const int r = 2 * i + e;
                    float p = exp2_fast(__builtin_fmaf(s[r], c, -lse[r]));
                    if constexpr (decltype(masked)::value) {
                        const int q = t * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
                        p = ((q < qlo) | (q > qhi)) ? 0.f : p;
                    }
                    pv[e] = p;
                    dv[e] = p * dp[r];
                }
                pp[i >> 2][i & 3] = pack2<T>(pv[0], pv[1]);
                dsp[i >> 2][i & 3] = pack2<T>(dv[0], dv[1]);
            }
        };
        if (t < ml || t >= mu)
            probs(std::true_type{});
        else
            probs(std::false_type{});
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int db = 0; db < DB; ++db) {
                dvacc[db] = mfma32x32x16<T>(W::v_frag(otb[P], offv, 0, j, db), pp[j], dvacc[db]);
                dkacc[db] = mfma32x32x16<T>(W::v_frag(qtb[P], offv, 0, j, db), dsp[j], dkacc[db]);
            }
    };
    for (int u = 0; u < nsh; u += 3) {
        step(P0{}, u);
        step(P1{}, u + 1);
        step(P2{}, u + 2);
    }
    wait_vmcnt0();  // the spare stagings of the last steps

    if constexpr (QS == 2) {
        // group 1 hands its fp32 partial sums to group 0 through LDS (two of
        // the staging arrays per wave, free once every wave is past the loop)
        static_assert(Cfg::NW == 4 && DB * 16 * 64 * 4 <= QS * Cfg::TILE, "exchange fits the staging arrays");
        __syncthreads();
        float* const xk = (float*)(wave == 0 ? qr0 : wave == 1 ? qr1 : wave == 2 ? qr2 : qt0);
        float* const xv = (float*)(wave == 0 ? qt1 : wave == 1 ? qt2 : wave == 2 ? or0 : or1);
        if (grp == 1) {
#pragma unroll
            for (int db = 0; db < DB; ++db)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    xk[(db * 16 + r) * 64 + lane] = dkacc[db][r];
                    xv[(db * 16 + r) * 64 + lane] = dvacc[db][r];
                }
        }
        __syncthreads();
        if (grp == 1) return;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                dkacc[db][r] += xk[(db * 16 + r) * 64 + lane];
                dvacc[db][r] += xv[(db * 16 + r) * 64 + lane];
            }
    }

    if (live && kw + n < Sk) {
        store_t<T, D, DB>(dK + kvhead, kw + n, h, dkacc, scale);
        store_t<T, D, DB>(dV + kvhead, kw + n, h, dvacc, 1.0f);
    }
}

}  // namespace fa
