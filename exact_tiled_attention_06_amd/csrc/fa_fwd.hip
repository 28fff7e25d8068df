// fa_fwd.hip -- the C ABI of the attention forward library: argument checks,
// kernel-instance selection and the launch on the caller's stream.
//
// Host-side plan ("T5 讲解：FlashAttention forward", sections ② and ⑥;
// "Triton 实现", section "Grid 与并行策略"): one workgroup per
// (query block, batch*head), i.e. ceil(S_q/BM) * B*H independent workgroups
// with no communication between them; the default scale 1/sqrt(D) is the
// caller's business (the Python binding supplies it).
#include <stdint.h>
#include <string.h>

#include <mutex>

#include <hip/hip_runtime.h>

#include "../../include/fa.h"
#include "fa_f32m.hpp"
#include "fa_mfma.hpp"
#include "fa_ksplit.hpp"
#include "fa_split.hpp"
#include "fa_bwd.hpp"
#include "fa_window.hpp"
#include "fa_split_window.hpp"

#ifndef FA_SPLIT_TBN
#define FA_SPLIT_TBN 128
#endif

namespace {

using namespace fa;

// Matrix-core kernel shapes per head dimension, chosen by measurement on the
// B=4 H=16 S=4096 workloads: {32-query blocks per wave, waves per workgroup,
// keys per compute step, software-pipelined, keys per LDS tile}.  Two query
// blocks per wave halve the LDS operand reads per MFMA; D = 128 keeps one
// (its accumulators fill the register budget) and uses eight waves.
template <int D>
struct Tiles {
    static constexpr int QB = (D == 16 || D == 128) ? 1 : 2;
    static constexpr int NW = (D == 128) ? 8 : 4;
    // D = 128 runs the pipelined loop on 32-key steps (exactly 256 VGPRs):
    // measured 5-6 % faster than the plain loop on 64-key steps
    static constexpr int BN = (D == 16) ? 64 : 32;
    static constexpr bool PIPE = true;
    // keys per LDS tile (one barrier each): the two-column-block kernel stages
    // 128 keys at D = 32 and 64 at D = 64 (B=4 H=16 S=4096: 1 % faster than
    // one 32-key tile per barrier, 128 keys gain less); the pipelined loop
    // stages one compute step per LDS tile
    static constexpr int TBN = D == 32 ? FA_SPLIT_TBN : D == 64 ? 64 : BN;
    // smaller grids: 64 query rows per workgroup, 128 at D = 128 (four waves:
    // their transfer offsets repeat per wave, so the pipelined loop fits in
    // 256 VGPRs; with two waves it spilled)
    static constexpr int SMALL_QB = 1;
    static constexpr int SMALL_NW = (D == 128) ? 4 : 2;
    static constexpr int SMALL_BN = (D == 16) ? 64 : 32;
    static constexpr bool SMALL_PIPE = true;
};

// A grid of at least this many workgroups fills the machine twice over.
constexpr int64_t kFullGrid = 512;
// compute units of the GPU (one workgroup each)
constexpr int64_t kCUs = 256;

int64_t elem_size(int dtype) { return dtype == FA_DTYPE_F32 ? 4 : 2; }

bool overlaps(const void* a, int64_t na, const void* b, int64_t nb) {
    const uintptr_t a0 = (uintptr_t)a, b0 = (uintptr_t)b;
    return a0 < b0 + (uintptr_t)nb && b0 < a0 + (uintptr_t)na;
}

// One forward call's device arguments and launch parameters.
struct Fwd {
    const void *q, *k, *v;
    void* o;
    float* lse;
    int Sq, Sk, BH, G;  // queries, keys per head; G query heads per K/V head
    int wl, wr;         // window (left, right); -1: no limit on that side
    float c;            // scale * log2(e)
    hipStream_t stream;
    bool single;        // race check: the single-buffered two-block kernel
    void* ws;           // caller's workspace for the key split of the longest blocks (or NULL)
    int64_t ws_bytes;
};

// Fills n 32-bit words with `value` (outputs of problems without keys or
// without queries).
__global__ void fa_fill_kernel(uint32_t* __restrict__ p, uint32_t value, int64_t n) {
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
        p[i] = value;
}

int fill_words(void* p, uint32_t value, int64_t bytes, hipStream_t stream) {
    const int64_t n = bytes / 4;
    if (n == 0) return FA_OK;
    const int64_t blocks = (n + 255) / 256;
    (void)hipGetLastError();
    hipLaunchKernelGGL(fa_fill_kernel, dim3((unsigned)(blocks < 4096 ? blocks : 4096)), dim3(256), 0, stream,
                       (uint32_t*)p, value, n);
    return hipGetLastError() == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

// Rows per workgroup of the kernel a causal problem without a window runs on,
// where that kernel can split its longest blocks' keys (0 elsewhere): the
// two-block kernel at D = 32, 64 (256 rows, from kFullGrid workgroups), the
// one-block kernel at D = 16 (128 rows, same rule) and at D = 128 between the
// key-split kernel and the large tile (128 rows).  Mirrors launch_mfma.
int64_t split_rows(int64_t D, int64_t S, int64_t BH) {
    auto grid = [&](int64_t bm) { return (S + bm - 1) / bm * BH; };
    if (D == 32 || D == 64) return grid(256) >= kFullGrid ? 256 : 0;
    if (D == 16) return grid(128) >= kFullGrid ? 128 : 0;
    return (grid(256) < kFullGrid && grid(64) >= kFullGrid) ? 128 : 0;
}

// Largest grid (workgroups of split_rows rows) whose longest blocks are split:
// where the whole grid is resident at once.  At D = 128 only a grid of one
// workgroup per compute unit: at two per unit (B=8 H=1 S=8192) the split
// measured no gain (156.0 against 156.8 us).
int64_t split_max_grid(int64_t D) { return D == 128 ? kCUs : 2 * kCUs; }

// Workspace for the key split of the longest blocks (nsplit > 0 in the
// two-block and one-block kernels), 0 when the problem does not use it.  The
// split pays where a kernel's whole grid is resident at once (at most
// split_max_grid workgroups): there no later workgroup balances the load, and
// the longest blocks' serial chains of tiles set the time.  The n_qblk / 2 longest blocks of every head then run as two key
// halves each, with an fp32 partial of BM rows x (D + 1) values per half, and
// the work items start longest first.  Causal, no window, S_q = S_k (every
// row of a split block then sees keys in both halves).
int64_t split_workspace_bytes(int64_t D, bool causal, int wl, int wr, int64_t Sq, int64_t Sk, int64_t BH) {
    if (!causal || wl >= 0 || wr >= 0 || Sq != Sk) return 0;
    const int64_t bm = split_rows(D, Sq, BH);
    if (bm == 0) return 0;
    const int64_t n_qblk = (Sq + bm - 1) / bm;
    if (n_qblk * BH > split_max_grid(D) || n_qblk < 2) return 0;
    return (n_qblk / 2) * BH * 2 * bm * (D + 1) * 4;
}

// The `round` argument of the two-block and key-split kernels.  When two of
// their 4-wave workgroups fit on a compute unit (two waves per SIMD, and LDS
// for two), a causal grid of more than one and at most two rounds of kCUs
// workgroups is resident all at once, workgroup i + kCUs on the unit of
// workgroup i, and pairs its rounds long with short.  Otherwise (0) the order
// stays longest first: the hardware then starts each later workgroup on the
// first unit to free up, which balances by itself.  Measured on B=8 H=1,
// causal: the key-split kernel gains at D = 32 and 64 (S=4096 D=64 32.0 ->
// 27.8 us) and the two-block kernel at D = 32 (S=16384 244.5 -> 215.8 us), but
// the two-block kernel at D = 64 loses (S=16384 314.0 -> 335.2 us): there the
// time is the longest block's own chain of tiles, which runs faster beside a
// second, lower-priority wave on its SIMDs than alone (1286 against 1340
// cycles per tile in per-wave timestamps), so it keeps longest first.
template <typename Cfg, int LDS_BYTES, bool SPLIT>
int two_round_order(int64_t grid) {
    constexpr bool two_per_cu = Cfg::NW == 4 && Cfg::OCC == 2 && Cfg::D <= 64 && 2 * LDS_BYTES <= 160 * 1024;
    constexpr bool gains = !SPLIT || Cfg::D <= 32;
    return (two_per_cu && gains && Cfg::CAUSAL && grid > kCUs && grid <= 2 * kCUs) ? (int)kCUs : 0;
}

template <typename T, typename Cfg, bool SINGLE = false>
int launch_cfg(const Fwd& a) {
    const int n_qblk = (a.Sq + Cfg::BM - 1) / Cfg::BM;
    const int64_t grid = (int64_t)n_qblk * a.BH;
    if (grid > (int64_t)1 << 24) return FA_ERR_TOO_LARGE;
    // the key split of the longest blocks, when the caller's workspace holds it
    int nsplit = 0;
    float *po = nullptr, *pl = nullptr;
    if constexpr (!SINGLE && Cfg::CAUSAL) {
        const int64_t need = split_workspace_bytes(Cfg::D, true, a.wl, a.wr, a.Sq, a.Sk, a.BH);
        if (need > 0 && a.ws && a.ws_bytes >= need && split_rows(Cfg::D, a.Sq, a.BH) == Cfg::BM) {
            nsplit = n_qblk / 2;
            po = (float*)a.ws;
            pl = po + (int64_t)nsplit * a.BH * 2 * Cfg::BM * Cfg::D;
        }
    }
    const int64_t g = grid + (int64_t)nsplit * a.BH;  // each split block: two workgroups
    (void)hipGetLastError();  // clear a stale error so the check below sees this launch only
    // (the split runs its own kernel instances, so that the plain ones carry
    // none of its code)
    auto launch = [&](auto ksplit) {
        constexpr bool KS = decltype(ksplit)::value && !SINGLE && Cfg::CAUSAL;
        if constexpr (Cfg::QB == 2 && Cfg::KB == 1 && Cfg::PIPE)
            hipLaunchKernelGGL((fa_fwd_split_kernel<T, Cfg, SINGLE, KS>), dim3((unsigned)g), dim3(Cfg::NT), 0,
                               a.stream, (const uint16_t*)a.q, (const uint16_t*)a.k, (const uint16_t*)a.v,
                               (uint16_t*)a.o, a.lse, a.Sq, a.Sk, a.BH, n_qblk, a.G, a.c,
                               KS ? 0 : two_round_order<Cfg, 4 * Cfg::TILE, true>(grid), po, pl, nsplit);
        else
            hipLaunchKernelGGL((fa_fwd_mfma_kernel<T, Cfg, KS>), dim3((unsigned)g), dim3(Cfg::NT), 0, a.stream,
                               (const uint16_t*)a.q, (const uint16_t*)a.k, (const uint16_t*)a.v, (uint16_t*)a.o,
                               a.lse, a.Sq, a.Sk, a.BH, n_qblk, a.G, a.c, po, pl, nsplit);
    };
    if (nsplit) launch(std::true_type{});
    else launch(std::false_type{});
    if (nsplit) {
        if (hipGetLastError() != hipSuccess) return FA_ERR_LAUNCH;
        const int64_t threads = (int64_t)nsplit * a.BH * Cfg::BM * (Cfg::D / 4);
        hipLaunchKernelGGL((fa_fwd_merge_kernel<T, Cfg::D, Cfg::BM>), dim3((unsigned)((threads + 255) / 256)),
                           dim3(256), 0, a.stream, (const float*)po, (const float*)pl, (uint16_t*)a.o, a.lse, a.Sq,
                           a.BH, n_qblk, nsplit);
    }
    return hipGetLastError() == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

// Thin grids: workgroups of NW waves that share BMW query rows and split the keys.
template <typename T, typename Cfg>
int launch_ksplit(const Fwd& a) {
    const int n_qblk = (a.Sq + Cfg::BMW - 1) / Cfg::BMW;
    const int64_t grid = (int64_t)n_qblk * a.BH;
    if (grid > (int64_t)1 << 24) return FA_ERR_TOO_LARGE;
    (void)hipGetLastError();
    hipLaunchKernelGGL((fa_fwd_ksplit_kernel<T, Cfg>), dim3((unsigned)grid), dim3(Cfg::NT), 0, a.stream,
                       (const uint16_t*)a.q, (const uint16_t*)a.k, (const uint16_t*)a.v, (uint16_t*)a.o, a.lse,
                       a.Sq, a.Sk, a.BH, n_qblk, a.G, a.c, two_round_order<Cfg, ksplit_lds_bytes<Cfg>(), false>(grid));
    return hipGetLastError() == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

// Sliding windows: at D = 32 and 64 the two-block kernel (4 waves of 2 x 32
// query rows), else the plain loop (4 waves of 32 rows); one 32-key tile per
// barrier either way.
template <typename T, int D, bool CAUSAL>
int launch_window(const Fwd& a) {
    using Cfg = std::conditional_t<(D == 32 || D == 64), MfmaConfig<D, CAUSAL, 2, 4, 32, true, 2, 32>,
                                   MfmaConfig<D, CAUSAL, 1, 4, 32, false, 2, 32>>;
    const int n_qblk = (a.Sq + Cfg::BM - 1) / Cfg::BM;
    const int64_t grid = (int64_t)n_qblk * a.BH;
    if (grid > (int64_t)1 << 24) return FA_ERR_TOO_LARGE;
    (void)hipGetLastError();
    if constexpr (D == 32 || D == 64)
        hipLaunchKernelGGL((fa_fwd_split_window_kernel<T, Cfg>), dim3((unsigned)grid), dim3(Cfg::NT), 0, a.stream,
                           (const uint16_t*)a.q, (const uint16_t*)a.k, (const uint16_t*)a.v, (uint16_t*)a.o, a.lse,
                           a.Sq, a.Sk, a.BH, n_qblk, a.G, a.wl, a.wr, a.c);
    else
        hipLaunchKernelGGL((fa_fwd_window_kernel<T, Cfg>), dim3((unsigned)grid), dim3(Cfg::NT), 0, a.stream,
                           (const uint16_t*)a.q, (const uint16_t*)a.k, (const uint16_t*)a.v, (uint16_t*)a.o, a.lse,
                           a.Sq, a.Sk, a.BH, n_qblk, a.G, a.wl, a.wr, a.c);
    return hipGetLastError() == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

template <typename T, int D, bool CAUSAL>
int launch_mfma(const Fwd& a) {
    if (a.single && (a.wl >= 0 || a.wr >= 0)) return FA_ERR_UNSUPPORTED;
    if (a.wl >= 0 || a.wr >= 0) return launch_window<T, D, CAUSAL>(a);
    using TL = Tiles<D>;
    using Large = MfmaConfig<D, CAUSAL, TL::QB, TL::NW, TL::BN, TL::PIPE, 2, TL::TBN>;
    using Small = MfmaConfig<D, CAUSAL, TL::SMALL_QB, TL::SMALL_NW, TL::SMALL_BN, TL::SMALL_PIPE>;
    const int64_t large_grid = (int64_t)((a.Sq + Large::BM - 1) / Large::BM) * a.BH;
    if (a.single) {
        // the race check exists for the double-buffered two-block kernel only
        if constexpr (D == 32 || D == 64) {
            if (large_grid >= kFullGrid) return launch_cfg<T, Large, true>(a);
        }
        return FA_ERR_UNSUPPORTED;
    }
    if (large_grid >= kFullGrid) return launch_cfg<T, Large>(a);
    // Thinner grids split each query block's keys over the 4 waves of its
    // workgroup.  Measured on the B=8 H=1 sweep: at D <= 64 blocks of 64 rows
    // (two per wave) unless even those give fewer than 256 workgroups, then
    // 32; at D = 128 blocks of 32 rows while 64-row blocks would give fewer
    // than kFullGrid workgroups (S <= 1024), else the pipelined one-block
    // kernel on 128-row workgroups (S=4096: 73.2 against 62.8 us).
    const int64_t grid64 = (int64_t)((a.Sq + 63) / 64) * a.BH;
    if constexpr (D <= 64) {
        if (grid64 < kFullGrid / 2) return launch_ksplit<T, MfmaConfig<D, CAUSAL, 1, 4, 32>>(a);
        return launch_ksplit<T, MfmaConfig<D, CAUSAL, 2, 4, 32>>(a);
    } else {
        if (grid64 < kFullGrid) return launch_ksplit<T, MfmaConfig<D, CAUSAL, 1, 4, 32>>(a);
        return launch_cfg<T, Small>(a);
    }
}

// fp32: workgroups of 32 query rows on the fp32 matrix cores
template <int D, bool CAUSAL>
int launch_f32(const Fwd& a) {
    const int n_qblk = (a.Sq + 31) / 32;
    const int64_t grid = (int64_t)n_qblk * a.BH;
    if (grid > (int64_t)1 << 24) return FA_ERR_TOO_LARGE;
    (void)hipGetLastError();
    hipLaunchKernelGGL((fa_fwd_f32m_kernel<D, CAUSAL>), dim3((unsigned)grid), dim3(F32mCfg<D>::NT), 0, a.stream,
                       (const float*)a.q, (const float*)a.k, (const float*)a.v, (float*)a.o, a.lse, a.Sq, a.Sk,
                       a.BH, n_qblk, a.G, a.wl, a.wr, a.c);
    return hipGetLastError() == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

template <int D, bool CAUSAL>
int dispatch_dtype(int dtype, const Fwd& a) {
    switch (dtype) {
        case FA_DTYPE_F16: return launch_mfma<F16, D, CAUSAL>(a);
        case FA_DTYPE_BF16: return launch_mfma<BF16, D, CAUSAL>(a);
        default: return a.single ? FA_ERR_UNSUPPORTED : launch_f32<D, CAUSAL>(a);
    }
}

template <bool CAUSAL>
int dispatch_d(int64_t D, int dtype, const Fwd& a) {
    switch (D) {
        case 16: return dispatch_dtype<16, CAUSAL>(dtype, a);
        case 32: return dispatch_dtype<32, CAUSAL>(dtype, a);
        case 64: return dispatch_dtype<64, CAUSAL>(dtype, a);
        default: return dispatch_dtype<128, CAUSAL>(dtype, a);
    }
}

// ------------------------------------------------------------------ backward

// One backward call's device arguments and launch parameters.
struct Bwd {
    const void *q, *k, *v, *o, *dout;
    const float* lse;
    void *dq, *dk, *dv;
    float* delta;
    int Sq, Sk, BH, G, wl, wr;
    float c, scale;
    hipStream_t stream;
};

// dQ (and D = rowsum(dO o O) into `delta`), then dK and dV, which read D
template <typename T, typename Cfg>
int launch_dq(const Bwd& a) {
    const int n_qblk = (a.Sq + Cfg::BMQ - 1) / Cfg::BMQ;  // query blocks
    if ((int64_t)n_qblk * a.BH > (int64_t)1 << 24) return FA_ERR_TOO_LARGE;
    (void)hipGetLastError();
    hipLaunchKernelGGL((fa_bwd_dq_kernel<T, Cfg>), dim3((unsigned)((int64_t)n_qblk * a.BH)), dim3(Cfg::NT_Q), 0,
                       a.stream, (const uint16_t*)a.q, (const uint16_t*)a.k, (const uint16_t*)a.v,
                       (const uint16_t*)a.o, (const uint16_t*)a.dout, a.lse, (uint16_t*)a.dq, a.delta, a.Sq, a.Sk,
                       a.BH, n_qblk, a.G, a.wl, a.wr, a.c, a.scale);
    return hipGetLastError() == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

template <typename T, typename Cfg>
int launch_dkdv(const Bwd& a) {
    const int n_blk = (a.Sk + Cfg::BM - 1) / Cfg::BM;  // key blocks
    const int BHkv = a.BH / a.G;
    if ((int64_t)n_blk * BHkv > (int64_t)1 << 24) return FA_ERR_TOO_LARGE;
    (void)hipGetLastError();
    hipLaunchKernelGGL((fa_bwd_dkdv_kernel<T, Cfg>), dim3((unsigned)((int64_t)n_blk * BHkv)), dim3(Cfg::NT_KV), 0,
                       a.stream, (const uint16_t*)a.q, (const uint16_t*)a.k, (const uint16_t*)a.v,
                       (const uint16_t*)a.dout, a.lse, (const float*)a.delta, (uint16_t*)a.dk, (uint16_t*)a.dv, a.Sq,
                       a.Sk, BHkv, n_blk, a.G, a.wl, a.wr, a.c, a.scale);
    return hipGetLastError() == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

template <typename T, int D, bool CAUSAL>
int launch_bwd(const Bwd& a) {
    // dQ kernel: two 32-query blocks per wave (D <= 64), unless that leaves
    // fewer workgroups than CUs; then one block per wave, twice the waves
    // (D = 128 has one block per wave anyway), and if that still leaves
    // fewer than two workgroups per CU, two groups of waves per query block
    // that split its key tiles (D >= 32): groups of 2 waves (64 rows, 4-wave
    // workgroups, 48 KB of LDS at D = 64) at D = 32, 64, where fewer waves
    // behind each barrier wait less; of 4 at D = 128, whose 96 KB of LDS
    // admit one workgroup per CU
    using Q2 = BwdConfig<D, CAUSAL, 4>;
    using Q1 = BwdConfig<D, CAUSAL, 4, 1>;
    using Q1K = BwdConfig<D, CAUSAL, (D == 32 || D == 64) ? 2 : 4, 1, 1, D >= 32 ? 2 : 1>;
    const int64_t grid_q2 = (int64_t)((a.Sq + Q2::BMQ - 1) / Q2::BMQ) * a.BH;
    const int64_t grid_q1 = (int64_t)((a.Sq + Q1::BMQ - 1) / Q1::BMQ) * a.BH;
    const int r = (D <= 64 && grid_q2 >= kCUs) ? launch_dq<T, Q2>(a)
                  : grid_q1 >= kFullGrid       ? launch_dq<T, Q1>(a)
                                               : launch_dq<T, Q1K>(a);
    if (r != FA_OK) return r;
    // dK/dV kernel: a wave owns 32 keys whatever the workgroup, so a grid of
    // fewer than two workgroups per CU splits each key block's query steps
    // over two groups of 4 waves (D = 32, 64)
    using KV = BwdConfig<D, CAUSAL, 4>;
    using KV2 = BwdConfig<D, CAUSAL, 4, Q2::QBQ, (D == 32 || D == 64) ? 2 : 1>;
    const int64_t grid_kv = (int64_t)((a.Sk + KV::BM - 1) / KV::BM) * (a.BH / a.G);
    return grid_kv >= kFullGrid ? launch_dkdv<T, KV>(a) : launch_dkdv<T, KV2>(a);
}

template <bool CAUSAL>
int dispatch_bwd(int64_t D, int dtype, const Bwd& a) {
#define FA_BWD_CASE(DD)                                                                          \
    case DD:                                                                                     \
        return dtype == FA_DTYPE_F16 ? launch_bwd<F16, DD, CAUSAL>(a) : launch_bwd<BF16, DD, CAUSAL>(a);
    switch (D) {
        FA_BWD_CASE(16)
        FA_BWD_CASE(32)
        FA_BWD_CASE(64)
        default: FA_BWD_CASE(128)
    }
#undef FA_BWD_CASE
}

// Checks shared by the entry points (no HIP call): shapes, head dim, grouped
// heads (H a multiple of H_kv), causal flag, window bounds, scale.
int check_problem(int64_t B, int64_t H, int64_t H_kv, int64_t Sq, int64_t Sk, int64_t D, int causal, int64_t wl,
                  int64_t wr, float scale) {
    if (B < 0 || H < 0 || Sq < 0 || Sk < 0 || H_kv < 0 || (H_kv == 0 ? H != 0 : H % H_kv != 0))
        return FA_ERR_SHAPE;
    if (D != 16 && D != 32 && D != 64 && D != 128) return FA_ERR_HEAD_DIM;
    if (causal != 0 && causal != 1) return FA_ERR_CAUSAL;
    if (wl < -1 || wr < -1) return FA_ERR_WINDOW;
    // finite and > 0, tested on the bits (the library is built without NaN semantics)
    uint32_t sbits;
    memcpy(&sbits, &scale, sizeof sbits);
    if (((sbits >> 23) & 0xFFu) == 0xFFu || (sbits >> 31) != 0u || (sbits & 0x7FFFFFFFu) == 0u)
        return FA_ERR_SCALE;
    return FA_OK;
}

// Index ranges shared by the entry points (S: the longer of the query and key
// lengths, > 0); H_kv > 0 here.
int check_sizes(int64_t B, int64_t H, int64_t S, int64_t D) {
    const int64_t kMaxInt = 2147483647;
    if (B > kMaxInt || H > kMaxInt || B * H > kMaxInt / 2 || S > (kMaxInt >> 1)) return FA_ERR_TOO_LARGE;
    const int64_t BH = B * H;
    if (BH > INT64_MAX / S || BH * S > INT64_MAX / (D * 8)) return FA_ERR_TOO_LARGE;
    return FA_OK;
}

// The window's limits clipped to the sequences: a side that reaches past both
// the queries and the keys (S = max(S_q, S_k)) is the same as no limit.
int clip_window(int64_t w, int64_t S) { return (w < 0 || w >= S) ? -1 : (int)w; }

}  // namespace

// ------------------------------------------------ backward: the entry points

namespace {

// The D = rowsum(dO o O) workspace of fa_bwd_noalloc: a static device array, one
// copy per GPU, held until the process ends.  Host code never passes the
// array's name to a kernel (on the host it only stands in for the symbol): each
// device's address comes from hipGetSymbolAddress, taken once per device with
// that device current, and only that address is used.
constexpr int64_t kScratchFloats = (int64_t)1 << 22;  // 16 MiB: B * H * S_q <= 4,194,304
__device__ __align__(256) float scratch[kScratchFloats];

constexpr int kMaxDevices = 64;
std::mutex scratch_mutex;
float* scratch_ptr[kMaxDevices] = {};

// The workspace address on the device that runs `stream` (NULL: the current
// device), looked up on the first call for that device.
int scratch_for(hipStream_t stream, float** out) {
    int cur = -1, dev = -1;
    if (hipGetDevice(&cur) != hipSuccess) return FA_ERR_LAUNCH;
    if (stream) {
        hipDevice_t d;
        if (hipStreamGetDevice(stream, &d) != hipSuccess) return FA_ERR_LAUNCH;
        dev = (int)d;
    } else {
        dev = cur;
    }
    if (dev < 0 || dev >= kMaxDevices) return FA_ERR_LAUNCH;
    std::lock_guard<std::mutex> lock(scratch_mutex);
    if (!scratch_ptr[dev]) {
        if (dev != cur && hipSetDevice(dev) != hipSuccess) return FA_ERR_LAUNCH;
        void* p = nullptr;
        const hipError_t rc = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (dev != cur && hipSetDevice(cur) != hipSuccess) return FA_ERR_LAUNCH;
        if (rc != hipSuccess || !p) return FA_ERR_LAUNCH;
        scratch_ptr[dev] = (float*)p;
    }
    *out = scratch_ptr[dev];
    return FA_OK;
}

// fa_bwd_ex's work; with `static_delta` the D workspace is the library's own
// static array (`delta` is ignored) instead of the caller's buffer.
int bwd_entry(const void* q, const void* k, const void* v, const void* o, const void* dout, const float* lse,
              void* dq, void* dk, void* dv, float* delta, bool static_delta, int64_t B, int64_t H, int64_t H_kv,
              int64_t S_q, int64_t S_k, int64_t D, int causal, int64_t window_left, int64_t window_right,
              float scale, int dtype, void* stream) {
    // ---- argument checks: no HIP call before all of them pass ----------------
    int rc = check_problem(B, H, H_kv, S_q, S_k, D, causal, window_left, window_right, scale);
    if (rc == FA_ERR_SHAPE || rc == FA_ERR_HEAD_DIM) return rc;
    if (dtype != FA_DTYPE_F16 && dtype != FA_DTYPE_BF16) return FA_ERR_DTYPE;
    if (rc != FA_OK) return rc;
    if (B == 0 || H == 0 || (S_q == 0 && S_k == 0)) return FA_OK;
    if (S_q > 0 && (!q || !o || !dout || !lse || !dq || (!static_delta && !delta))) return FA_ERR_NULL_POINTER;
    if (S_k > 0 && (!k || !v || !dk || !dv)) return FA_ERR_NULL_POINTER;
    const int64_t S = S_q > S_k ? S_q : S_k;
    if ((rc = check_sizes(B, H, S, D)) != FA_OK) return rc;
    if (S * D * 2 > 2147483647) return FA_ERR_TOO_LARGE;
    const int64_t BH = B * H;
    if (static_delta && BH * S_q > kScratchFloats) return FA_ERR_WORKSPACE;
    const int64_t tb = BH * S_q * D * 2, kvb = B * H_kv * S_k * D * 2, vb = BH * S_q * 4;
    if (((uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)o | (uintptr_t)dout | (uintptr_t)dq |
         (uintptr_t)dk | (uintptr_t)dv) & 15)
        return FA_ERR_ALIGNMENT;
    if (((uintptr_t)lse | (static_delta ? 0 : (uintptr_t)delta)) & 3) return FA_ERR_ALIGNMENT;
    // every output (dq, dk, dv, delta) apart from every other buffer (the
    // static workspace is an allocation of its own)
    const int nout = static_delta ? 3 : 4;
    const void* outs[4] = {dq, dk, dv, delta};
    const int64_t out_bytes[4] = {tb, kvb, kvb, vb};
    const void* all[10] = {q, k, v, o, dout, lse, dq, dk, dv, delta};
    const int64_t all_bytes[10] = {tb, kvb, kvb, tb, tb, vb, tb, kvb, kvb, vb};
    const int nall = static_delta ? 9 : 10;
    for (int i = 0; i < nout; ++i)
        for (int j = 0; j < nall; ++j)
            if (j != 6 + i && overlaps(outs[i], out_bytes[i], all[j], all_bytes[j])) return FA_ERR_ALIAS;

    // no keys: every dQ is 0 (dK, dV are empty); no queries: dK = dV = 0
    if (S_k == 0) return fill_words(dq, 0u, tb, (hipStream_t)stream);
    if (S_q == 0) {
        if ((rc = fill_words(dk, 0u, kvb, (hipStream_t)stream)) != FA_OK) return rc;
        return fill_words(dv, 0u, kvb, (hipStream_t)stream);
    }
    // the dQ kernel writes D for every query row before the dK/dV kernel reads
    // it, so the workspace needs no clearing
    if (static_delta && (rc = scratch_for((hipStream_t)stream, &delta)) != FA_OK) return rc;
    Bwd a{q, k, v, o, dout, lse, dq, dk, dv, delta, (int)S_q, (int)S_k, (int)BH, (int)(H / H_kv),
          clip_window(window_left, S), clip_window(window_right, S),
          (float)((double)scale * 1.4426950408889634), scale, (hipStream_t)stream};
    return causal ? dispatch_bwd<true>(D, dtype, a) : dispatch_bwd<false>(D, dtype, a);
}

}  // namespace

extern "C" int fa_bwd_ex(const void* q, const void* k, const void* v, const void* o, const void* dout,
                         const float* lse, void* dq, void* dk, void* dv, float* delta, int64_t B, int64_t H,
                         int64_t H_kv, int64_t S_q, int64_t S_k, int64_t D, int causal, int64_t window_left,
                         int64_t window_right, float scale, int dtype, void* stream) {
    return bwd_entry(q, k, v, o, dout, lse, dq, dk, dv, delta, false, B, H, H_kv, S_q, S_k, D, causal, window_left,
                     window_right, scale, dtype, stream);
}

extern "C" int fa_bwd_noalloc(const void* q, const void* k, const void* v, const void* o, const void* dout,
                              const float* lse, void* dq, void* dk, void* dv, int64_t B, int64_t H, int64_t H_kv,
                              int64_t S_q, int64_t S_k, int64_t D, int causal, int64_t window_left,
                              int64_t window_right, float scale, int dtype, void* stream) {
    return bwd_entry(q, k, v, o, dout, lse, dq, dk, dv, nullptr, true, B, H, H_kv, S_q, S_k, D, causal,
                     window_left, window_right, scale, dtype, stream);
}

extern "C" int fa_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout,
                      const float* lse, void* dq, void* dk, void* dv, float* delta, int64_t B, int64_t H,
                      int64_t S, int64_t D, int causal, float scale, int dtype, void* stream) {
    return fa_bwd_ex(q, k, v, o, dout, lse, dq, dk, dv, delta, B, H, H, S, S, D, causal, -1, -1, scale, dtype,
                     stream);
}

namespace {

// fa_fwd_ex's work; `single` selects the single-buffered race-check variant,
// `ws` / `ws_bytes` the caller's workspace of fa_fwd_ws (NULL / 0: none).
int fwd_entry(const void* q, const void* k, const void* v, void* o, float* lse, int64_t B, int64_t H, int64_t H_kv,
              int64_t S_q, int64_t S_k, int64_t D, int causal, int64_t window_left, int64_t window_right,
              float scale, int dtype, void* stream, bool single, void* ws = nullptr, int64_t ws_bytes = 0) {
    // ---- argument checks: no HIP call before all of them pass ----------------
    int rc = check_problem(B, H, H_kv, S_q, S_k, D, causal, window_left, window_right, scale);
    if (rc == FA_ERR_SHAPE || rc == FA_ERR_HEAD_DIM) return rc;
    if (dtype != FA_DTYPE_F32 && dtype != FA_DTYPE_F16 && dtype != FA_DTYPE_BF16) return FA_ERR_DTYPE;
    if (rc != FA_OK) return rc;
    if (B == 0 || H == 0 || S_q == 0) return FA_OK;  // no query row: nothing to write
    if (!q || !o || !lse || (S_k > 0 && (!k || !v))) return FA_ERR_NULL_POINTER;
    const int64_t S = S_q > S_k ? S_q : S_k;
    if ((rc = check_sizes(B, H, S, D)) != FA_OK) return rc;
    // the matrix-core kernels address one head's K or V rows through a buffer
    // resource with a 32-bit extent: S_k * D * 2 bytes must stay below 2^31
    if (dtype != FA_DTYPE_F32 && S * D * 2 > 2147483647) return FA_ERR_TOO_LARGE;
    const int64_t BH = B * H;
    const int64_t tensor_bytes = BH * S_q * D * elem_size(dtype);
    const int64_t kv_bytes = B * H_kv * S_k * D * elem_size(dtype);
    const int64_t lse_bytes = BH * S_q * 4;
    if (((uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)o) & 15) return FA_ERR_ALIGNMENT;
    if (((uintptr_t)lse) & 3) return FA_ERR_ALIGNMENT;
    if (overlaps(o, tensor_bytes, q, tensor_bytes) || overlaps(o, tensor_bytes, k, kv_bytes) ||
        overlaps(o, tensor_bytes, v, kv_bytes) || overlaps(o, tensor_bytes, lse, lse_bytes) ||
        overlaps(lse, lse_bytes, q, tensor_bytes) || overlaps(lse, lse_bytes, k, kv_bytes) ||
        overlaps(lse, lse_bytes, v, kv_bytes))
        return FA_ERR_ALIAS;
    // the workspace, when given, is written: 16-byte aligned, apart from every
    // tensor of the call
    if (ws_bytes < 0) return FA_ERR_WORKSPACE;
    if (!ws) ws_bytes = 0;
    if (ws_bytes > 0) {
        if ((uintptr_t)ws & 15) return FA_ERR_ALIGNMENT;
        if (overlaps(ws, ws_bytes, q, tensor_bytes) || overlaps(ws, ws_bytes, k, kv_bytes) ||
            overlaps(ws, ws_bytes, v, kv_bytes) || overlaps(ws, ws_bytes, o, tensor_bytes) ||
            overlaps(ws, ws_bytes, lse, lse_bytes))
            return FA_ERR_ALIAS;
    }

    // no keys: every row is empty, O = 0 and lse = ln 0 = -inf
    if (S_k == 0) {
        if ((rc = fill_words(o, 0u, tensor_bytes, (hipStream_t)stream)) != FA_OK) return rc;
        return fill_words(lse, 0xFF800000u, lse_bytes, (hipStream_t)stream);
    }
    // c = scale * log2(e), rounded once to fp32: scores enter exp2 as S*c - m.
    Fwd a{q, k, v, o, lse, (int)S_q, (int)S_k, (int)BH, (int)(H / H_kv), clip_window(window_left, S),
          clip_window(window_right, S), (float)((double)scale * 1.4426950408889634), (hipStream_t)stream, single,
          ws, ws_bytes};
    return causal ? dispatch_d<true>(D, dtype, a) : dispatch_d<false>(D, dtype, a);
}

}  // namespace

extern "C" int fa_fwd_ex(const void* q, const void* k, const void* v, void* o, float* lse, int64_t B, int64_t H,
                         int64_t H_kv, int64_t S_q, int64_t S_k, int64_t D, int causal, int64_t window_left,
                         int64_t window_right, float scale, int dtype, void* stream) {
    return fwd_entry(q, k, v, o, lse, B, H, H_kv, S_q, S_k, D, causal, window_left, window_right, scale, dtype,
                     stream, false);
}

extern "C" int64_t fa_fwd_workspace_bytes(int64_t B, int64_t H, int64_t H_kv, int64_t S_q, int64_t S_k, int64_t D,
                                          int causal, int64_t window_left, int64_t window_right, int dtype) {
    if (check_problem(B, H, H_kv, S_q, S_k, D, causal, window_left, window_right, 1.0f) != FA_OK) return 0;
    if (dtype != FA_DTYPE_F16 && dtype != FA_DTYPE_BF16) return 0;
    if (B == 0 || H == 0 || S_q == 0 || S_k == 0) return 0;
    const int64_t S = S_q > S_k ? S_q : S_k;
    if (check_sizes(B, H, S, D) != FA_OK || S * D * 2 > 2147483647) return 0;
    return split_workspace_bytes(D, causal != 0, clip_window(window_left, S), clip_window(window_right, S), S_q, S_k,
                                 B * H);
}

extern "C" int fa_fwd_ws(const void* q, const void* k, const void* v, void* o, float* lse, int64_t B, int64_t H,
                         int64_t H_kv, int64_t S_q, int64_t S_k, int64_t D, int causal, int64_t window_left,
                         int64_t window_right, float scale, int dtype, void* workspace, int64_t workspace_bytes,
                         void* stream) {
    return fwd_entry(q, k, v, o, lse, B, H, H_kv, S_q, S_k, D, causal, window_left, window_right, scale, dtype,
                     stream, false, workspace, workspace_bytes);
}

extern "C" int fa_fwd_single_buffered(const void* q, const void* k, const void* v, void* o, float* lse, int64_t B,
                                      int64_t H, int64_t S, int64_t D, int causal, float scale, int dtype,
                                      void* stream) {
    return fwd_entry(q, k, v, o, lse, B, H, H, S, S, D, causal, -1, -1, scale, dtype, stream, true);
}

extern "C" int fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int64_t B, int64_t H,
                      int64_t S, int64_t D, int causal, float scale, int dtype, void* stream) {
    return fa_fwd_ex(q, k, v, o, lse, B, H, H, S, S, D, causal, -1, -1, scale, dtype, stream);
}

extern "C" const char* fa_status_string(int status) {
    switch (status) {
        case FA_OK: return "ok";
        case FA_ERR_NULL_POINTER: return "a tensor pointer is NULL";
        case FA_ERR_SHAPE: return "B, H, S_q, S_k must be >= 0 and H a multiple of H_kv";
        case FA_ERR_HEAD_DIM: return "head dim D must be 16, 32, 64 or 128";
        case FA_ERR_DTYPE: return "dtype must be FA_DTYPE_F32, FA_DTYPE_F16 or FA_DTYPE_BF16";
        case FA_ERR_CAUSAL: return "causal must be 0 or 1";
        case FA_ERR_SCALE: return "scale must be finite and > 0";
        case FA_ERR_ALIAS: return "outputs must not overlap each other or the inputs";
        case FA_ERR_TOO_LARGE: return "problem size exceeds the kernels' index ranges";
        case FA_ERR_LAUNCH: return "the HIP runtime rejected the kernel launch";
        case FA_ERR_ALIGNMENT: return "[B,H,S,D] tensors and the fa_fwd_ws workspace must be 16-byte aligned, lse and delta 4-byte aligned";
        case FA_ERR_WINDOW: return "window bounds must be >= -1 (-1: no limit on that side)";
        case FA_ERR_UNSUPPORTED: return "fa_fwd_single_buffered: only the two-block kernel (D = 32, 64, fp16 / bf16, B*H*ceil(S/256) >= 512, no window) has a single-buffered variant";
        case FA_ERR_WORKSPACE: return "workspace: fa_bwd_noalloc needs B * H * S_q <= 4,194,304; fa_fwd_ws needs workspace_bytes >= 0";
        default: return "unknown status";
    }
}
