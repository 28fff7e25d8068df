// fa_mfma.hpp -- FlashAttention-2 forward for fp16 / bf16 inputs on the gfx950 matrix cores.
//
// One workgroup owns one block of BM = NW * 32 * QB query rows of one
// (batch, head) and streams that head's keys and values through LDS in tiles
// of BN rows (query blocks outer, key/value blocks inner: "Triton 实现",
// sections "Grid 与并行策略" and "Q-outer 主循环"; "T5 讲解", section ②).
// Each wave owns 32 * QB whole query rows, so no softmax statistics cross a
// wave ("Inside FlashAttention", section 4.3, split-Q).
//
// Work per wave and key tile t:
//   S^T = K_t * Q^T           32x32x16 MFMAs, fp32 accumulators.  Computing the
//                             transpose puts one query per lane column, so a row
//                             maximum or sum is a reduction inside the lane plus
//                             one exchange between the two wave halves.
//   mask                      only on tiles that cross the causal diagonal or the
//                             end of the sequence; off-band tiles take no compare
//                             ("Triton 实现", section "Causal Mask 的处理";
//                             "T5 讲解", section ⑤).
//   online softmax            exp2 form, c = scale * log2(e) ("Triton 实现",
//                             section "内层循环"): p = exp2(S*c - m), l += rowsum(p),
//                             P rounded (nearest-even) to the input type.
//   O^T += V_t^T * P^T        fp32 accumulation.
// The epilogue divides by l once and writes O and lse = ln2 * (m + log2 l), the
// natural-log form ("Inside FlashAttention", sections 2.4 and 4.1).
//
// The running reference m.  The pages move m to the running row maximum on
// every tile and rescale l and acc by alpha = exp(m_old - m_new)
// ("从零训练语言模型（第二部分）", section "安全 / 在线 softmax").  Here m moves
// only when it must: each tile is first exponentiated against the current m;
// if any of the wave's partial row sums of that tile exceeds 2^14 (so some
// p > 2^14, or an exp2 overflowed), the tile is redone the pages' way -- m_new =
// max(m, c * rowmax(S)), l and acc rescaled by alpha = exp2(m - m_new), p
// recomputed.  Every accepted p is <= 2^14, inside fp16 range, and the result
// is the same exact attention; on typical inputs only the first tile of a row
// takes the slow path, which removes the per-element maximum from all others.
//
// Two loop shapes (Cfg::PIPE).  Pipelined: within one wave the MFMAs of a tile
// depend on that tile's softmax and the other way round, so iteration t issues,
// as one straight-line block, the S MFMAs of tile t+1 and the P*V MFMAs of tile
// t-1 together with the softmax of tile t; the matrix cores then work on the
// neighbouring tiles while the vector ALUs run the exponentials.  This needs two
// sets of score and P registers.  Plain: one tile after the other (S, mask,
// softmax, P*V) with one register set, and an LDS tile of TBN keys consumed in
// TBN / BN compute steps between barriers; used where the accumulators leave no
// room for a second set (D = 128), with the other waves of the SIMD providing
// the overlap.
//
// Data movement: Q fragments live in VGPRs for the whole loop ("T5 讲解",
// section ③).  K and V tiles go from HBM straight into LDS with 16-byte
// global_load_lds transfers (no VGPR staging), two buffers each in separately
// declared LDS arrays (so the compiler's LDS-DMA tracking sees them apart); in
// the pipelined loop K runs one tile ahead of V.  Both are stored row-major with an XOR swizzle of
// 16-byte chunks per row (applied on the HBM side of the transfer), chosen so
// that the K operand reads (ds_read_b128 of one chunk of 32 consecutive rows)
// and the V operand reads (ds_read_b64_tr_b16 of 8-byte pieces of four
// consecutive rows, transposed across lanes) hit distinct banks.
#pragma once

#include <type_traits>

#include "fa_common.hpp"

#define FA_LDS __attribute__((address_space(3)))

namespace fa {

typedef short s16x4 __attribute__((ext_vector_type(4)));

template <int D_, bool CAUSAL_, int QB_, int NW_, int BN_, bool PIPE_ = true, int OCC_ = 2, int TBN_ = BN_>
struct MfmaConfig {
    static constexpr int TBN = TBN_;        // keys per LDS tile (a multiple of BN; BN = keys per compute step)
    static constexpr bool PIPE = PIPE_;     // software-pipelined tile loop (two score/P sets)
    static constexpr int OCC = OCC_;        // waves per SIMD the register budget is sized for
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
    static constexpr int TILE = TBN * RB;   // bytes per K or V LDS tile
    static constexpr int LOADS = TILE / 1024;            // 1 KiB wave transfers per tile
    static constexpr int LOADS_PER_WAVE = (LOADS + NW - 1) / NW;
    static_assert(D == 16 || D == 32 || D == 64 || D == 128, "head dim");
    static_assert(BN % 32 == 0, "BN must be a multiple of 32");
    static_assert(TBN % BN == 0, "LDS tile = whole compute steps");
    static_assert(TILE % 1024 == 0 && (LOADS % NW == 0 || LOADS < NW), "tile transfers per wave");
    static_assert(2 * 2 * TILE <= 160 * 1024, "LDS");
};

// A tile's partial row sums above this trigger the exact rescale path.
constexpr float kSumLimit = 16384.0f;

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

// Wait until at most N of this wave's vector-memory operations are
// outstanding (they complete in issue order).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N <= 15, "vmcnt immediate");
    __builtin_amdgcn_s_waitcnt(0x0F70 | N);
}

// Workgroup barrier that orders LDS accesses only: it waits for this wave's
// LDS operations (lgkmcnt) but not for its vector-memory loads, so HBM -> LDS
// transfers of later tiles stay in flight across it (__syncthreads' fence
// waits for those too).  Data written by such a transfer is published by the
// issuing wave's own vmcnt wait before the barrier.  The memory clobber keeps
// the compiler from moving memory accesses across it.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// Per-lane byte offset (within one head's K or V) of this wave's i-th 16-byte
// transfer of a tile starting at key 0: transfer `inst` of the tile covers LDS
// bytes inst*1024 .. +1023, lane l fills 16 bytes at l*16 of it, i.e. row
// slot / CPR, chunk slot % CPR (slot = inst*64 + l); the chunk read from HBM is
// that position's swizzled chunk.
template <typename Cfg, bool ISV>
__device__ __forceinline__ uint32_t tile_lane_offset(int inst, int lane) {
    const int slot = inst * 64 + lane;
    const int row = slot / Cfg::CPR;
    const int p = slot % Cfg::CPR;
    const int c = p ^ (ISV ? swz_v<Cfg::D>(row) : swz_k<Cfg::D>(row));
    return (uint32_t)(row * Cfg::RB + c * 16);
}

// Buffer-resource word 3 for raw (untyped) dword buffer loads on gfx9-class
// hardware: a non-zero data format, everything else default.
constexpr int kBufferFlags = 0x00020000;

// Buffer resource of one head's K or V rows (`bytes` long): transfers that
// reach at or beyond its end read zeros.  (Templated on the element type, like
// every helper that calls target builtins here, so that every kernel instance
// has its own copy: the host-side pass of one instance cannot then poison the
// overload for the next.)
template <typename T>
__device__ __forceinline__ __amdgpu_buffer_rsrc_t head_rsrc(const uint16_t* head, int bytes) {
    return __builtin_amdgcn_make_buffer_rsrc((void*)head, 0, bytes, kBufferFlags);
}

// Issue this wave's share of the HBM -> LDS transfers of one K or V tile (rows
// k0 .. k0+TBN-1 of the head behind `rsrc`), as buffer loads that write LDS
// directly; rows at or beyond S read as zeros (their keys are masked to -inf and
// their values only ever meet p = 0).  Transfer i of the wave (inst = wave +
// i*NW) covers rows i*NW*1024/RB further on than transfer 0; when that is a
// multiple of the swizzles' 16-row period, its lane offsets are transfer 0's
// (lane_off) plus i*NW KiB, so no per-transfer offset occupies a register.
template <typename T, typename Cfg, bool ISV>
__device__ __forceinline__ void load_tile(FA_LDS char* dst, __amdgpu_buffer_rsrc_t rsrc, uint32_t lane_off, int k0,
                                          int wave, int lane) {
    constexpr bool kPeriodic = (Cfg::NW * 1024 / Cfg::RB) % 16 == 0;
#pragma unroll
    for (int i = 0; i < Cfg::LOADS_PER_WAVE; ++i) {
        const int inst = wave + i * Cfg::NW;
        if (Cfg::LOADS < Cfg::NW && inst >= Cfg::LOADS) break;  // wave-uniform
        const uint32_t off = kPeriodic ? lane_off + (uint32_t)(i * Cfg::NW * 1024) : tile_lane_offset<Cfg, ISV>(inst, lane);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (FA_LDS void*)(dst + inst * 1024), 16,
                                                 off + (uint32_t)(k0 * Cfg::RB), 0, 0, 0);
    }
}

// One row-sum step for a pair (p0, p1) of a lane's probabilities: two fp32 adds
// of the unrounded values (the pages sum p before it is rounded for the P*V
// product).  Every path sums the pairs of a tile in the same order, so a row's l
// does not depend on which path (steady, edge, rescale) handled a tile.
__device__ __forceinline__ float pair_sum(float acc, float p0, float p1, bool first) {
    return first ? p0 + p1 : acc + (p0 + p1);
}

// One 1 KiB HBM -> LDS transfer (64 lanes x 16 bytes): the lane's 16 bytes at
// lane_off + k0 * RB of the head behind `rsrc` to dst + lane * 16.
template <typename T, typename Cfg>
__device__ __forceinline__ void load_part(FA_LDS char* dst, __amdgpu_buffer_rsrc_t rsrc, uint32_t lane_off, int k0) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (FA_LDS void*)dst, 16, lane_off + (uint32_t)(k0 * Cfg::RB), 0, 0, 0);
}

// Work order of a causal grid whose workgroups are longest first, heads
// fastest (position p: head p % BH, rank p / BH).  With `round` > 0 (a grid of
// at most two resident rounds of `round` workgroups: all of it fits on the GPU
// at once, and workgroup i + round lands on the compute unit of workgroup i),
// the second round takes its blocks in the opposite order, so that a unit that
// got a long block in the first round gets a short one next.  When BH divides
// both rounds, only the ranks are reversed and every workgroup keeps its head,
// so a head's workgroups stay on the XCD (and L2) the plain order gives them.
// Returns this workgroup's position in the longest-first order.
__device__ __forceinline__ int causal_work_index(int round, int BH) {
    int lin = blockIdx.x;
    if (round > 0 && lin >= round && lin < 2 * round) {
        const int m = min(round, (int)gridDim.x - round);  // second-round workgroups
        if (round % BH == 0 && m % BH == 0)
            lin = round + (m / BH - 1 - (lin - round) / BH) * BH + lin % BH;
        else
            lin = 2 * round + m - 1 - lin;
    }
    return lin;
}

// The work items of one head when its nsplit longest causal blocks are split
// into two key halves (blocks m = n - nsplit .. n - 1 as two halves, blocks
// 0 .. m - 1 whole; causal block q holds q + 1 blocks' worth of keys, so in
// units of half that, half q has length q + 1 and whole q length 2(q + 1)),
// listed longest first (a whole block before two halves of its length, part 0
// before part 1).
// The grid is resident all at once and the hardware starts each further
// workgroup on the first free slot, so this order is the longest-processing-
// time-first rule: long items start together and short ones fill the gaps.
// Item `rank` is found by a binary search on its length L: count(L), the
// number of items of length >= L, is a closed form.
__device__ __forceinline__ void split_work_item(int rank, int n, int nsplit, int& qblk, int& part) {
    const int m = n - nsplit;
    auto count = [&](int L) {  // items of length >= L (L >= 1)
        const int halves = 2 * max(0, n - max(m, L - 1));
        const int wholes = max(0, m - max(0, (L + 1) / 2 - 1));
        return halves + wholes;
    };
    // largest L in [1, 2n] with count(L) > rank (count(1) = n + nsplit > rank)
    int lo = 1, hi = 2 * n;
    while (lo < hi) {
        const int mid = (lo + hi + 1) / 2;
        if (count(mid) > rank) lo = mid;
        else hi = mid - 1;
    }
    int off = rank - count(lo + 1);  // position among the items of length lo
    const int qw = lo / 2 - 1;       // the whole block of this length, if any
    if ((lo & 1) == 0 && qw >= 0 && qw < m) {
        if (off == 0) {
            qblk = qw;
            part = -1;
            return;
        }
        --off;
    }
    qblk = lo - 1;  // the split block of this length: part 0, then part 1
    part = off;
}

// A key half's partial result for one 32-row column block of a wave (fp32,
// rows `row0` + n of the workspace, n = lane % 32): O normalised by the half's
// own l, and its lse = ln2 * (m + log2 l) (-inf for a row with no key in the
// half: weight 0 in the merge).
template <int D, int DB>
__device__ __forceinline__ void store_partial(float* __restrict__ PO, float* __restrict__ PL, int64_t row0,
                                              const f32x16 (&o)[DB], float l_lane, float m, int n, int h) {
    const float l = halves_sum(l_lane);
    const float inv = l > 0.f ? 1.0f / l : 0.f;
    const int64_t row = row0 + n;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const int d = db * 32 + 8 * g + 4 * h;
            if (d < D) {
                f32x4 w;
#pragma unroll
                for (int e = 0; e < 4; ++e) w[e] = o[db][4 * g + e] * inv;
                *reinterpret_cast<f32x4*>(PO + row * D + d) = w;
            }
        }
    if (h == 0) PL[row] = kLn2 * (m + log2_fast(l));
}

// Per-wave state and the pieces of work on one tile.
template <typename T, typename Cfg>
struct WaveTile {
    static constexpr int D = Cfg::D, QB = Cfg::QB, KB = Cfg::KB, KS = Cfg::KS, DB = Cfg::DB;
    static constexpr int RB = Cfg::RB;
    static constexpr int NQK = KB * KS * QB;      // S^T MFMAs per tile
    static constexpr int NPV = KB * 2 * DB * QB;  // O^T MFMAs per tile
    static constexpr int NP = QB * KB * 8;        // score pairs per lane per tile

    // K fragment of 32-key block kb, k-step ks: A operand K[32kb + n][16ks + 8h .. +7].
    static __device__ __forceinline__ u32x4 k_frag(const FA_LDS char* kt, const int (&offk)[KS], int kb, int ks) {
        return *reinterpret_cast<const FA_LDS u32x4*>(kt + kb * 32 * RB + offk[ks]);
    }

    // V^T fragment of keys 32kb + 16j + {4h..4h+3, 8+4h..8+4h+3}, dims 32db + n,
    // via two transposed 8-byte reads.
    static __device__ __forceinline__ u32x4 v_frag(const FA_LDS char* vt, const int (&offv)[DB], int kb, int j,
                                                   int db) {
        const FA_LDS char* base = vt + (kb * 32 + 16 * j) * RB + offv[db];
        const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((FA_LDS s16x4*)base);
        const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((FA_LDS s16x4*)(base + 8 * RB));
        const u32x2 lo2 = __builtin_bit_cast(u32x2, lo), hi2 = __builtin_bit_cast(u32x2, hi);
        return u32x4{lo2[0], lo2[1], hi2[0], hi2[1]};
    }

    // S^T = K Q^T for the tile in `kt`.
    static __device__ __forceinline__ void qk(const FA_LDS char* kt, const int (&offk)[KS],
                                              const u32x4 (&qf)[QB][KS], f32x16 (&s)[QB][KB]) {
        const f32x16 zero = {};
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                const u32x4 kf = k_frag(kt, offk, kb, ks);
#pragma unroll
                for (int qb = 0; qb < QB; ++qb)
                    s[qb][kb] = mfma32x32x16<T>(kf, qf[qb][ks], ks == 0 ? zero : s[qb][kb]);
            }
    }

    // O^T += V^T P^T for the tile in `vt`.
    static __device__ __forceinline__ void pv(const FA_LDS char* vt, const int (&offv)[DB],
                                              const u32x4 (&pk)[QB][KB][2], f32x16 (&oacc)[QB][DB]) {
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int db = 0; db < DB; ++db) {
                    const u32x4 vf = v_frag(vt, offv, kb, j, db);
#pragma unroll
                    for (int qb = 0; qb < QB; ++qb)
                        oacc[qb][db] = mfma32x32x16<T>(vf, pk[qb][kb][j], oacc[qb][db]);
                }
    }

    // Causal / sequence-end mask: key of register r of block kb is
    // k0 + 32kb + 4h + 8(r/4) + r%4; it is visible iff key <= last[qb].
    static __device__ __forceinline__ void mask(f32x16 (&s)[QB][KB], const int (&last)[QB], int k0, int h) {
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) {
                const int lim = last[qb] - (k0 + kb * 32 + 4 * h);
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    if (8 * (r >> 2) + (r & 3) > lim) s[qb][kb][r] = kNegInf;
            }
    }

    // Pair e of the lane's scores: column block qb = e / (8 KB), key block
    // kb = (e / 8) % KB, registers r = 2 (e % 8) and r + 1.  Its packed P lands in
    // slot (e % 8) % 4 of MFMA operand (e % 8) / 4 (operand j holds registers
    // 8j .. 8j+7, i.e. keys 16j + {4h..4h+3, 8+4h..8+4h+3} of the block).
    struct Pair {
        float p0, p1;
    };
    static __device__ __forceinline__ Pair pair_exp(const f32x16 (&s)[QB][KB], const float (&m_run)[QB], float c,
                                                    int e) {
        const int qb = e / (8 * KB), kb = (e / 8) % KB, r = 2 * (e % 8);
        return {exp2_fast(__builtin_fmaf(s[qb][kb][r], c, -m_run[qb])),
                exp2_fast(__builtin_fmaf(s[qb][kb][r + 1], c, -m_run[qb]))};
    }
    static __device__ __forceinline__ void pair_pack(Pair x, int e, u32x4 (&pk)[QB][KB][2], float (&rs)[QB]) {
        const int qb = e / (8 * KB), kb = (e / 8) % KB, i = e % 8;
        pk[qb][kb][i >> 2][i & 3] = pack2<T>(x.p0, x.p1);
        rs[qb] = pair_sum(rs[qb], x.p0, x.p1, kb == 0 && i == 0);
    }

    // p = exp2(S*c - m): packs P for the P*V MFMAs and returns the lane's
    // partial row sums in rs.
    static __device__ __forceinline__ void expo(const f32x16 (&s)[QB][KB], const float (&m_run)[QB], float c,
                                                u32x4 (&pk)[QB][KB][2], float (&rs)[QB]) {
#pragma unroll
        for (int e = 0; e < NP; ++e) pair_pack(pair_exp(s, m_run, c, e), e, pk, rs);
        // Materialise P here: otherwise the packing sinks below the rescale
        // branch and keeps every unpacked fp32 p alive across it.
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) {
                pin(pk[qb][kb][0]);
                pin(pk[qb][kb][1]);
            }
    }

    // Row maximum of the lane's query column over the tile (both wave halves).
    static __device__ __forceinline__ float row_max(const f32x16 (&s)[QB][KB], int qb) {
        float a = s[qb][0][0], b = s[qb][0][1];
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
            for (int r = (kb == 0 ? 2 : 0); r < 16; r += 4) {
                a = fmaxf(fmaxf(a, s[qb][kb][r]), s[qb][kb][r + 1]);
                b = fmaxf(fmaxf(b, s[qb][kb][r + 2]), s[qb][kb][r + 3]);
            }
        return halves_max(fmaxf(a, b));
    }

    // A row's first tile: m = c * rowmax, so every p <= 1 and the sum cannot
    // overflow.
    static __device__ __forceinline__ void first(const f32x16 (&s)[QB][KB], float (&m_run)[QB], float (&l_run)[QB],
                                                 float c, u32x4 (&pk)[QB][KB][2]) {
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) m_run[qb] = fmaxf(m_run[qb], row_max(s, qb) * c);
        expo(s, m_run, c, pk, l_run);
    }

    // One steady pipelined step: S^T of tile t+1 (K in kn), O^T += V^T P^T of
    // tile t-1 (V in vp, P in p_prv) and the softmax of tile t (s_cur -> p_cur).
    // Written in issue order -- operand reads from LDS first, two pairs of
    // scores exponentiated while they are in flight, then every MFMA followed by
    // its share of the softmax -- and left to the compiler's scheduler (pinning
    // the order measured slower).  Same arithmetic as qk + pv + expo.
    // PIN_ORDER: pin the issue order at D = 128 (the one-block kernel; the
    // key-split kernel, whose D = 128 instance runs one wave per SIMD, measured
    // slower with it: B=8 H=1 S=1024 12.3 -> 14.0 us)
    template <bool PIN_ORDER = false>
    static __device__ __forceinline__ void step(const FA_LDS char* kn, const FA_LDS char* vp, const int (&offk)[KS],
                                                const int (&offv)[DB], const u32x4 (&qf)[QB][KS],
                                                const f32x16 (&s_cur)[QB][KB], f32x16 (&s_nxt)[QB][KB],
                                                const u32x4 (&p_prv)[QB][KB][2], u32x4 (&p_cur)[QB][KB][2],
                                                f32x16 (&oacc)[QB][DB], const float (&m_run)[QB], float c,
                                                float (&rs)[QB]) {
        constexpr int NM = NQK + NPV;
        constexpr int LEAD = 2;
        u32x4 kf[KB][KS];
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) kf[kb][ks] = k_frag(kn, offk, kb, ks);
        u32x4 vf[KB][2][DB];
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int db = 0; db < DB; ++db) vf[kb][j][db] = v_frag(vp, offv, kb, j, db);
        Pair x[NP];
        int nf = 0, nc = 0;
#pragma unroll
        for (; nf < LEAD; ++nf) x[nf] = pair_exp(s_cur, m_run, c, nf);
        const f32x16 zero = {};
#pragma unroll
        for (int i = 0; i < NM; ++i) {
            if (i < NQK) {
                const int kb = i / (KS * QB), ks = (i / QB) % KS, qb = i % QB;
                s_nxt[qb][kb] = mfma32x32x16<T>(kf[kb][ks], qf[qb][ks], ks == 0 ? zero : s_nxt[qb][kb]);
            } else {
                const int u = i - NQK;
                const int kb = u / (2 * DB * QB), j = (u / (DB * QB)) % 2, db = (u / QB) % DB, qb = u % QB;
                oacc[qb][db] = mfma32x32x16<T>(vf[kb][j][db], p_prv[qb][kb][j], oacc[qb][db]);
            }
            // this slot's share: exponentials up to f_end, packing up to c_end
            const int nf0 = nf;
            const int f_end = i == NM - 1 ? NP : LEAD + ((i + 1) * (NP - LEAD) + NM / 2) / NM;
            const int c_end = i == NM - 1 ? NP : min(((i + 1) * NP + NM / 2) / NM, nf0);
#pragma unroll
            for (; nf < f_end; ++nf) x[nf] = pair_exp(s_cur, m_run, c, nf);
#pragma unroll
            for (; nc < c_end; ++nc) pair_pack(x[nc], nc, p_cur, rs);
        }
        if constexpr (PIN_ORDER && Cfg::D == 128 && QB == 1 && KB == 1) {
            // D = 128, 32-key steps: the issue order pinned by scheduling
            // groups, four vector instructions first, then every MFMA followed
            // by three of them (measured 1-8 % faster than the compiler's
            // order; lead 8, or four per MFMA, gained less)
            __builtin_amdgcn_sched_group_barrier(kSchedValu, 4, 0);
#pragma unroll
            for (int i = 0; i < NM; ++i) {
                __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
                __builtin_amdgcn_sched_group_barrier(kSchedValu, 3, 0);
            }
        }
    }

    // True when some lane's partial sum of this tile is out of range (or inf).
    static __device__ __forceinline__ bool needs_rescale(const float (&rs)[QB]) {
        float mx = rs[0];
#pragma unroll
        for (int qb = 1; qb < QB; ++qb) mx = fmaxf(mx, rs[qb]);
        return __builtin_amdgcn_ballot_w64(!(mx <= kSumLimit)) != 0;
    }

    // The exact path: move m to max(m, c * rowmax(S)), rescale l and acc by
    // alpha = exp2(m_old - m_new), and exponentiate the tile again.
    static __device__ __forceinline__ void rescale(const f32x16 (&s)[QB][KB], float (&m_run)[QB], float (&l_run)[QB],
                                                   f32x16 (&oacc)[QB][DB], float c, u32x4 (&pk)[QB][KB][2],
                                                   float (&rs)[QB]) {
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
            const float m_new = fmaxf(m_run[qb], row_max(s, qb) * c);
            const float alpha = exp2_fast(m_run[qb] - m_new);
            m_run[qb] = m_new;
            l_run[qb] *= alpha;
#pragma unroll
            for (int db = 0; db < DB; ++db)
#pragma unroll
                for (int r = 0; r < 16; ++r) oacc[qb][db][r] *= alpha;
        }
        expo(s, m_run, c, pk, rs);
    }
};

template <typename T, typename Cfg, bool KSPLIT = false>
__global__ __attribute__((amdgpu_flat_work_group_size(Cfg::NT, Cfg::NT), amdgpu_waves_per_eu(Cfg::OCC, Cfg::OCC)))
void fa_fwd_mfma_kernel(const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
                        const uint16_t* __restrict__ V, uint16_t* __restrict__ O, float* __restrict__ LSE,
                        int Sq, int Sk, int BH, int n_qblk, int G, float c, float* __restrict__ PO,
                        float* __restrict__ PL, int nsplit) {
    using W = WaveTile<T, Cfg>;
    constexpr int D = Cfg::D, QB = Cfg::QB, KB = Cfg::KB, KS = Cfg::KS, DB = Cfg::DB;
    constexpr int BN = Cfg::BN, BM = Cfg::BM, BMW = Cfg::BMW, RB = Cfg::RB;
    constexpr bool CAUSAL = Cfg::CAUSAL;
    static_assert(!Cfg::PIPE || Cfg::TBN == BN, "the pipelined loop stages one compute tile per LDS tile");

    __shared__ __attribute__((aligned(1024))) char k_lds0[Cfg::TILE];
    __shared__ __attribute__((aligned(1024))) char k_lds1[Cfg::TILE];
    __shared__ __attribute__((aligned(1024))) char v_lds0[Cfg::TILE];
    __shared__ __attribute__((aligned(1024))) char v_lds1[Cfg::TILE];
    FA_LDS char* const kbuf[2] = {(FA_LDS char*)k_lds0, (FA_LDS char*)k_lds1};
    FA_LDS char* const vbuf[2] = {(FA_LDS char*)v_lds0, (FA_LDS char*)v_lds1};

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int n = lane & 31;  // MFMA output column = this lane's query within a 32-block
    const int h = lane >> 5;  // wave half

    // Workgroup -> (head, query block).  Heads vary fastest so that the
    // workgroups of one head land on one XCD (dispatch is round-robin over the
    // 8 XCDs) and share its K/V in that XCD's L2; causal blocks go longest first.
    // With KSPLIT (causal, a workspace PO / PL) the nsplit longest blocks of
    // every head run as two workgroups over the two halves of their keys
    // (split_work_item), each writing an fp32 partial result that
    // fa_fwd_merge_kernel combines by the log-sum-exp rule ("T5 讲解", section
    // ⑥; "Inside FlashAttention", section 2.4).
    int bh, qblk;
    int part = -1;  // -1: the whole block; 0, 1: its first or second key half
    if constexpr (KSPLIT) {
        static_assert(CAUSAL, "the key split serves causal problems");
        bh = blockIdx.x % BH;
        split_work_item(blockIdx.x / BH, n_qblk, nsplit, qblk, part);
    } else {
        const int wg = blockIdx.x;
        bh = wg % BH;
        const int rank = wg / BH;
        qblk = CAUSAL ? (n_qblk - 1 - rank) : rank;
    }
    const int q0 = qblk * BM;
    const int qw = q0 + wave * BMW;

    // The block's key tiles and this workgroup's range [tb, te) of them (all,
    // for a whole block; halves split at a multiple of the LDS tile).  The K/V
    // resources start at key kb = tb * BN, and tile indices, key limits and
    // masks below are relative to it (kb = 0 for a whole block).
    constexpr int SUB = Cfg::TBN / BN;
    const int ntiles_blk = ((CAUSAL ? min(q0 + BM, Sk) : Sk) + BN - 1) / BN;
    const int tsplit = (ntiles_blk / 2) / SUB * SUB;
    const int tb = part == 1 ? tsplit : 0;
    const int te = part == 0 ? tsplit : ntiles_blk;
    const int kb = tb * BN;
    const int Skr = Sk - kb;  // keys from kb on
    const int qwr = qw - kb;  // this wave's first query, relative to kb

    const int64_t head = (int64_t)bh * Sq * D;
    // grouped heads: G query heads per K/V head
    const int64_t kvhead = (int64_t)(bh / G) * Sk * D + (int64_t)kb * D;
    const uint16_t* qh = Q + head;
    const __amdgpu_buffer_rsrc_t krs = head_rsrc<T>(K + kvhead, Skr * RB);
    const __amdgpu_buffer_rsrc_t vrs = head_rsrc<T>(V + kvhead, Skr * RB);
    const uint32_t koff = tile_lane_offset<Cfg, false>(wave, lane);
    const uint32_t voff = tile_lane_offset<Cfg, true>(wave, lane);

    const int ntiles = te - tb;
    // tiles this wave attends to (its last query's diagonal for causal)
    const int wend = CAUSAL ? min(qw + BMW, Sk) : Sk;
    const int wtiles = qw < Sq ? max(0, min(te, (wend + BN - 1) / BN) - tb) : 0;

    // First tiles in flight before anything else: K(0) and, pipelined, K(1);
    // otherwise K(0) and V(0).
    load_tile<T, Cfg, false>(kbuf[0], krs, koff, 0, wave, lane);
    if constexpr (Cfg::PIPE) {
        if (ntiles > 1) load_tile<T, Cfg, false>(kbuf[1], krs, koff, BN, wave, lane);
    } else {
        load_tile<T, Cfg, true>(vbuf[0], vrs, voff, 0, wave, lane);
    }

    // Q^T operand fragments: lane holds Q[query][16ks + 8h .. +7].  Rows beyond
    // S repeat row S-1; their outputs are never stored.
    u32x4 qf[QB][KS];
    int last[QB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        const int qrow = min(qw + qb * 32 + n, Sq - 1);
        last[qb] = (CAUSAL ? min(qrow, Sk - 1) : Sk - 1) - kb;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
            qf[qb][ks] = *reinterpret_cast<const u32x4*>(qh + (int64_t)qrow * D + ks * 16 + h * 8);
    }
    // Q stays resident for the whole loop: read once ("T5 讲解", section ③)
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) pin(qf[qb][ks]);

    // Per-lane LDS byte offsets of the operand reads (constant over tiles).
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

    // Two sets of score and probability registers trade roles every tile.
    f32x16 sA[QB][KB], sB[QB][KB];
    u32x4 pA[QB][KB][2], pB[QB][KB][2];

    if constexpr (!Cfg::PIPE) {
        // One LDS tile (TBN keys) per barrier; inside it, compute steps of BN
        // keys: S, (mask), softmax, P*V -- single register sets.
        const int nlds = (ntiles + SUB - 1) / SUB;
        auto simple = [&](int lt, FA_LDS char* kc, FA_LDS char* vc, FA_LDS char* kn, FA_LDS char* vn)
                          __attribute__((always_inline)) {
            wait_vmcnt0();
            __syncthreads();
            if (lt + 1 < nlds) {
                load_tile<T, Cfg, false>(kn, krs, koff, (lt + 1) * Cfg::TBN, wave, lane);
                load_tile<T, Cfg, true>(vn, vrs, voff, (lt + 1) * Cfg::TBN, wave, lane);
            }
#pragma unroll
            for (int sub = 0; sub < SUB; ++sub) {
                const int t = lt * SUB + sub;
                if (t >= wtiles) break;  // wave-uniform
                const int k0 = t * BN;
                W::qk(kc + sub * BN * RB, offk, qf, sA);
                if ((CAUSAL && k0 + BN - 1 > qwr) || k0 + BN > Skr) W::mask(sA, last, k0, h);
                if (t == 0) {
                    W::first(sA, m_run, l_run, c, pA);
                } else {
                    float rs[QB];
                    W::expo(sA, m_run, c, pA, rs);
                    if (W::needs_rescale(rs)) W::rescale(sA, m_run, l_run, oacc, c, pA, rs);
#pragma unroll
                    for (int qb = 0; qb < QB; ++qb) l_run[qb] += rs[qb];
                }
                W::pv(vc + sub * BN * RB, offv, pA, oacc);
            }
        };
        for (int lt = 0; lt < nlds; lt += 2) {
            simple(lt, kbuf[0], vbuf[0], kbuf[1], vbuf[1]);
            if (lt + 1 < nlds) simple(lt + 1, kbuf[1], vbuf[1], kbuf[0], vbuf[0]);
        }
    } else {
        wait_vmcnt0();
        __syncthreads();
        if (wtiles > 0) W::qk(kbuf[0], offk, qf, sA);

        // Iteration t: S(t) in s_cur, S(t+1) goes to s_nxt, P(t-1) in p_prv, P(t)
        // goes to p_cur; K(t) / V(t) live in buffer t&1, K(t+1) / V(t-1) in the
        // other.  Steady iterations (1 <= t, t+1 < wtiles, tile t unmasked) are
        // branch-free so that their MFMAs and exponentials form one basic block.
        auto iter = [&](auto kind, int t, FA_LDS char* kc, FA_LDS char* kn, FA_LDS char* vc, FA_LDS char* vp,
                        f32x16 (&s_cur)[QB][KB], f32x16 (&s_nxt)[QB][KB], u32x4 (&p_prv)[QB][KB][2],
                        u32x4 (&p_cur)[QB][KB][2]) __attribute__((always_inline)) {
            constexpr int KIND = decltype(kind)::value;  // 0 first, 1 steady, 2 edge
            const int k0 = t * BN;
            wait_vmcnt0();
            __syncthreads();  // K(t+1) and V(t-1) visible; K(t) and V(t-2) no longer read
            if (KIND == 1 || t + 2 < ntiles) load_tile<T, Cfg, false>(kc, krs, koff, k0 + 2 * BN, wave, lane);
            load_tile<T, Cfg, true>(vc, vrs, voff, k0, wave, lane);

            if constexpr (KIND == 0) {
                if (t >= wtiles) return;
                if (t + 1 < wtiles) W::qk(kn, offk, qf, s_nxt);
                if ((CAUSAL && k0 + BN - 1 > qwr) || k0 + BN > Skr) W::mask(s_cur, last, k0, h);
                W::first(s_cur, m_run, l_run, c, p_cur);
                return;
            }
            float rs[QB];
            if constexpr (KIND == 1) {
                W::template step<true>(kn, vp, offk, offv, qf, s_cur, s_nxt, p_prv, p_cur, oacc, m_run, c, rs);
            } else {
                const bool do_qk = t + 1 < wtiles;
                const bool do_pv = t <= wtiles;
                if (t >= wtiles) {
                    if (do_pv) W::pv(vp, offv, p_prv, oacc);  // this wave's last tile, while V(t-1) is resident
                    return;
                }
                if (do_qk) W::qk(kn, offk, qf, s_nxt);
                W::pv(vp, offv, p_prv, oacc);
                if ((CAUSAL && k0 + BN - 1 > qwr) || k0 + BN > Skr) W::mask(s_cur, last, k0, h);
                W::expo(s_cur, m_run, c, p_cur, rs);
            }
            // P*V of tile t-1 is in acc now, so a rescale covers every earlier term.
            if (W::needs_rescale(rs)) W::rescale(s_cur, m_run, l_run, oacc, c, p_cur, rs);
#pragma unroll
            for (int qb = 0; qb < QB; ++qb) l_run[qb] += rs[qb];
        };
        using First = std::integral_constant<int, 0>;
        using Steady = std::integral_constant<int, 1>;
        using Edge = std::integral_constant<int, 2>;

        // leading tiles that need no mask for any of this wave's rows
        const int unmasked = min(CAUSAL ? (qwr + 1) / BN : ntiles, Skr / BN);
        const int steady_end = min(wtiles - 1, unmasked);  // steady for 1 <= t < steady_end

        iter(First{}, 0, kbuf[0], kbuf[1], vbuf[0], vbuf[1], sA, sB, pA, pB);
        int t = 1;
        for (; t + 1 < steady_end; t += 2) {
            iter(Steady{}, t, kbuf[1], kbuf[0], vbuf[1], vbuf[0], sB, sA, pB, pA);
            iter(Steady{}, t + 1, kbuf[0], kbuf[1], vbuf[0], vbuf[1], sA, sB, pA, pB);
        }
        for (; t < ntiles; t += 2) {
            iter(Edge{}, t, kbuf[1], kbuf[0], vbuf[1], vbuf[0], sB, sA, pB, pA);
            if (t + 1 < ntiles) iter(Edge{}, t + 1, kbuf[0], kbuf[1], vbuf[0], vbuf[1], sA, sB, pA, pB);
        }
        // drain: P*V of the last tile for waves that attend to every tile
        wait_vmcnt0();
        __syncthreads();
        if (wtiles == ntiles && wtiles > 0) {
            if ((ntiles - 1) & 1) W::pv(vbuf[1], offv, pA, oacc);
            else W::pv(vbuf[0], offv, pB, oacc);
        }
    }

    // ---- epilogue: O = acc / l, lse = ln2 * (m + log2 l) ---------------------------
    if (KSPLIT && part >= 0) {
        // a key half: its fp32 partial, item (2j + part) * BH + bh of BM rows
        // (j: the block's rank among the split ones), rows in block order
        const int64_t item = ((int64_t)(2 * (n_qblk - 1 - qblk) + part) * BH + bh) * BM;
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
            store_partial<D, DB>(PO, PL, item + (qw - q0) + 32 * qb, oacc[qb], l_run[qb], m_run[qb], n, h);
        return;
    }
    uint16_t* oh = O + head;
    float* lh = LSE + (int64_t)bh * Sq;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        const float l = halves_sum(l_run[qb]);
        const float inv = 1.0f / l;
        const int qrow = qw + qb * 32 + n;
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

// Combines the two key halves of every split block (fa_fwd_split_kernel with
// nsplit > 0) by the log-sum-exp rule: with partial results (O_h, lse_h),
//     M = max_h lse_h,  w_h = exp(lse_h - M),  O = sum_h w_h O_h / sum_h w_h,
//     lse = M + ln(sum_h w_h),
// rounded to the input type once.  One thread per 4 dims of a row.
template <typename T, int D, int BM>
__global__ __launch_bounds__(256) void fa_fwd_merge_kernel(const float* __restrict__ PO, const float* __restrict__ PL,
                                                           uint16_t* __restrict__ O, float* __restrict__ LSE, int Sq,
                                                           int BH, int n_qblk, int nsplit) {
    constexpr int CH = D / 4;  // 4-dim chunks per row
    const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (t >= (int64_t)nsplit * BH * BM * CH) return;
    const int chunk = (int)(t % CH);
    const int64_t r = t / CH;
    const int i = (int)(r % BM);
    const int bh = (int)((r / BM) % BH);
    const int j = (int)(r / ((int64_t)BM * BH));
    const int qrow = (n_qblk - 1 - j) * BM + i;
    if (qrow >= Sq) return;
    const int64_t r0 = ((int64_t)(2 * j) * BH + bh) * BM + i;
    const int64_t r1 = ((int64_t)(2 * j + 1) * BH + bh) * BM + i;
    const float l0 = PL[r0], l1 = PL[r1];
    const float mx = fmaxf(l0, l1);
    const float w0 = exp2_fast((l0 - mx) * kLog2e), w1 = exp2_fast((l1 - mx) * kLog2e);
    const float ws = w0 + w1;
    const float inv = 1.0f / ws;
    const f32x4 a = *reinterpret_cast<const f32x4*>(PO + r0 * D + 4 * chunk);
    const f32x4 b = *reinterpret_cast<const f32x4*>(PO + r1 * D + 4 * chunk);
    u32x2 w;
    w[0] = pack2<T>((w0 * a[0] + w1 * b[0]) * inv, (w0 * a[1] + w1 * b[1]) * inv);
    w[1] = pack2<T>((w0 * a[2] + w1 * b[2]) * inv, (w0 * a[3] + w1 * b[3]) * inv);
    *reinterpret_cast<u32x2*>(O + ((int64_t)bh * Sq + qrow) * D + 4 * chunk) = w;
    if (chunk == 0) LSE[(int64_t)bh * Sq + qrow] = mx + kLn2 * log2_fast(ws);
}

}  // namespace fa
