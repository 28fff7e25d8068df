/*
 * fa_micro.h -- issue-rate microbenchmarks of the gfx950 instructions the
 * attention kernels are made of (a measurement tool beside libfa.so, built
 * into libfa_micro.so; not part of the attention computation).
 *
 * Why: per attended (query, key) pair the attention forward costs 4*D
 * matrix-core FLOPs but also one exponential and a few vector ALU
 * operations, which cost far more per FLOP than the matrix products
 * ("Inside FlashAttention", section 4.1); "从零训练语言模型（第二部分）",
 * section "先做性能分析", starts optimisation from measuring where the time
 * goes.  These probes measure the issue cost of each instruction kind alone,
 * and how vector work overlaps the matrix cores within one wave and between
 * the two waves that share a SIMD, so that the vector-side bound of the
 * attention kernels can be stated in cycles.
 */
#ifndef FA_MICRO_H_
#define FA_MICRO_H_

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define FA_MICRO_OK 0
#define FA_MICRO_ERR_ARG 1      /* an argument outside the ranges below */
#define FA_MICRO_ERR_LAUNCH 2   /* the HIP runtime rejected the launch */

/* vector instruction kinds (op) */
#define FA_MICRO_OP_EXP 0       /* v_exp_f32 */
#define FA_MICRO_OP_FMA 1       /* v_fma_f32 */
#define FA_MICRO_OP_ADD 2       /* v_add_f32 */
#define FA_MICRO_OP_CVT 3       /* v_cvt_pk_f16_f32 */
#define FA_MICRO_OP_EXP16 4     /* v_exp_f16 */
#define FA_MICRO_OP_PKADD16 5   /* v_pk_add_f16 */
#define FA_MICRO_OP_MAX3 6      /* v_max3_f32 */

/* what the waves run (mode) */
#define FA_MICRO_MIXED 0        /* every wave: 8 x (one 32x32x16 fp16 MFMA, then k vector ops) */
#define FA_MICRO_PRODUCTS 1     /* every wave: 8 MFMAs on 4 independent accumulators */
#define FA_MICRO_VECTOR 2       /* every wave: 8*k vector ops (32 if k = 0), 16 independent registers */
#define FA_MICRO_SPLIT 3        /* 8 waves: waves 0-3 PRODUCTS, waves 4-7 VECTOR (two per SIMD) */

/*
 * fa_micro -- one workgroup of `waves` waves (wave w on SIMD w % 4) runs
 * `iters` iterations of the body `mode` selects and each wave writes the
 * shader-clock cycles its loop took (s_memtime) to cycles[w].
 *
 *   op      FA_MICRO_OP_*: the vector instruction of the body.
 *   k       vector instructions per MFMA (mixed) or the vector body's length
 *           / 8: 0, 1, 2, 4, 8 or 16.
 *   agpr    1: MFMA accumulators in AGPRs; 0: in arch VGPRs.
 *   mode    FA_MICRO_MIXED .. FA_MICRO_SPLIT.
 *   waves   1..8 (SPLIT: exactly 8).
 *   iters   1 .. 2^20.
 *   cycles  device pointer to `waves` uint64_t, written.
 *   stream  hipStream_t to enqueue on (NULL = default stream).
 *
 * Returns FA_MICRO_ERR_ARG before any HIP call for an argument out of range,
 * FA_MICRO_ERR_LAUNCH when the runtime rejects the launch, else FA_MICRO_OK.
 * The call returns at once; the cycles are ready when the stream reaches it.
 */
int fa_micro(int op, int k, int agpr, int mode, int waves, int iters, uint64_t *cycles, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* FA_MICRO_H_ */
