/*
 * attn_oracle.c -- plain, slow, double-precision attention forward on the CPU.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the parity oracle for the HIP
 * kernels of this repository.  Only the test suite, the smoke check and the
 * CPU-baseline leg of the benchmark may load it; the product library never
 * links, includes or calls anything from here, and this file includes nothing
 * from the product.
 *
 * What it computes (exact attention, written out as its definition):
 *
 *   For every batch b, head h and query row i, with the attended key set
 *   J = {0..S-1} (non-causal) or J = {0..i} (causal, key j visible iff j <= i):
 *
 *     s_j    = scale * sum_{d=0}^{D-1} q[i,d] * k[j,d]          (j in J)
 *     m      = max_{j in J} s_j
 *     p_j    = exp(s_j - m),  l = sum_{j in J} p_j
 *     o[i,d] = (sum_{j in J} p_j * v[j,d]) / l
 *     lse[i] = m + ln(l)                       (natural logarithm)
 *
 * Sources on the pages:
 *   - the attention definition O = softmax(Q K^T * scale) V over [B,H,S,D]
 *     tensors: "T5 讲解：FlashAttention forward", section ① ; "Inside
 *     FlashAttention", section 1.1 (the three-step naive implementation);
 *   - subtracting the row maximum before exponentiating (stable softmax):
 *     "从零训练语言模型（第二部分）", section "安全 / 在线 softmax";
 *   - lse = m + log l, one scalar per row, kept for the backward pass:
 *     "Inside FlashAttention", section 2.4; same page 2 section "使用 LSE";
 *   - causal visibility (query i sees keys 0..i; the upper triangle above the
 *     diagonal is masked): "Triton 实现", the naive pytorch_attention listing
 *     (triu with diagonal=1 filled with -inf) and section "Causal Mask 的处理".
 *
 * This is deliberately NOT the tiled / online algorithm: no blocking, no
 * running maximum, no rescaling.  Scores are summed over d in ascending order,
 * weights and outputs over j in ascending order.  All arithmetic is IEEE
 * double with the C library's exp and log.
 *
 * Layout: q, k, v, o are contiguous [B,H,S,D] arrays of double; lse is a
 * contiguous [B,H,S] array of double.  Rows are independent, so an OpenMP
 * loop over (b,h,i) is the only parallelism.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* Status codes of the oracle entry points. */
#define ORACLE_OK 0
#define ORACLE_BAD_ARGS 1
#define ORACLE_NO_MEMORY 2

/*
 * One query row.  q_i points at q[b,h,i,:]; k_bh and v_bh at k[b,h,0,:] and
 * v[b,h,0,:]; n_keys = |J| (keys 0..n_keys-1 are attended).  `p` is scratch of
 * n_keys doubles, `acc` scratch of D doubles.
 */
static void attend_one_row(const double *q_i, const double *k_bh, const double *v_bh,
                           int64_t n_keys, int64_t D, double scale,
                           double *p, double *acc, double *o_i, double *lse_i)
{
    /* scores s_j = scale * <q_i, k_j> */
    for (int64_t j = 0; j < n_keys; ++j) {
        const double *k_j = k_bh + j * D;
        double dot = 0.0;
        for (int64_t d = 0; d < D; ++d)
            dot += q_i[d] * k_j[d];
        p[j] = scale * dot;
    }

    /* m = max_j s_j */
    double m = -INFINITY;
    for (int64_t j = 0; j < n_keys; ++j)
        if (p[j] > m)
            m = p[j];

    /* p_j = exp(s_j - m), l = sum_j p_j */
    double l = 0.0;
    for (int64_t j = 0; j < n_keys; ++j) {
        p[j] = exp(p[j] - m);
        l += p[j];
    }

    /* o = (sum_j p_j v_j) / l */
    for (int64_t d = 0; d < D; ++d)
        acc[d] = 0.0;
    for (int64_t j = 0; j < n_keys; ++j) {
        const double *v_j = v_bh + j * D;
        for (int64_t d = 0; d < D; ++d)
            acc[d] += p[j] * v_j[d];
    }
    for (int64_t d = 0; d < D; ++d)
        o_i[d] = acc[d] / l;

    *lse_i = m + log(l);
}

static int check_args(const double *q, const double *k, const double *v,
                      int64_t B, int64_t H, int64_t S, int64_t D, int causal)
{
    if (B < 0 || H < 0 || S < 0 || D <= 0)
        return ORACLE_BAD_ARGS;
    if (causal != 0 && causal != 1)
        return ORACLE_BAD_ARGS;
    if (B * H * S > 0 && (!q || !k || !v))
        return ORACLE_BAD_ARGS;
    return ORACLE_OK;
}

/*
 * Attention over selected rows.  rows[r] is a flat row index
 * (b*H + h)*S + i; the row's output goes to o_rows[r*D .. r*D+D-1] and
 * lse_rows[r].  Returns ORACLE_OK, or an error code without writing anything.
 */
int oracle_attn_fwd_rows(const double *q, const double *k, const double *v,
                         int64_t B, int64_t H, int64_t S, int64_t D, int causal, double scale,
                         const int64_t *rows, int64_t n_rows, double *o_rows, double *lse_rows)
{
    int rc = check_args(q, k, v, B, H, S, D, causal);
    if (rc != ORACLE_OK)
        return rc;
    if (n_rows < 0 || (n_rows > 0 && (!rows || !o_rows || !lse_rows)))
        return ORACLE_BAD_ARGS;
    const int64_t total = B * H * S;
    for (int64_t r = 0; r < n_rows; ++r)
        if (rows[r] < 0 || rows[r] >= total)
            return ORACLE_BAD_ARGS;

    int failed = 0;
#pragma omp parallel
    {
        double *p = (double *)malloc((size_t)(S > 0 ? S : 1) * sizeof(double));
        double *acc = (double *)malloc((size_t)D * sizeof(double));
        if (!p || !acc) {
#pragma omp atomic write
            failed = 1;
        }
#pragma omp for schedule(dynamic, 16)
        for (int64_t r = 0; r < n_rows; ++r) {
            if (!p || !acc)
                continue;
            const int64_t flat = rows[r];
            const int64_t bh = flat / S;
            const int64_t i = flat % S;
            const double *k_bh = k + bh * S * D;
            const double *v_bh = v + bh * S * D;
            const int64_t n_keys = causal ? i + 1 : S;
            attend_one_row(q + flat * D, k_bh, v_bh, n_keys, D, scale, p, acc,
                           o_rows + r * D, lse_rows + r);
        }
        free(p);
        free(acc);
    }
    return failed ? ORACLE_NO_MEMORY : ORACLE_OK;
}

/* Attention over every row: o is [B,H,S,D], lse is [B,H,S]. */
int oracle_attn_fwd(const double *q, const double *k, const double *v, double *o, double *lse,
                    int64_t B, int64_t H, int64_t S, int64_t D, int causal, double scale)
{
    int rc = check_args(q, k, v, B, H, S, D, causal);
    if (rc != ORACLE_OK)
        return rc;
    const int64_t total = B * H * S;
    if (total == 0)
        return ORACLE_OK;
    if (!o || !lse)
        return ORACLE_BAD_ARGS;

    int failed = 0;
#pragma omp parallel
    {
        double *p = (double *)malloc((size_t)S * sizeof(double));
        double *acc = (double *)malloc((size_t)D * sizeof(double));
        if (!p || !acc) {
#pragma omp atomic write
            failed = 1;
        }
#pragma omp for schedule(dynamic, 16)
        for (int64_t flat = 0; flat < total; ++flat) {
            if (!p || !acc)
                continue;
            const int64_t bh = flat / S;
            const int64_t i = flat % S;
            const int64_t n_keys = causal ? i + 1 : S;
            attend_one_row(q + flat * D, k + bh * S * D, v + bh * S * D, n_keys, D, scale,
                           p, acc, o + flat * D, lse + flat);
        }
        free(p);
        free(acc);
    }
    return failed ? ORACLE_NO_MEMORY : ORACLE_OK;
}

/* Number of OpenMP threads a parallel region of the oracle uses. */
int oracle_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
