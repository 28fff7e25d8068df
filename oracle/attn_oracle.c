/*
 * attn_oracle.c -- plain, slow, double-precision attention forward and
 * backward on the CPU.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the parity oracle for the HIP
 * kernels of this repository.  Only the test suite, the smoke check and the
 * CPU-baseline leg of the benchmark may load it; the product library never
 * links, includes or calls anything from here, and this file includes nothing
 * from the product.
 *
 * What the forward computes (exact attention, written out as its definition;
 * the backward, further down, is described where it is defined):
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

/* ------------------------------------------------------------------------
 * Backward pass: gradients of exact attention, written out from the
 * definition.  For one head, with P the row-wise softmax of scale * Q K^T over
 * each row's attended keys (other keys carry weight 0), O = P V and an upstream
 * gradient dO of O:
 *
 *   dV_j  = sum_i P_ij dO_i
 *   dP_ij = <dO_i, V_j>
 *   dS_ij = P_ij (dP_ij - sum_t P_it dP_it)     (Jacobian of the softmax of row i)
 *   dQ_i  = scale * sum_j dS_ij K_j
 *   dK_j  = scale * sum_i dS_ij Q_i
 *
 * Sources: "从零训练语言模型（第二部分）", section "反向传播" (the same five
 * equations, the row term there being rowsum(dO o O), which equals
 * sum_t P_it dP_it because O_i = sum_t P_it V_t); the CS336 write-up's
 * recompute backward (problem flash_backward) for the scale on dQ and dK.
 * The oracle computes P from its own stable softmax (row maximum subtracted,
 * normalised by the row sum) -- no saved lse, no tiling -- and the row term
 * from P and dP, not from O.
 * ------------------------------------------------------------------------ */

/* Softmax weights of one query row over keys 0..n_keys-1: w[j] = P_ij. */
static void bwd_row_weights(const double *q_i, const double *k_bh, int64_t n_keys, int64_t D,
                            double scale, double *w)
{
    double top = -INFINITY;
    for (int64_t j = 0; j < n_keys; ++j) {
        const double *kr = k_bh + j * D;
        double acc = 0.0;
        for (int64_t d = 0; d < D; ++d)
            acc += q_i[d] * kr[d];
        w[j] = scale * acc;
        if (w[j] > top)
            top = w[j];
    }
    double total = 0.0;
    for (int64_t j = 0; j < n_keys; ++j) {
        w[j] = exp(w[j] - top);
        total += w[j];
    }
    for (int64_t j = 0; j < n_keys; ++j)
        w[j] /= total;
}

/* g[j] = dP_ij = <dO_i, V_j> for keys 0..n_keys-1; returns sum_j P_ij dP_ij. */
static double bwd_row_dp(const double *do_i, const double *v_bh, int64_t n_keys, int64_t D,
                         const double *w, double *g)
{
    double row = 0.0;
    for (int64_t j = 0; j < n_keys; ++j) {
        const double *vr = v_bh + j * D;
        double acc = 0.0;
        for (int64_t d = 0; d < D; ++d)
            acc += do_i[d] * vr[d];
        g[j] = acc;
        row += w[j] * acc;
    }
    return row;
}

/* Gradients of one head: dq, dk, dv are [S,D] and fully written. */
static void bwd_one_head(const double *q_bh, const double *k_bh, const double *v_bh, const double *do_bh,
                         int64_t S, int64_t D, int causal, double scale,
                         double *dq_bh, double *dk_bh, double *dv_bh, double *w, double *g)
{
    for (int64_t x = 0; x < S * D; ++x) {
        dk_bh[x] = 0.0;
        dv_bh[x] = 0.0;
    }
    for (int64_t i = 0; i < S; ++i) {
        const int64_t n_keys = causal ? i + 1 : S;
        const double *q_i = q_bh + i * D;
        const double *do_i = do_bh + i * D;
        bwd_row_weights(q_i, k_bh, n_keys, D, scale, w);
        const double row = bwd_row_dp(do_i, v_bh, n_keys, D, w, g);
        double *dq_i = dq_bh + i * D;
        for (int64_t d = 0; d < D; ++d)
            dq_i[d] = 0.0;
        for (int64_t j = 0; j < n_keys; ++j) {
            const double ds = w[j] * (g[j] - row);
            const double *kr = k_bh + j * D;
            double *dk_j = dk_bh + j * D;
            double *dv_j = dv_bh + j * D;
            for (int64_t d = 0; d < D; ++d) {
                dq_i[d] += scale * ds * kr[d];
                dk_j[d] += scale * ds * q_i[d];
                dv_j[d] += w[j] * do_i[d];
            }
        }
    }
}

/* Gradients of every head: dq, dk, dv are [B,H,S,D]. */
int oracle_attn_bwd(const double *q, const double *k, const double *v, const double *dout,
                    double *dq, double *dk, double *dv,
                    int64_t B, int64_t H, int64_t S, int64_t D, int causal, double scale)
{
    int rc = check_args(q, k, v, B, H, S, D, causal);
    if (rc != ORACLE_OK)
        return rc;
    if (B * H * S == 0)
        return ORACLE_OK;
    if (!dout || !dq || !dk || !dv)
        return ORACLE_BAD_ARGS;
    const int64_t heads = B * H;
    int failed = 0;
#pragma omp parallel
    {
        double *w = (double *)malloc((size_t)S * sizeof(double));
        double *g = (double *)malloc((size_t)S * sizeof(double));
        if (!w || !g) {
#pragma omp atomic write
            failed = 1;
        }
#pragma omp for schedule(dynamic, 1)
        for (int64_t bh = 0; bh < heads; ++bh) {
            if (!w || !g)
                continue;
            const int64_t base = bh * S * D;
            bwd_one_head(q + base, k + base, v + base, dout + base, S, D, causal, scale,
                         dq + base, dk + base, dv + base, w, g);
        }
        free(w);
        free(g);
    }
    return failed ? ORACLE_NO_MEMORY : ORACLE_OK;
}

/*
 * Gradients at selected positions.  rows[r] is a flat index (b*H + h)*S + t;
 * dq_rows[r*D ..] receives dQ of query t, dk_rows / dv_rows of key t (all of
 * head b*H + h).  Every head named by `rows` first gets, for all of its query
 * rows i, the softmax maximum and sum and the row term sum_j P_ij dP_ij; then
 * each key gradient is one pass over the queries that see the key.
 */
int oracle_attn_bwd_rows(const double *q, const double *k, const double *v, const double *dout,
                         int64_t B, int64_t H, int64_t S, int64_t D, int causal, double scale,
                         const int64_t *rows, int64_t n_rows,
                         double *dq_rows, double *dk_rows, double *dv_rows)
{
    int rc = check_args(q, k, v, B, H, S, D, causal);
    if (rc != ORACLE_OK)
        return rc;
    if (n_rows < 0 || (n_rows > 0 && (!rows || !dout || !dq_rows || !dk_rows || !dv_rows)))
        return ORACLE_BAD_ARGS;
    const int64_t total = B * H * S;
    for (int64_t r = 0; r < n_rows; ++r)
        if (rows[r] < 0 || rows[r] >= total)
            return ORACLE_BAD_ARGS;
    if (n_rows == 0)
        return ORACLE_OK;

    /* heads that are needed, and their per-row statistics */
    const int64_t heads = B * H;
    int64_t *slot = (int64_t *)malloc((size_t)heads * sizeof(int64_t));
    if (!slot)
        return ORACLE_NO_MEMORY;
    for (int64_t bh = 0; bh < heads; ++bh)
        slot[bh] = -1;
    int64_t n_heads = 0;
    for (int64_t r = 0; r < n_rows; ++r) {
        const int64_t bh = rows[r] / S;
        if (slot[bh] < 0)
            slot[bh] = n_heads++;
    }
    int64_t *head_of = (int64_t *)malloc((size_t)n_heads * sizeof(int64_t));
    double *top = (double *)malloc((size_t)(n_heads * S) * sizeof(double));
    double *sum = (double *)malloc((size_t)(n_heads * S) * sizeof(double));
    double *rowt = (double *)malloc((size_t)(n_heads * S) * sizeof(double));
    if (!head_of || !top || !sum || !rowt) {
        free(slot); free(head_of); free(top); free(sum); free(rowt);
        return ORACLE_NO_MEMORY;
    }
    for (int64_t bh = 0; bh < heads; ++bh)
        if (slot[bh] >= 0)
            head_of[slot[bh]] = bh;

    int failed = 0;
#pragma omp parallel
    {
        double *w = (double *)malloc((size_t)S * sizeof(double));
        double *g = (double *)malloc((size_t)S * sizeof(double));
        if (!w || !g) {
#pragma omp atomic write
            failed = 1;
        }
        /* per query row i of each needed head: max, sum and row term */
#pragma omp for schedule(dynamic, 16)
        for (int64_t x = 0; x < n_heads * S; ++x) {
            if (!w || !g)
                continue;
            const int64_t hs = x / S, i = x % S;
            const int64_t base = head_of[hs] * S * D;
            const int64_t n_keys = causal ? i + 1 : S;
            const double *q_i = q + base + i * D;
            double hi = -INFINITY;
            for (int64_t j = 0; j < n_keys; ++j) {
                const double *kr = k + base + j * D;
                double acc = 0.0;
                for (int64_t d = 0; d < D; ++d)
                    acc += q_i[d] * kr[d];
                w[j] = scale * acc;
                if (w[j] > hi)
                    hi = w[j];
            }
            double l = 0.0;
            for (int64_t j = 0; j < n_keys; ++j) {
                w[j] = exp(w[j] - hi);
                l += w[j];
            }
            for (int64_t j = 0; j < n_keys; ++j)
                w[j] /= l;
            top[x] = hi;
            sum[x] = l;
            rowt[x] = bwd_row_dp(dout + base + i * D, v + base, n_keys, D, w, g);
        }
        /* each requested position: dQ of its query, dK and dV of its key */
#pragma omp for schedule(dynamic, 1)
        for (int64_t r = 0; r < n_rows; ++r) {
            if (!w || !g)
                continue;
            const int64_t bh = rows[r] / S, t = rows[r] % S;
            const int64_t hs = slot[bh];
            const int64_t base = bh * S * D;
            const int64_t n_keys = causal ? t + 1 : S;
            bwd_row_weights(q + base + t * D, k + base, n_keys, D, scale, w);
            const double row = bwd_row_dp(dout + base + t * D, v + base, n_keys, D, w, g);
            double *dq_t = dq_rows + r * D;
            double *dk_t = dk_rows + r * D;
            double *dv_t = dv_rows + r * D;
            for (int64_t d = 0; d < D; ++d) {
                dq_t[d] = 0.0;
                dk_t[d] = 0.0;
                dv_t[d] = 0.0;
            }
            for (int64_t j = 0; j < n_keys; ++j) {
                const double ds = w[j] * (g[j] - row);
                for (int64_t d = 0; d < D; ++d)
                    dq_t[d] += scale * ds * k[base + j * D + d];
            }
            /* key t is seen by queries i >= t (causal) or by all */
            const double *k_t = k + base + t * D;
            const double *v_t = v + base + t * D;
            for (int64_t i = causal ? t : 0; i < S; ++i) {
                const double *q_i = q + base + i * D;
                const double *do_i = dout + base + i * D;
                double acc = 0.0, dpv = 0.0;
                for (int64_t d = 0; d < D; ++d) {
                    acc += q_i[d] * k_t[d];
                    dpv += do_i[d] * v_t[d];
                }
                const int64_t x = hs * S + i;
                const double p = exp(scale * acc - top[x]) / sum[x];
                const double ds = p * (dpv - rowt[x]);
                for (int64_t d = 0; d < D; ++d) {
                    dk_t[d] += scale * ds * q_i[d];
                    dv_t[d] += p * do_i[d];
                }
            }
        }
        free(w);
        free(g);
    }
    free(slot); free(head_of); free(top); free(sum); free(rowt);
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
