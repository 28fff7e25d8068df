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
 *   For every batch b, head h and query row i = 0..Sq-1, with the attended key
 *   set J = {0..Sk-1} (non-causal) or J = {j < Sk : j <= i} (causal, key j
 *   visible iff j <= i in absolute positions), narrowed to i - left .. i + right
 *   by an optional window (see key_range), and keys / values taken from the
 *   head's key/value head (see kv_head):
 *
 *     s_j    = scale * sum_{d=0}^{D-1} q[i,d] * k[j,d]          (j in J)
 *     m      = max_{j in J} s_j
 *     p_j    = exp(s_j - m),  l = sum_{j in J} p_j
 *     o[i,d] = (sum_{j in J} p_j * v[j,d]) / l
 *     lse[i] = m + ln(l)                       (natural logarithm)
 *
 *   A row whose key set is empty (a window can cut every key off when Sk < Sq,
 *   and Sk = 0 leaves none) has o = 0 and lse = -inf: the log of an empty sum.
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
 *     (triu with diagonal=1 filled with -inf) and section "Causal Mask 的处理";
 *   - separate query and key counts (Sq queries, Sk keys; keys at or past Sk
 *     do not exist, and the causal test compares absolute query and key
 *     positions): the CS336 write-up's forward kernel, its causal-mask and
 *     tail-boundary (N_QUERIES / N_KEYS) sections.
 *
 * This is deliberately NOT the tiled / online algorithm: no blocking, no
 * running maximum, no rescaling.  Scores are summed over d in ascending order,
 * weights and outputs over j in ascending order.  All arithmetic is IEEE
 * double with the C library's exp and log.
 *
 * Layout: q and o are contiguous [B,H,Sq,D] arrays of double, k and v
 * [B,Hkv,Sk,D]; lse is a contiguous [B,H,Sq] array of double.  Rows are independent, so an OpenMP
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
 * One query row.  q_i points at q[b,h,i,:]; k_bh and v_bh at the first
 * attended key and value row; n_keys = |J| (those keys and the n_keys - 1
 * after them are attended; n_keys <= 0: none, o = 0 and lse = -inf).  `p` is
 * scratch of n_keys doubles, `acc` scratch of D doubles.
 */
static void attend_one_row(const double *q_i, const double *k_bh, const double *v_bh,
                           int64_t n_keys, int64_t D, double scale,
                           double *p, double *acc, double *o_i, double *lse_i)
{
    if (n_keys <= 0) {
        for (int64_t d = 0; d < D; ++d)
            o_i[d] = 0.0;
        *lse_i = -INFINITY;
        return;
    }
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
                      int64_t B, int64_t H, int64_t Hkv, int64_t Sq, int64_t Sk, int64_t D, int causal,
                      int64_t wl, int64_t wr)
{
    if (B < 0 || H < 0 || Sq < 0 || Sk < 0 || D <= 0)
        return ORACLE_BAD_ARGS;
    if (Hkv <= 0 ? H != 0 : H % Hkv != 0)
        return ORACLE_BAD_ARGS;
    if (causal != 0 && causal != 1)
        return ORACLE_BAD_ARGS;
    if (wl < -1 || wr < -1)
        return ORACLE_BAD_ARGS;
    if ((B * H * Sq > 0 && !q) || (B * H * Sk > 0 && (!k || !v)))
        return ORACLE_BAD_ARGS;
    return ORACLE_OK;
}

/*
 * The keys query i attends to form one range [*lo, *hi]: 0 .. Sk-1, cut at i
 * by causal masking (key j visible iff j <= i), at i - wl by a left window
 * and at i + wr by a right window (wl, wr = -1: no limit on that side).
 * This is the window_size = (left, right) convention of "Inside
 * FlashAttention", section 6.1.  For square attention (Sq = Sk) the range
 * always holds key i itself; otherwise it may be empty (*lo > *hi).
 */
static void key_range(int64_t i, int64_t Sk, int causal, int64_t wl, int64_t wr,
                      int64_t *lo, int64_t *hi)
{
    int64_t a = 0, b = causal && i < Sk - 1 ? i : Sk - 1;
    if (wl >= 0 && i - wl > a)
        a = i - wl;
    if (wr >= 0 && i + wr < b)
        b = i + wr;
    *lo = a;
    *hi = b;
}

/*
 * Grouped heads (GQA / MQA, "Inside FlashAttention", section 6.1): H query
 * heads share Hkv key/value heads, G = H / Hkv consecutive query heads per
 * key/value head, so query head bh = b*H + h reads key/value head
 * b*Hkv + h / G = bh / G.
 */
static int64_t kv_head(int64_t bh, int64_t H, int64_t Hkv)
{
    return bh / (H / Hkv);
}

/*
 * Attention over selected rows.  rows[r] is a flat row index
 * (b*H + h)*Sq + i; the row's output goes to o_rows[r*D .. r*D+D-1] and
 * lse_rows[r].  Returns ORACLE_OK, or an error code without writing anything.
 */
int oracle_attn_fwd_rows_ex(const double *q, const double *k, const double *v,
                            int64_t B, int64_t H, int64_t Hkv, int64_t Sq, int64_t Sk, int64_t D, int causal,
                            int64_t wl, int64_t wr, double scale,
                            const int64_t *rows, int64_t n_rows, double *o_rows, double *lse_rows)
{
    int rc = check_args(q, k, v, B, H, Hkv, Sq, Sk, D, causal, wl, wr);
    if (rc != ORACLE_OK)
        return rc;
    if (n_rows < 0 || (n_rows > 0 && (!rows || !o_rows || !lse_rows)))
        return ORACLE_BAD_ARGS;
    const int64_t total = B * H * Sq;
    for (int64_t r = 0; r < n_rows; ++r)
        if (rows[r] < 0 || rows[r] >= total)
            return ORACLE_BAD_ARGS;

    int failed = 0;
#pragma omp parallel
    {
        double *p = (double *)malloc((size_t)(Sk > 0 ? Sk : 1) * sizeof(double));
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
            const int64_t bh = flat / Sq;
            const int64_t i = flat % Sq;
            const int64_t kvh = kv_head(bh, H, Hkv);
            const double *k_bh = k + kvh * Sk * D;
            const double *v_bh = v + kvh * Sk * D;
            int64_t lo, hi;
            key_range(i, Sk, causal, wl, wr, &lo, &hi);
            attend_one_row(q + flat * D, k_bh + lo * D, v_bh + lo * D, hi - lo + 1, D, scale, p, acc,
                           o_rows + r * D, lse_rows + r);
        }
        free(p);
        free(acc);
    }
    return failed ? ORACLE_NO_MEMORY : ORACLE_OK;
}

/* Attention over every row: o is [B,H,Sq,D], lse is [B,H,Sq]; k, v are [B,Hkv,Sk,D]. */
int oracle_attn_fwd_ex(const double *q, const double *k, const double *v, double *o, double *lse,
                       int64_t B, int64_t H, int64_t Hkv, int64_t Sq, int64_t Sk, int64_t D, int causal,
                       int64_t wl, int64_t wr, double scale)
{
    int rc = check_args(q, k, v, B, H, Hkv, Sq, Sk, D, causal, wl, wr);
    if (rc != ORACLE_OK)
        return rc;
    const int64_t total = B * H * Sq;
    if (total == 0)
        return ORACLE_OK;
    if (!o || !lse)
        return ORACLE_BAD_ARGS;

    int failed = 0;
#pragma omp parallel
    {
        double *p = (double *)malloc((size_t)(Sk > 0 ? Sk : 1) * sizeof(double));
        double *acc = (double *)malloc((size_t)D * sizeof(double));
        if (!p || !acc) {
#pragma omp atomic write
            failed = 1;
        }
#pragma omp for schedule(dynamic, 16)
        for (int64_t flat = 0; flat < total; ++flat) {
            if (!p || !acc)
                continue;
            const int64_t bh = flat / Sq;
            const int64_t i = flat % Sq;
            const int64_t kvh = kv_head(bh, H, Hkv);
            int64_t lo, hi;
            key_range(i, Sk, causal, wl, wr, &lo, &hi);
            attend_one_row(q + flat * D, k + (kvh * Sk + lo) * D, v + (kvh * Sk + lo) * D, hi - lo + 1, D,
                           scale, p, acc, o + flat * D, lse + flat);
        }
        free(p);
        free(acc);
    }
    return failed ? ORACLE_NO_MEMORY : ORACLE_OK;
}

int oracle_attn_fwd_rows(const double *q, const double *k, const double *v,
                         int64_t B, int64_t H, int64_t S, int64_t D, int causal, double scale,
                         const int64_t *rows, int64_t n_rows, double *o_rows, double *lse_rows)
{
    return oracle_attn_fwd_rows_ex(q, k, v, B, H, H, S, S, D, causal, -1, -1, scale, rows, n_rows, o_rows,
                                   lse_rows);
}

int oracle_attn_fwd(const double *q, const double *k, const double *v, double *o, double *lse,
                    int64_t B, int64_t H, int64_t S, int64_t D, int causal, double scale)
{
    return oracle_attn_fwd_ex(q, k, v, o, lse, B, H, H, S, S, D, causal, -1, -1, scale);
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
 * With grouped heads, a key/value head's dK and dV sum these terms over the
 * query heads that share it.  A query row that attends to no key (see
 * key_range) has no terms: its dQ is 0 and it adds nothing to dK and dV.
 *
 * Sources: "从零训练语言模型（第二部分）", section "反向传播" (the same five
 * equations, the row term there being rowsum(dO o O), which equals
 * sum_t P_it dP_it because O_i = sum_t P_it V_t); the CS336 write-up's
 * recompute backward (problem flash_backward) for the scale on dQ and dK.
 * The oracle computes P from its own stable softmax (row maximum subtracted,
 * normalised by the row sum) -- no saved lse, no tiling -- and the row term
 * from P and dP, not from O.
 * ------------------------------------------------------------------------ */

/* Softmax weights of one query row over n_keys keys: w[j] = P_ij. */
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

/* g[j] = dP_ij = <dO_i, V_j> over n_keys keys; returns sum_j P_ij dP_ij. */
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

/*
 * Gradients for one key/value head and the G query heads that read it:
 * q_g, do_g, dq_g are those G heads' [G,Sq,D] blocks; k_h, v_h, dk_h, dv_h the
 * key/value head's [Sk,D].  Everything is written.
 */
static void bwd_one_group(const double *q_g, const double *k_h, const double *v_h, const double *do_g,
                          int64_t G, int64_t Sq, int64_t Sk, int64_t D, int causal, int64_t wl, int64_t wr,
                          double scale, double *dq_g, double *dk_h, double *dv_h, double *w, double *g)
{
    for (int64_t x = 0; x < Sk * D; ++x) {
        dk_h[x] = 0.0;
        dv_h[x] = 0.0;
    }
    for (int64_t hq = 0; hq < G; ++hq) {
        for (int64_t i = 0; i < Sq; ++i) {
            int64_t lo, hi;
            key_range(i, Sk, causal, wl, wr, &lo, &hi);
            const int64_t n_keys = hi - lo + 1;
            const double *q_i = q_g + (hq * Sq + i) * D;
            const double *do_i = do_g + (hq * Sq + i) * D;
            double *dq_i = dq_g + (hq * Sq + i) * D;
            for (int64_t d = 0; d < D; ++d)
                dq_i[d] = 0.0;
            if (n_keys <= 0)
                continue;
            bwd_row_weights(q_i, k_h + lo * D, n_keys, D, scale, w);
            const double row = bwd_row_dp(do_i, v_h + lo * D, n_keys, D, w, g);
            for (int64_t j = 0; j < n_keys; ++j) {
                const double ds = w[j] * (g[j] - row);
                const double *kr = k_h + (lo + j) * D;
                double *dk_j = dk_h + (lo + j) * D;
                double *dv_j = dv_h + (lo + j) * D;
                for (int64_t d = 0; d < D; ++d) {
                    dq_i[d] += scale * ds * kr[d];
                    dk_j[d] += scale * ds * q_i[d];
                    dv_j[d] += w[j] * do_i[d];
                }
            }
        }
    }
}

/* Gradients: dq is [B,H,Sq,D], dk and dv are [B,Hkv,Sk,D]. */
int oracle_attn_bwd_ex(const double *q, const double *k, const double *v, const double *dout,
                       double *dq, double *dk, double *dv,
                       int64_t B, int64_t H, int64_t Hkv, int64_t Sq, int64_t Sk, int64_t D, int causal,
                       int64_t wl, int64_t wr, double scale)
{
    int rc = check_args(q, k, v, B, H, Hkv, Sq, Sk, D, causal, wl, wr);
    if (rc != ORACLE_OK)
        return rc;
    if (B * H * (Sq + Sk) == 0)
        return ORACLE_OK;
    if ((Sq > 0 && (!dout || !dq)) || (Sk > 0 && (!dk || !dv)))
        return ORACLE_BAD_ARGS;
    const int64_t groups = B * Hkv, G = H / Hkv;
    int failed = 0;
#pragma omp parallel
    {
        double *w = (double *)malloc((size_t)(Sk > 0 ? Sk : 1) * sizeof(double));
        double *g = (double *)malloc((size_t)(Sk > 0 ? Sk : 1) * sizeof(double));
        if (!w || !g) {
#pragma omp atomic write
            failed = 1;
        }
#pragma omp for schedule(dynamic, 1)
        for (int64_t kvh = 0; kvh < groups; ++kvh) {
            if (!w || !g)
                continue;
            const int64_t qbase = kvh * G * Sq * D, kbase = kvh * Sk * D;
            bwd_one_group(q + qbase, k + kbase, v + kbase, dout + qbase, G, Sq, Sk, D, causal, wl, wr, scale,
                          dq + qbase, dk + kbase, dv + kbase, w, g);
        }
        free(w);
        free(g);
    }
    return failed ? ORACLE_NO_MEMORY : ORACLE_OK;
}

int oracle_attn_bwd(const double *q, const double *k, const double *v, const double *dout,
                    double *dq, double *dk, double *dv,
                    int64_t B, int64_t H, int64_t S, int64_t D, int causal, double scale)
{
    return oracle_attn_bwd_ex(q, k, v, dout, dq, dk, dv, B, H, H, S, S, D, causal, -1, -1, scale);
}

/*
 * Gradients at selected positions.  qrows[r] is a flat query-row index
 * (b*H + h)*Sq + t: dq_rows[r*D ..] receives dQ of that row.  krows[r] is a
 * flat key/value-row index (b*Hkv + hk)*Sk + t: dk_rows / dv_rows[r*D ..]
 * receive dK and dV of that key, summed over the query heads of its group.
 * Every key/value head named by `krows` first gets, for all query rows of its
 * group, the softmax maximum and sum and the row term sum_j P_ij dP_ij; then
 * each key gradient is one pass over the rows that see the key.
 */
int oracle_attn_bwd_rows_ex(const double *q, const double *k, const double *v, const double *dout,
                            int64_t B, int64_t H, int64_t Hkv, int64_t Sq, int64_t Sk, int64_t D, int causal,
                            int64_t wl, int64_t wr, double scale,
                            const int64_t *qrows, int64_t n_qrows, double *dq_rows,
                            const int64_t *krows, int64_t n_krows, double *dk_rows, double *dv_rows)
{
    int rc = check_args(q, k, v, B, H, Hkv, Sq, Sk, D, causal, wl, wr);
    if (rc != ORACLE_OK)
        return rc;
    if (n_qrows < 0 || n_krows < 0 || (n_qrows > 0 && (!qrows || !dout || !dq_rows)) ||
        (n_krows > 0 && (!krows || !dout || !dk_rows || !dv_rows)))
        return ORACLE_BAD_ARGS;
    for (int64_t r = 0; r < n_qrows; ++r)
        if (qrows[r] < 0 || qrows[r] >= B * H * Sq)
            return ORACLE_BAD_ARGS;
    for (int64_t r = 0; r < n_krows; ++r)
        if (krows[r] < 0 || krows[r] >= B * Hkv * Sk)
            return ORACLE_BAD_ARGS;
    if (n_qrows + n_krows == 0)
        return ORACLE_OK;

    /* key/value heads that are needed, and the statistics of their groups' rows */
    const int64_t G = H / Hkv, kvheads = B * Hkv;
    int64_t *slot = (int64_t *)malloc((size_t)(kvheads > 0 ? kvheads : 1) * sizeof(int64_t));
    if (!slot)
        return ORACLE_NO_MEMORY;
    for (int64_t x = 0; x < kvheads; ++x)
        slot[x] = -1;
    int64_t n_groups = 0;
    for (int64_t r = 0; r < n_krows; ++r) {
        const int64_t kvh = krows[r] / Sk;
        if (slot[kvh] < 0)
            slot[kvh] = n_groups++;
    }
    const int64_t n_stat = n_groups * G * Sq;
    int64_t *group_of = (int64_t *)malloc((size_t)(n_groups > 0 ? n_groups : 1) * sizeof(int64_t));
    double *top = (double *)malloc((size_t)(n_stat > 0 ? n_stat : 1) * sizeof(double));
    double *sum = (double *)malloc((size_t)(n_stat > 0 ? n_stat : 1) * sizeof(double));
    double *rowt = (double *)malloc((size_t)(n_stat > 0 ? n_stat : 1) * sizeof(double));
    if (!group_of || !top || !sum || !rowt) {
        free(slot); free(group_of); free(top); free(sum); free(rowt);
        return ORACLE_NO_MEMORY;
    }
    for (int64_t x = 0; x < kvheads; ++x)
        if (slot[x] >= 0)
            group_of[slot[x]] = x;

    int failed = 0;
#pragma omp parallel
    {
        double *w = (double *)malloc((size_t)(Sk > 0 ? Sk : 1) * sizeof(double));
        double *g = (double *)malloc((size_t)(Sk > 0 ? Sk : 1) * sizeof(double));
        if (!w || !g) {
#pragma omp atomic write
            failed = 1;
        }
        /* per query row of each needed group: max, sum and row term (a row
           that sees no key gets none: no key gradient visits it) */
#pragma omp for schedule(dynamic, 16)
        for (int64_t x = 0; x < n_stat; ++x) {
            if (!w || !g)
                continue;
            const int64_t gs = x / (G * Sq), hq = (x / Sq) % G, i = x % Sq;
            const int64_t kvh = group_of[gs];
            const int64_t qrow = (kvh * G + hq) * Sq + i;
            const double *q_i = q + qrow * D;
            const double *k_h = k + kvh * Sk * D, *v_h = v + kvh * Sk * D;
            int64_t lo, hi;
            key_range(i, Sk, causal, wl, wr, &lo, &hi);
            const int64_t n_keys = hi - lo + 1;
            if (n_keys <= 0)
                continue;
            double mx = -INFINITY;
            for (int64_t j = 0; j < n_keys; ++j) {
                const double *kr = k_h + (lo + j) * D;
                double acc = 0.0;
                for (int64_t d = 0; d < D; ++d)
                    acc += q_i[d] * kr[d];
                w[j] = scale * acc;
                if (w[j] > mx)
                    mx = w[j];
            }
            double l = 0.0;
            for (int64_t j = 0; j < n_keys; ++j) {
                w[j] = exp(w[j] - mx);
                l += w[j];
            }
            for (int64_t j = 0; j < n_keys; ++j)
                w[j] /= l;
            top[x] = mx;
            sum[x] = l;
            rowt[x] = bwd_row_dp(dout + qrow * D, v_h + lo * D, n_keys, D, w, g);
        }
        /* dQ of each requested query row */
#pragma omp for schedule(dynamic, 1)
        for (int64_t r = 0; r < n_qrows; ++r) {
            if (!w || !g)
                continue;
            const int64_t bh = qrows[r] / Sq, t = qrows[r] % Sq;
            const int64_t kvh = kv_head(bh, H, Hkv);
            const double *k_h = k + kvh * Sk * D, *v_h = v + kvh * Sk * D;
            int64_t lo, hi;
            key_range(t, Sk, causal, wl, wr, &lo, &hi);
            const int64_t n_keys = hi - lo + 1;
            double *dq_t = dq_rows + r * D;
            for (int64_t d = 0; d < D; ++d)
                dq_t[d] = 0.0;
            if (n_keys <= 0)
                continue;
            bwd_row_weights(q + qrows[r] * D, k_h + lo * D, n_keys, D, scale, w);
            const double row = bwd_row_dp(dout + qrows[r] * D, v_h + lo * D, n_keys, D, w, g);
            for (int64_t j = 0; j < n_keys; ++j) {
                const double ds = w[j] * (g[j] - row);
                for (int64_t d = 0; d < D; ++d)
                    dq_t[d] += scale * ds * k_h[(lo + j) * D + d];
            }
        }
        /* dK and dV of each requested key: every row of the group that sees it */
#pragma omp for schedule(dynamic, 1)
        for (int64_t r = 0; r < n_krows; ++r) {
            const int64_t kvh = krows[r] / Sk, t = krows[r] % Sk;
            const int64_t gs = slot[kvh];
            const double *k_t = k + krows[r] * D;
            const double *v_t = v + krows[r] * D;
            double *dk_t = dk_rows + r * D;
            double *dv_t = dv_rows + r * D;
            for (int64_t d = 0; d < D; ++d) {
                dk_t[d] = 0.0;
                dv_t[d] = 0.0;
            }
            for (int64_t hq = 0; hq < G; ++hq) {
                for (int64_t i = 0; i < Sq; ++i) {
                    int64_t lo, hi;
                    key_range(i, Sk, causal, wl, wr, &lo, &hi);
                    if (t < lo || t > hi)
                        continue;
                    const int64_t qrow = (kvh * G + hq) * Sq + i;
                    const double *q_i = q + qrow * D;
                    const double *do_i = dout + qrow * D;
                    double acc = 0.0, dpv = 0.0;
                    for (int64_t d = 0; d < D; ++d) {
                        acc += q_i[d] * k_t[d];
                        dpv += do_i[d] * v_t[d];
                    }
                    const int64_t x = (gs * G + hq) * Sq + i;
                    const double p = exp(scale * acc - top[x]) / sum[x];
                    const double ds = p * (dpv - rowt[x]);
                    for (int64_t d = 0; d < D; ++d) {
                        dk_t[d] += scale * ds * q_i[d];
                        dv_t[d] += p * do_i[d];
                    }
                }
            }
        }
        free(w);
        free(g);
    }
    free(slot); free(group_of); free(top); free(sum); free(rowt);
    return failed ? ORACLE_NO_MEMORY : ORACLE_OK;
}

/*
 * Gradients at selected positions (square attention, one head per key/value
 * head): for rows[r] = (b*H + h)*S + t, dQ of query t and dK, dV of key t of
 * that head.
 */
int oracle_attn_bwd_rows(const double *q, const double *k, const double *v, const double *dout,
                         int64_t B, int64_t H, int64_t S, int64_t D, int causal, double scale,
                         const int64_t *rows, int64_t n_rows,
                         double *dq_rows, double *dk_rows, double *dv_rows)
{
    return oracle_attn_bwd_rows_ex(q, k, v, dout, B, H, H, S, S, D, causal, -1, -1, scale, rows, n_rows, dq_rows,
                                   rows, n_rows, dk_rows, dv_rows);
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
