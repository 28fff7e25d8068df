/*
 * fa.h -- FlashAttention-2 forward and backward passes for AMD Instinct
 * MI355X (gfx950).
 *
 * One call computes exact attention for every (batch, head):
 *
 *     O   = softmax(Q K^T * scale) V
 *     lse = m + ln(l)      per query row (m: row maximum of the scaled scores,
 *                          l: sum of exp(score - m) over the attended keys)
 *
 * with query blocks as the outer loop and key/value blocks streamed through an
 * inner loop under an online softmax (running maximum, running sum and an fp32
 * output accumulator rescaled by exp(m_old - m_new)).  The [S,S] score and
 * probability matrices never reach device memory; only O and lse are written.
 *
 * Where the operation is defined on the pages:
 *   - the attention definition and the [B,H,S,D] layout: "T5 讲解：
 *     FlashAttention forward", section ① ;
 *   - the Q-outer / K,V-inner loop with the running m, l, acc state and the
 *     rescale factor alpha: same page, sections ③-④ ; "Triton 实现", sections
 *     "Q-outer 主循环" and "内层循环" ; "从零训练语言模型（第二部分）", section
 *     "安全 / 在线 softmax" ;
 *   - causal masking (query i sees keys 0..i) split into off-band blocks with
 *     no mask and on-band diagonal blocks with a mask: "Triton 实现", section
 *     "Causal Mask 的处理：off-band 与 on-band" ; "T5 讲解", section ⑤ ;
 *   - the saved lse = m + log l: "Inside FlashAttention", section 2.4 ;
 *     "T5 讲解", section ⑥ ;
 *   - the default scale 1/sqrt(D) and head dims 16..128: "T5 讲解", section ⑥.
 *
 * Thread safety: calls are independent; the library keeps no state besides
 * the kernels' code objects and allocates, frees and synchronises nothing.
 */
#ifndef FA_H_
#define FA_H_

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- status codes ------------------------------------------------------- */
#define FA_OK 0
#define FA_ERR_NULL_POINTER 1   /* a tensor pointer is NULL for a non-empty problem */
#define FA_ERR_SHAPE 2          /* B, H, S (S_q, S_k) negative, or H not a multiple of H_kv */
#define FA_ERR_HEAD_DIM 3       /* D is not 16, 32, 64 or 128 */
#define FA_ERR_DTYPE 4          /* dtype is not FA_DTYPE_F32 / _F16 / _BF16 (fa_bwd: _F16 / _BF16) */
#define FA_ERR_CAUSAL 5         /* causal is not 0 or 1 */
#define FA_ERR_SCALE 6          /* scale is not finite or not > 0 */
#define FA_ERR_ALIAS 7          /* an output overlaps another output or an input */
#define FA_ERR_TOO_LARGE 8      /* sizes overflow the kernels' index ranges (for fp16 / bf16
                                   also: one head's K or V, S * D * 2 bytes, must be < 2^31) */
#define FA_ERR_LAUNCH 9         /* the HIP runtime rejected the kernel launch */
#define FA_ERR_ALIGNMENT 10     /* a [B,H,S,D] tensor or the fa_fwd_ws workspace not 16-byte aligned,
                                   or lse / delta not 4-byte aligned */
#define FA_ERR_WINDOW 11        /* a window bound is below -1 */
#define FA_ERR_WORKSPACE 12     /* fa_bwd_noalloc: B * H * S_q exceeds its static workspace;
                                   fa_fwd_ws: workspace_bytes < 0 */
#define FA_ERR_UNSUPPORTED 13   /* fa_fwd_single_buffered: no single-buffered variant for this problem */

/* ---- element types (the dtype argument) --------------------------------- */
#define FA_DTYPE_F32 0
#define FA_DTYPE_F16 1
#define FA_DTYPE_BF16 2

/*
 * fa_fwd -- attention forward over B*H independent (batch, head) problems.
 *
 *   q, k, v  device pointers to contiguous [B,H,S,D] tensors of `dtype`
 *            (row-major, last dimension contiguous, 16-byte aligned; they
 *            may alias one another, e.g. q == k).
 *   o        device pointer to a contiguous [B,H,S,D] output of `dtype`.
 *   lse      device pointer to a contiguous [B,H,S] float32 output: the
 *            natural-log log-sum-exp of each query row's scaled scores.
 *   B, H, S  batch, heads, sequence length (queries = keys = S).  Any of them
 *            may be 0 (an empty problem: nothing is launched, FA_OK).
 *   D        head dimension: 16, 32, 64 or 128.
 *   causal   0: every query sees every key; 1: query i sees keys 0..i.
 *   scale    score multiplier, finite and > 0 (callers normally pass
 *            1/sqrt(D) rounded to float32).
 *   dtype    FA_DTYPE_F16 / FA_DTYPE_BF16: both contractions run on the
 *            matrix cores with fp32 accumulation; the softmax weights are
 *            rounded to dtype (nearest-even) before the P*V product.
 *            FA_DTYPE_F32: all arithmetic in fp32.
 *   stream   hipStream_t to enqueue on (NULL = the default stream).
 *
 * Ownership: the caller allocates all five buffers; o and lse must not
 * overlap each other or the inputs.  The library never allocates, frees or
 * synchronises: the kernel is enqueued on `stream` and the call returns at
 * once, so results are ready once the stream reaches that point.
 *
 * Errors: argument checks run before any HIP call and return the FA_ERR_*
 * code of the first failed check, writing nothing.  FA_ERR_LAUNCH reports a
 * launch rejected by the runtime (hipGetLastError); faults during execution
 * surface on the stream, as for any kernel.
 */
int fa_fwd(const void *q, const void *k, const void *v, void *o, float *lse,
           int64_t B, int64_t H, int64_t S, int64_t D,
           int causal, float scale, int dtype, void *stream);

/*
 * fa_bwd -- gradients of the attention above for an upstream gradient dO of O.
 *
 * With P = exp(scale * Q K^T - lse) recomputed from the saved lse (masked
 * keys get 0), D_i = rowsum(dO_i o O_i) and dS = P o (dO V^T - D):
 *
 *     dQ = scale * dS K,   dK = scale * dS^T Q,   dV = P^T dO
 *
 * ("从零训练语言模型（第二部分）", sections "使用 LSE 连接正向和反向传播" and
 * "反向传播": recompute P from lse, then dV, dP, dS, dQ and dK; the CS336
 * write-up, problem flash_backward, for the same equations with the scale.)
 *
 *   q, k, v, o, dout  device pointers to contiguous [B,H,S,D] tensors of
 *                     `dtype` (16-byte aligned): the forward's inputs, its
 *                     output O and the upstream gradient dO.  They may alias
 *                     one another.
 *   lse               device pointer to the forward's float32 [B,H,S] lse
 *                     (natural log), 4-byte aligned.
 *   dq, dk, dv        device pointers to contiguous [B,H,S,D] outputs of
 *                     `dtype` (16-byte aligned), fully written.
 *   delta             device workspace of B*H*S floats (4-byte aligned): the
 *                     call writes D_i there before it reads it; its content
 *                     afterwards is D.
 *   B, H, S, D, causal, scale, stream   as for fa_fwd (the same values the
 *                     forward was called with).
 *   dtype             FA_DTYPE_F16 or FA_DTYPE_BF16 (fp32 is not supported by
 *                     the backward: FA_ERR_DTYPE).  The products run on the
 *                     matrix cores with fp32 accumulation; P and dS are
 *                     rounded (nearest-even) to dtype before the products
 *                     that consume them; the outputs are rounded to dtype.
 *
 * Ownership: the caller allocates all ten buffers; dq, dk, dv and delta must
 * not overlap each other or any input.  Two kernels are enqueued on `stream`
 * (dQ and D, then dK and dV) and the call returns at once; nothing is
 * allocated, freed or synchronised.
 *
 * Errors: as for fa_fwd (checks before any HIP call, the first failed check's
 * code, nothing written), with FA_ERR_DTYPE also for FA_DTYPE_F32.
 */
int fa_bwd(const void *q, const void *k, const void *v, const void *o, const void *dout,
           const float *lse, void *dq, void *dk, void *dv, float *delta,
           int64_t B, int64_t H, int64_t S, int64_t D,
           int causal, float scale, int dtype, void *stream);

/*
 * fa_fwd_ex, fa_bwd_ex -- fa_fwd and fa_bwd with grouped key/value heads, a
 * sliding window, and queries and keys of different length ("Inside
 * FlashAttention", section 6.1: MQA / GQA pass K and V with fewer heads instead
 * of replicating them; window_size = (left, right) limits each query to nearby
 * keys, and whole blocks outside the window are skipped like the blocks above
 * the causal diagonal; the CS336 write-up's forward kernel for separate query
 * and key counts, with keys past the key count absent and the causal test on
 * absolute positions).
 *
 *   H_kv          key/value heads: k, v (and dk, dv) are [B,H_kv,S_k,D]; H
 *                 must be a multiple of H_kv, and query head h reads key/value
 *                 head h / (H / H_kv).  H_kv = H is plain multi-head attention,
 *                 H_kv = 1 is MQA.  The backward sums each shared head's dK and
 *                 dV over its H / H_kv query heads.
 *   S_q, S_k      query rows and key rows per head: q, o, dout, dq are
 *                 [B,H,S_q,D], lse and delta [B,H,S_q], k, v, dk, dv
 *                 [B,H_kv,S_k,D].  Query i and key j sit at positions i and j.
 *   window_left,  query i attends to keys i - window_left .. i + window_right
 *   window_right  (and, when causal, to none past i); -1 leaves that side
 *                 unlimited.  A bound of max(S_q, S_k) or more is the same as -1.
 *   every other argument as for fa_fwd / fa_bwd; fa_fwd(...) is
 *   fa_fwd_ex(..., H_kv = H, S_q = S_k = S, ..., window_left = window_right =
 *   -1, ...), and likewise fa_bwd.
 *
 * A query row that attends to no key (S_k = 0, or a window that leaves the row
 * none, possible only when S_k < S_q) gets O = 0 and lse = -inf (the log of an
 * empty sum); its dQ is 0 and it adds nothing to dK, dV.  With S_q = 0 the
 * backward writes dK = dV = 0; with S_k = 0 it writes dQ = 0 and leaves delta
 * unwritten.
 *
 * Errors: as for fa_fwd / fa_bwd, plus FA_ERR_SHAPE when H is not a multiple
 * of H_kv or S_q, S_k is negative, and FA_ERR_WINDOW for a window bound below
 * -1.  Pointers of a side with no rows (S_q = 0 or S_k = 0) may be NULL.
 */
int fa_fwd_ex(const void *q, const void *k, const void *v, void *o, float *lse,
              int64_t B, int64_t H, int64_t H_kv, int64_t S_q, int64_t S_k, int64_t D,
              int causal, int64_t window_left, int64_t window_right,
              float scale, int dtype, void *stream);
int fa_bwd_ex(const void *q, const void *k, const void *v, const void *o, const void *dout,
              const float *lse, void *dq, void *dk, void *dv, float *delta,
              int64_t B, int64_t H, int64_t H_kv, int64_t S_q, int64_t S_k, int64_t D,
              int causal, int64_t window_left, int64_t window_right,
              float scale, int dtype, void *stream);

/*
 * fa_fwd_workspace_bytes, fa_fwd_ws -- fa_fwd_ex with a caller-given device
 * workspace, which lets the forward split the longest query blocks of a
 * causal problem over two workgroups each.  Every workgroup of a causal grid
 * walks the keys of one query block, so the blocks next to the diagonal's far
 * end are the longest serial chains; when the whole grid is resident on the
 * GPU at once they, not the total work, set the time.  With the workspace, the
 * longer half of the blocks of every head run as two key ranges each, and a
 * second kernel combines the two partial results (O_1, lse_1), (O_2, lse_2) by
 * the log-sum-exp rule
 *
 *     M = max(lse_1, lse_2),  w_i = exp(lse_i - M),
 *     O = (w_1 O_1 + w_2 O_2) / (w_1 + w_2),  lse = M + ln(w_1 + w_2)
 *
 * (the partial results and their merge through the saved lse: "T5 讲解：
 * FlashAttention forward", section ⑥; "Inside FlashAttention", section 2.4).
 * The partials stay fp32, and O is rounded to dtype once, after the merge; the
 * results equal fa_fwd_ex's to within fp32 rounding (the order of the key
 * sums differs), not bit for bit.
 *
 * fa_fwd_workspace_bytes returns the bytes the split needs for a problem (the
 * arguments as for fa_fwd_ex), or 0 when fa_fwd_ws runs it without a
 * workspace, exactly as fa_fwd_ex (no split for that problem, or invalid
 * arguments, which fa_fwd_ws then reports).  Currently: causal, no window,
 * S_q = S_k, dtype fp16 or bf16, and a grid the GPU holds at once (at most 512
 * workgroups of BM query rows): D = 32 or 64 with B * H * ceil(S / 256) = 512
 * (BM = 256); D = 16 with B * H * ceil(S / 128) = 512 (BM = 128); D = 128
 * with B * H * ceil(S / 64) >= 512 and B * H * ceil(S / 128) <= 256
 * (BM = 128).  The size is
 * (ceil(S / BM) / 2) * B * H * 2 * BM * (D + 1) * 4 bytes (about 33 MiB at
 * B * H = 8, S = 16384, D = 64).  No HIP call.
 *
 * fa_fwd_ws: every argument as for fa_fwd_ex, plus
 *   workspace        device memory, 16-byte aligned, apart from every tensor
 *                    of the call; NULL with workspace_bytes = 0 is allowed.
 *   workspace_bytes  its size; >= 0 (FA_ERR_WORKSPACE otherwise).  Below
 *                    fa_fwd_workspace_bytes(...) the call runs without the
 *                    split, as fa_fwd_ex.
 * The call writes the workspace (no initial content is read) and leaves
 * scratch values there; the caller owns it, and two calls in flight at once
 * must not share one.  Like every entry point it allocates, frees and
 * synchronises nothing: with the split it enqueues two kernels on `stream`.
 * Errors: as for fa_fwd_ex, plus FA_ERR_ALIGNMENT for a misaligned workspace
 * and FA_ERR_ALIAS for a workspace that overlaps a tensor (when
 * workspace_bytes > 0).
 */
int64_t fa_fwd_workspace_bytes(int64_t B, int64_t H, int64_t H_kv, int64_t S_q, int64_t S_k, int64_t D,
                               int causal, int64_t window_left, int64_t window_right, int dtype);
int fa_fwd_ws(const void *q, const void *k, const void *v, void *o, float *lse,
              int64_t B, int64_t H, int64_t H_kv, int64_t S_q, int64_t S_k, int64_t D,
              int causal, int64_t window_left, int64_t window_right,
              float scale, int dtype, void *workspace, int64_t workspace_bytes, void *stream);

/*
 * fa_fwd_single_buffered -- race check of the forward's double-buffered K/V
 * staging (a test entry point, not a faster path): fa_fwd computed by the same
 * two-block kernel with one K and one V LDS buffer, each tile's HBM -> LDS
 * transfers issued only after a barrier that follows every wave's last read
 * of the previous tile.  Same arithmetic in the same order, so O and lse must
 * equal fa_fwd's bit for bit; a difference exposes a read of a buffer while a
 * transfer refills it.  (Double buffering of the K/V tiles: "T5 讲解：
 * FlashAttention forward", section ③; "Triton 实现", section "内层循环",
 * num_stages.)
 *
 *   arguments as for fa_fwd.
 *
 * Exists for the problems fa_fwd runs on that kernel: dtype fp16 or bf16,
 * D = 32 or 64, B * H * ceil(S / 256) >= 512.  Any other problem returns
 * FA_ERR_UNSUPPORTED before any HIP call (after the argument checks of
 * fa_fwd, whose codes come first).
 */
int fa_fwd_single_buffered(const void *q, const void *k, const void *v, void *o, float *lse,
                           int64_t B, int64_t H, int64_t S, int64_t D,
                           int causal, float scale, int dtype, void *stream);

/*
 * fa_bwd_noalloc -- fa_bwd_ex without the delta workspace argument, for callers
 * that cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc): the D = rowsum(dO o O)
 * workspace is a static device array inside the library, one per GPU, of
 * 4,194,304 floats (16 MiB, held until the process ends).
 *
 *   every argument as for fa_bwd_ex (same kernels, same results); there is
 *   no delta.
 *
 * Limit: B * H * S_q <= 4,194,304 (FA_ERR_WORKSPACE otherwise, before any HIP
 * call).  The call allocates and frees nothing; on its first use on a device
 * it looks up that device's copy of the array (hipGetSymbolAddress, with the
 * device that runs `stream` current).  The array keeps the last call's D
 * values; nothing in it needs to start at zero.
 *
 * Calls on one GPU share its array: two calls whose executions overlap on the
 * same GPU (e.g. on two streams without ordering between them) race on it and
 * must not be issued.  Calls on one stream are ordered and safe.
 */
int fa_bwd_noalloc(const void *q, const void *k, const void *v, const void *o, const void *dout,
                   const float *lse, void *dq, void *dk, void *dv,
                   int64_t B, int64_t H, int64_t H_kv, int64_t S_q, int64_t S_k, int64_t D,
                   int causal, int64_t window_left, int64_t window_right,
                   float scale, int dtype, void *stream);

/* A static, human-readable description of a status code (never NULL). */
const char *fa_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* FA_H_ */
