/*
 * entmax_attn.h -- C ABI of the alpha-entmax attention library for AMD MI355X (gfx950).
 *
 * The operation (AdaSplash-2, "Faster Differentiable Sparse Attention", gist.science
 * summaries): alpha-entmax attention, a sparse and differentiable replacement of
 * softmax attention whose normaliser tau is found per query row by root finding
 * (AdaSplash-2 (zh, ja, es) §1). For row i with scores s_ij = scale * q_i . k_j:
 *
 *     x_ij = (alpha - 1) s_ij,   p_ij = [x_ij - tau_i]_+^(1/(alpha-1)),   sum_j p_ij = 1,
 *     o_i  = sum_j p_ij v_j.
 *
 * tau_i is initialised from a B-bin histogram of the row's scores built while keys
 * stream through on-chip memory (AdaSplash-2 (zh) §2.1; AdaSplash-2 (ja) §2.1,
 * Proposition 1: tau* - 1/B < tau_h <= tau*), refined by a safeguarded hybrid
 * solver -- Halley for alpha <= 1.5, Newton for 1.5 < alpha <= 2, secant above,
 * bisection whenever a step leaves the bracket (AdaSplash-2 (zh) §2.2; AdaSplash-2 (ja)
 * §2.2) -- and a bit-packed block mask, 32 key blocks per 32-bit word,
 * lets the forward and backward skip all-zero key blocks (AdaSplash-2 (zh) §2.3;
 * AdaSplash-2 (ja) §2.3). Threshold, bins and bracket live on the x-scale above.
 *
 * Layout (all tensors contiguous, row-major):
 *   q, dout, dq            [batch, heads_q,  seqlen, head_dim]   dtype
 *   k, v, dk, dv           [batch, heads_kv, seqlen, head_dim]   dtype
 *   o                      [batch, heads_q,  seqlen, head_dim]   float32 (accumulated in
 *                          fp32 for both dtypes; cast it if a narrower type is wanted)
 *   tau, tau_h             [batch, heads_q,  seqlen]             float32
 *   hist_counts            [batch, heads_q,  seqlen, n_bins]     int32
 *   block_mask             [batch, heads_q,  Tr, W]              uint32
 *                          Tr = seqlen/block_q, Tc = seqlen/block_k, W = ceil(Tc/32);
 *                          bit J%32 of word J/32 of row I is set iff query tile I and key
 *                          block J hold a pair (i, j) with p_ij > 0; unused bits are 0.
 *   aux                    forward-to-backward context, entmax_attn_aux_bytes() bytes,
 *                          opaque to the caller (pass the forward's aux to the backward).
 * Grouped-query attention: query head h reads KV head h / (heads_q / heads_kv).
 *   slopes                 [heads_q] float32, optional (NULL = no position bias):
 *                          query head h adds -slopes[h] * |i - j| to s_ij before the
 *                          transform (ALiBi; slope 0 = a head without position encoding,
 *                          so NAPE -- half the heads without encoding, half ALiBi, AdaSplash-2
 *                          (it) §4 and (zh) §4.2 -- is one slopes array). Under the
 *                          causal mask |i - j| = i - j. Forward and backward must get the
 *                          same slopes.
 *
 * Ownership and execution: the caller allocates every buffer (device memory)
 * and the workspace; the library keeps no pointer after a call returns and
 * allocates no device memory. Work is enqueued on `stream` (HIP stream; NULL =
 * the null stream) and the calls return without synchronising. Results are
 * bitwise deterministic for identical inputs (no floating-point atomics).
 *
 * Errors: every argument is checked before anything is enqueued; on an argument
 * error no output is touched and a status != ENTMAX_OK is returned, with detail
 * text in entmax_last_error() (thread-local). A HIP launch error returns
 * ENTMAX_ERR_HIP; outputs are then undefined. Data values are not checked:
 * NaN and Inf propagate.
 */
#ifndef ENTMAX_ATTN_H
#define ENTMAX_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    ENTMAX_OK = 0,
    ENTMAX_ERR_NULL = 1,        /* a required pointer is NULL */
    ENTMAX_ERR_SHAPE = 2,       /* sizes negative, inconsistent or not divisible by the blocks */
    ENTMAX_ERR_ALPHA = 3,       /* alpha not in (1, 16], or not finite */
    ENTMAX_ERR_UNSUPPORTED = 4, /* a valid but unimplemented combination (dtype, head_dim, blocks, bins) */
    ENTMAX_ERR_ALIGN = 5,       /* a pointer is not aligned as required */
    ENTMAX_ERR_WORKSPACE = 6,   /* workspace NULL or smaller than the *_workspace_bytes() query */
    ENTMAX_ERR_HIP = 7          /* a HIP runtime call failed */
} entmax_status;

typedef enum { ENTMAX_F32 = 0, ENTMAX_BF16 = 1 } entmax_dtype;

typedef struct {
    int32_t batch, heads_q, heads_kv, seqlen, head_dim;  /* heads_q % heads_kv == 0 */
    int32_t dtype;        /* entmax_dtype: F32 (fp32 matrix cores) or BF16 (bf16 in, fp32 accumulate) */
    float alpha;          /* 1 < alpha <= 16 */
    int32_t causal;       /* 0: every key is valid; 1: key j is valid for query i iff j <= i */
    int32_t block_q;      /* Br, rows of a mask tile: 32, 64 or 128; seqlen % Br == 0 */
    int32_t block_k;      /* Bc, keys of a mask block: 32, 64 or 128; seqlen % Bc == 0 */
    int32_t n_bins;       /* B, histogram bins: 2, 4, 8 or 16 (bin width 1/B on the x-scale) */
    float scale;          /* score scale; 0 means 1/sqrt(head_dim) */
    int32_t max_iters;    /* cap on refinement passes; 0 means 8 for alpha <= 1.5, 12 for
                             1.5 < alpha <= 2, 30 for alpha > 2 (where a key sitting on the
                             root can stall the secant; those rows end at the cap or when
                             fp32 can no longer move tau); at most 30 */
    float tol;            /* alpha 1.5 and 2: stop when |step| <= tol * max(1, |tau|); 0 means
                             2^-20. Other alpha stop when |sum p - 1| <= 1e-4 min(1, |f'|)
                             at the evaluated tau, f' = -sum_j p_ij^(2-alpha) / (alpha - 1)
                             the slope of sum p in tau (tol unused there) */
    int32_t tau_init;     /* start of the refinement: 0 = the histogram bound tau_h and the
                             bracket [tau_h, tau_h + 1/B] (AdaSplash-2 (zh) §2.1-2.2, AdaSplash-2 (ja)
                             §2.1-2.2); 1 = no histogram, the plain bracket
                             [x_max - 1, x_max - n_valid^(1-alpha)] from its lower end (the
                             start the pages measure the histogram against, AdaSplash-2 (es) §4),
                             for ablation; max_iters 0 then means 15 (30 for alpha > 2) */
    int32_t dense;        /* 0 = skip all-zero key blocks (the method, AdaSplash-2 (zh) §2.3:
                             work O(|M|) instead of O(Tr x Tc)); 1 = ablation without
                             skipping: refinement, output and both backward kernels visit
                             every causally valid block and multiply it in full, and the
                             forward returns a block_mask with every valid bit set. tau, o,
                             aux and the gradients equal those of dense = 0 (the skipped
                             blocks hold only zero weights); only the time differs */
} entmax_attn_desc;

/* Supported: head_dim 64 or 128 (bf16 and fp32); seqlen <= 2^19 (and a multiple of both blocks). */

/* Bytes of workspace the forward / backward need for `desc` (0 if desc is invalid). */
size_t entmax_attn_fwd_workspace_bytes(const entmax_attn_desc *desc);
size_t entmax_attn_bwd_workspace_bytes(const entmax_attn_desc *desc);
/* Bytes of the aux buffer (fp32 [b, hq, n, d]: o~_i = sum_j g_ij v_j / sum_j g_ij, the
 * support-weighted mean of V with g = p^(2-alpha), from which the backward forms
 * delta_i = dO_i . o~_i). */
size_t entmax_attn_aux_bytes(const entmax_attn_desc *desc);
/* 32-bit words of block_mask: batch * heads_q * Tr * W. */
size_t entmax_attn_mask_words(const entmax_attn_desc *desc);

/*
 * Forward (AdaSplash-2 (zh, ja, es) §2): per query row, one streaming pass over every
 * valid key block builds the B-bin histogram and tau_h; refinement passes over
 * the candidate key blocks find tau; a last pass over the blocks that hold a
 * non-zero weight forms o, aux and the exact block mask.
 * Required: q, k, v, o, tau, block_mask, aux (16-byte aligned; tau and mask 4-byte).
 * Optional (NULL to skip): slopes (position bias, 4-byte aligned, device memory);
 * hist_counts and tau_h (the histogram stage's output,
 * a test hook), stats (device uint64[32], accumulated, never cleared by the library:
 * stats[p] for p = 1..max_iters counts query rows whose refinement stopped after p
 * passes, stats[max_iters + 1] rows that hit the cap, except that rows with 16 or more
 * passes (or capped at 16 or more) all count in stats[16]; stats[20] key sub-blocks
 * (32 keys x 32 rows) scored by the histogram pass, stats[21] by refinement passes,
 * stats[22] by the output pass with a non-zero weight, stats[23] sub-blocks that the
 * histogram pass marked as candidates).
 * workspace: at least entmax_attn_fwd_workspace_bytes(desc) bytes, 256-byte aligned.
 */
entmax_status entmax_attn_fwd(const entmax_attn_desc *desc,
                              const void *q, const void *k, const void *v, const float *slopes,
                              void *o, float *tau, uint32_t *block_mask, void *aux,
                              int32_t *hist_counts, float *tau_h, uint64_t *stats,
                              void *workspace, size_t workspace_bytes, void *stream);

/*
 * Backward: the exact gradient of alpha-entmax attention (the pages state only
 * that the backward also skips zero blocks, AdaSplash-2 (zh) §2.3). With
 * g_ij = [x_ij - tau_i]_+^(1/(alpha-1) - 1), dP_ij = dO_i . v_j, delta_i = dO_i . o~_i:
 *   dS_ij = g_ij (dP_ij - delta_i),  dq_i = scale sum_j dS_ij k_j,
 *   dk_j = scale sum_i dS_ij q_i,    dv_j = sum_i p_ij dO_i  (summed over the GQA group).
 * Only key blocks set in block_mask are visited. tau, block_mask and aux must come from
 * entmax_attn_fwd with the same desc, inputs and slopes (the bias enters x, not the
 * gradient formulas; NULL = none). dq, dk, dv are overwritten.
 * Alignment: every tensor 16 bytes (tau included), block_mask 4 bytes.
 * workspace: at least entmax_attn_bwd_workspace_bytes(desc) bytes, 256-byte aligned.
 */
entmax_status entmax_attn_bwd(const entmax_attn_desc *desc,
                              const void *q, const void *k, const void *v, const void *dout,
                              const float *slopes, const float *tau, const uint32_t *block_mask,
                              const void *aux,
                              void *dq, void *dk, void *dv,
                              void *workspace, size_t workspace_bytes, void *stream);

/*
 * Decode: one new query row per (sequence, query head) against a KV cache, forward only
 * (the pages leave inference to future work, AdaSplash-2 (ja) §5; DashAttention decodes
 * incrementally on the same primitives, DashAttention (it)). The query follows the cached keys, so
 * keys 0..len_b-1 of sequence b are all valid and, with a position bias, key j sits at
 * distance len_b - 1 - j. The threshold is found as in the forward: the B-bin histogram
 * of the row's scores gives tau_h (Proposition 1), the same hybrid solver refines it, and
 * o = sum_j p_j v_j. The result equals the last row of a causal forward over the cache.
 *
 * desc: batch, heads_q, heads_kv (heads_q / heads_kv <= 16), seqlen = cache capacity n_ctx
 *       (1..2^19, any value), head_dim, dtype, alpha, n_bins, scale, max_iters, tol and
 *       tau_init as for the forward; causal, block_q and block_k are not used.
 * q        [batch, heads_q, head_dim] dtype             k_cache, v_cache [batch, heads_kv, n_ctx, head_dim] dtype
 * lengths  [batch] int32, device, optional (NULL = n_ctx): valid keys of each sequence,
 *          values are clamped to 1..n_ctx
 * slopes   [heads_q] float32, device, optional: position bias as in the forward
 * o        [batch, heads_q, head_dim] float32            tau, tau_h [batch, heads_q] float32
 * hist_counts [batch, heads_q, n_bins] int32, optional; tau_h optional
 * Alignment: q, k_cache, v_cache, o 16 bytes; tau, lengths, slopes, tau_h, counts 4 bytes.
 * workspace: at least entmax_attn_decode_workspace_bytes(desc) bytes, 256-byte aligned
 * (the score rows, fp32 [batch, heads_q, n_ctx], and per-split partial results).
 */
size_t entmax_attn_decode_workspace_bytes(const entmax_attn_desc *desc);
entmax_status entmax_attn_decode(const entmax_attn_desc *desc,
                                 const void *q, const void *k_cache, const void *v_cache,
                                 const int32_t *lengths, const float *slopes,
                                 float *o, float *tau, int32_t *hist_counts, float *tau_h,
                                 void *workspace, size_t workspace_bytes, void *stream);

/*
 * Decode without allocation, for callers that cannot allocate device memory or pass a
 * workspace: code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc. Same arguments, results and checks as entmax_attn_decode, minus the
 * workspace: the library uses a static scratch of ENTMAX_DECODE_SCRATCH_BYTES bytes per
 * device instead (allocated when the library's code is loaded on a device, held until the
 * process ends; its address is looked up on the first call on each device). This call
 * makes no hipMalloc, hipFree or allocating library call.
 * Limit: problems whose entmax_attn_decode_workspace_bytes() exceeds the scratch size
 * (about 16 MB of fp32 scores for 32 query heads x 128K cached keys, plus partial sums)
 * return ENTMAX_ERR_WORKSPACE before anything is enqueued.
 * Sharing: every call on a device uses that device's one scratch, and its contents are
 * left from the last call (nothing in it is read before it is written within a call).
 * Calls that overlap on one device -- on different streams or host threads without
 * ordering between them -- race on the scratch; serialise them (one stream, or events).
 * The stream must belong to the current device.
 */
#define ENTMAX_DECODE_SCRATCH_BYTES ((size_t)32 << 20)
entmax_status entmax_attn_decode_noalloc(const entmax_attn_desc *desc,
                                         const void *q, const void *k_cache, const void *v_cache,
                                         const int32_t *lengths, const float *slopes,
                                         float *o, float *tau, int32_t *hist_counts, float *tau_h,
                                         void *stream);

const char *entmax_status_string(entmax_status s);
const char *entmax_last_error(void);

/*
 * Kernel timing. While enabled, every kernel launch of this library is bracketed by
 * two hipEvents recorded on the launch stream. entmax_attn_profile_read waits for the
 * recorded events, writes up to max_entries per-kernel totals since the last read
 * (name, summed milliseconds, launch count), sets *n_entries and clears the record.
 */
typedef struct {
    char name[32];
    double total_ms;
    int64_t launches;
} entmax_kernel_time;

entmax_status entmax_attn_profile(int enable);
entmax_status entmax_attn_profile_read(entmax_kernel_time *out, int max_entries, int *n_entries);

#ifdef __cplusplus
}
#endif
#endif /* ENTMAX_ATTN_H */
