/*
 * dash_attn.h -- C ABI of the DashAttention forward (stages 1 and 2) in the alpha-entmax
 * attention library for AMD MI355X (gfx950).
 *
 * The operation (DashAttention page, Italian summary, "Metodologia", stages 1-2): the
 * keys are cut into chunks of C; stage 0 (outside this call) gives one summary vector per
 * chunk. Query row i of head h (KV group g = h / (heads_q / heads_kv)) has
 * m_i = floor(i / C) complete chunks before its own.
 *
 *   Stage 1, routing: zbar_c = gamma * scale * q_i . ksum_c for c < m_i;
 *     w_h(i, .) = alpha-entmax(zbar) (threshold tau on the x-scale (alpha - 1) zbar, found
 *     by the same safeguarded hybrid solver as the attention forward, started from the
 *     bracket [x_max - 1, x_max - m_i^(1-alpha)]); the heads of a KV group average their
 *     weights, wbar(g, i, c) = mean_h w_h(i, c), and share the support {c : wbar > 0}.
 *   Stage 2, prior-induced sparse softmax: the softmax whose KL reference is the prior is
 *     softmax(s + log prior). Keys of routed chunks get s_ij = scale q_i . k_j +
 *     sigma ln wbar(g, i, c(j)); the diagonal branch (the query's own chunk, keys
 *     m_i C .. i) gets s_ij = scale q_i . k_j; every other key is masked.
 *     o_i = sum_j softmax(s_i)_j v_j,  lse_i = ln sum_j exp(s_ij).
 *   Rows with m_i = 0 route nothing (tau reported as 0) and attend their diagonal keys.
 *
 * Layout (contiguous, row-major):
 *   q                  [batch, heads_q,  seqlen, head_dim]   dtype
 *   k, v               [batch, heads_kv, seqlen, head_dim]   dtype
 *   k_summary          [batch, heads_kv, n_chunks, head_dim] dtype, n_chunks = seqlen / chunk
 *   o                  [batch, heads_q,  seqlen, head_dim]   float32
 *   lse, route_tau     [batch, heads_q,  seqlen]             float32
 *   route_w            [batch, heads_kv, n_chunks, seqlen]   float32, chunk-major: wbar of
 *                      (chunk c, row i) at c * seqlen + i; 0 for every chunk a row does not route
 *   chunk_mask         [batch, heads_kv, seqlen / 64, ceil(n_chunks / 32)] uint32: bit c % 32
 *                      of word c / 32 of query tile t (rows 64 t .. 64 t + 63) is set iff a
 *                      row of the tile routes chunk c (wbar > 0); unused bits are 0.
 *
 * Ownership, streams and errors as in entmax_attn.h: the caller allocates every buffer
 * (device memory) and the workspace, work is enqueued on `stream`, arguments are checked
 * before anything is enqueued (status != ENTMAX_OK and entmax_last_error() text on an
 * error; no output touched), results are bitwise deterministic.
 */
#ifndef DASH_ATTN_H
#define DASH_ATTN_H

#include "entmax_attn.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef struct {
    int32_t batch, heads_q, heads_kv, seqlen, head_dim;  /* heads_q % heads_kv == 0 */
    int32_t dtype;        /* entmax_dtype */
    int32_t chunk;        /* C: keys per chunk, 64, 128 or 256; seqlen % chunk == 0 and
                             seqlen / chunk <= 256 */
    float route_alpha;    /* alpha of the routing entmax, in (1, 16] */
    float gamma;          /* routing logit multiplier, > 0; 0 means 1 */
    float sigma;          /* prior strength, >= 0 (0: uniform over the active keys) */
    float scale;          /* score scale; 0 means 1/sqrt(head_dim) */
    int32_t max_iters;    /* routing solver pass cap, 0 (= 15, 30 for alpha > 2) or 1..30 */
    float tol;            /* routing solver tolerance as in entmax_attn_desc; 0 means 2^-20 */
} entmax_dash_desc;

/* Supported: head_dim 64 or 128 (bf16 and fp32); seqlen a multiple of chunk, at most
 * 256 chunks (64K tokens at chunk 256). */

/* Bytes of workspace for `desc` (the fragment-major copies of K and V); 0 if invalid. */
size_t entmax_dash_fwd_workspace_bytes(const entmax_dash_desc *desc);
/* 32-bit words of chunk_mask: batch * heads_kv * (seqlen / 64) * ceil(n_chunks / 32). */
size_t entmax_dash_mask_words(const entmax_dash_desc *desc);

/*
 * Forward of stages 1 and 2. Required: q, k, v, k_summary, o, route_w, chunk_mask.
 * Optional (NULL to skip): lse, route_tau. Alignment: q, k, v, k_summary, o 16 bytes;
 * lse, route_tau, route_w, chunk_mask 4 bytes. workspace: at least
 * entmax_dash_fwd_workspace_bytes(desc) bytes, 256-byte aligned.
 */
entmax_status entmax_dash_fwd(const entmax_dash_desc *desc,
                              const void *q, const void *k, const void *v, const void *k_summary,
                              float *o, float *lse, float *route_tau, float *route_w,
                              uint32_t *chunk_mask,
                              void *workspace, size_t workspace_bytes, void *stream);

/*
 * Backward of stages 1 and 2 (DashAttention page, Italian summary, stage 1: the routing is
 * differentiable, so the gradients reach the chunk summaries). Given dO = dL/do, returns
 *   dq, dk, dv   the gradients of q, k, v (stage 2 is softmax attention with the prior
 *                sigma ln wbar as an additive term on routed chunks; dq also carries the
 *                routing's share, below);
 *   dk_summary   [batch, heads_kv, n_chunks, head_dim], the gradient of the summaries.
 * The prior term of chunk c in row i gets s_ic = sum over the chunk's keys of
 * dS_ij = p_ij (dO_i . v_j - dO_i . o_i); the group's routing weights get
 * dwbar(c) = sigma / wbar(c) * sum over the group's heads of s_ic, each head's weights
 * dwbar / G, and through the alpha-entmax Jacobian diag(g) - g g^T / sum g, with
 * g = [x - tau]_+^(1/(alpha-1) - 1) at the forward's tau, the logits get
 * du = g (dw - (g . dw) / sum g); then dq += gamma scale du . k_summary and
 * dk_summary(c) = gamma scale sum over the group's heads and rows of du(c) q. Chunks outside
 * a row's support carry no gradient.
 * Inputs: q, k, v, k_summary and the forward's outputs o, lse, route_tau, route_w and
 * chunk_mask (all required), dout [batch, heads_q, seqlen, head_dim] in dtype. Outputs
 * dq, dk, dv, dk_summary in dtype. Alignment: 16 bytes (route_tau, chunk_mask 4 bytes).
 * workspace: at least entmax_dash_bwd_workspace_bytes(desc) bytes, 256-byte aligned.
 * Results are bitwise deterministic (fixed reduction orders, no atomics).
 */
size_t entmax_dash_bwd_workspace_bytes(const entmax_dash_desc *desc);
entmax_status entmax_dash_bwd(const entmax_dash_desc *desc,
                              const void *q, const void *k, const void *v, const void *k_summary,
                              const float *o, const float *lse, const float *route_tau,
                              const float *route_w, const uint32_t *chunk_mask, const void *dout,
                              void *dq, void *dk, void *dv, void *dk_summary,
                              void *workspace, size_t workspace_bytes, void *stream);

#ifdef __cplusplus
}
#endif
#endif /* DASH_ATTN_H */
