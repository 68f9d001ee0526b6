/* Plain C use of the library's C ABI, without Python and without a GPU: descriptor set-up,
 * workspace and buffer size queries, argument errors (every check runs before any HIP call)
 * and the empty-problem no-op. Built and run by tests/test_abi.py with gcc. Exit status 0
 * when every expectation holds; the first failure is printed. */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "dash_attn.h"
#include "entmax_attn.h"

#define EXPECT(cond)                                                          \
    do {                                                                      \
        if (!(cond)) {                                                        \
            printf("FAILED line %d: %s (%s)\n", __LINE__, #cond, entmax_last_error()); \
            return 1;                                                         \
        }                                                                     \
    } while (0)

static entmax_attn_desc attn_desc(void) {
    entmax_attn_desc d;
    memset(&d, 0, sizeof d);
    d.batch = 2; d.heads_q = 8; d.heads_kv = 2; d.seqlen = 4096; d.head_dim = 64;
    d.dtype = ENTMAX_BF16; d.alpha = 1.5f; d.causal = 1; d.block_q = 64; d.block_k = 64;
    d.n_bins = 16;
    return d;
}

int main(void) {
    entmax_attn_desc d = attn_desc();
    /* sizes: the mask has ceil(Tc / 32) words per query tile and head; aux is o~ in fp32 */
    EXPECT(entmax_attn_mask_words(&d) == (size_t)2 * 8 * 64 * 2);
    EXPECT(entmax_attn_aux_bytes(&d) == (size_t)2 * 8 * 4096 * 64 * 4);
    EXPECT(entmax_attn_fwd_workspace_bytes(&d) > 0);
    EXPECT(entmax_attn_bwd_workspace_bytes(&d) > 0);
    EXPECT(entmax_attn_decode_workspace_bytes(&d) > 0);

    /* argument errors, reported before anything is enqueued */
    void *p = (void *)(uintptr_t)4096;
    size_t big = (size_t)1 << 40;
    entmax_attn_desc bad = d;
    bad.alpha = 1.0f;
    EXPECT(entmax_attn_fwd(&bad, p, p, p, NULL, p, p, p, p, NULL, NULL, NULL, p, big, NULL) == ENTMAX_ERR_ALPHA);
    EXPECT(strlen(entmax_last_error()) > 0);
    bad = d;
    bad.head_dim = 96;
    EXPECT(entmax_attn_fwd(&bad, p, p, p, NULL, p, p, p, p, NULL, NULL, NULL, p, big, NULL) == ENTMAX_ERR_UNSUPPORTED);
    bad = d;
    bad.seqlen = 4000;
    EXPECT(entmax_attn_bwd(&bad, p, p, p, p, NULL, p, p, p, p, p, p, p, big, NULL) == ENTMAX_ERR_SHAPE);
    EXPECT(entmax_attn_fwd(&d, NULL, p, p, NULL, p, p, p, p, NULL, NULL, NULL, p, big, NULL) == ENTMAX_ERR_NULL);
    EXPECT(entmax_attn_fwd(&d, (void *)(uintptr_t)4098, p, p, NULL, p, p, p, p, NULL, NULL, NULL, p, big, NULL) ==
           ENTMAX_ERR_ALIGN);
    EXPECT(entmax_attn_fwd(&d, p, p, p, NULL, p, p, p, p, NULL, NULL, NULL, p, 16, NULL) == ENTMAX_ERR_WORKSPACE);
    EXPECT(strcmp(entmax_status_string(ENTMAX_ERR_WORKSPACE), "workspace missing or too small") == 0);

    /* an empty problem is a no-op that touches nothing */
    entmax_attn_desc empty = d;
    empty.seqlen = 0;
    EXPECT(entmax_attn_fwd(&empty, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, 0, NULL) ==
           ENTMAX_OK);

    /* DashAttention: 4096 tokens in chunks of 64, GQA 4 */
    entmax_dash_desc dd;
    memset(&dd, 0, sizeof dd);
    dd.batch = 1; dd.heads_q = 8; dd.heads_kv = 2; dd.seqlen = 4096; dd.head_dim = 128;
    dd.dtype = ENTMAX_BF16; dd.chunk = 64; dd.route_alpha = 1.5f; dd.gamma = 8.0f; dd.sigma = 1.0f;
    EXPECT(entmax_dash_mask_words(&dd) == (size_t)1 * 2 * 64 * 2);
    EXPECT(entmax_dash_fwd_workspace_bytes(&dd) == (size_t)2 * 1 * 2 * 4096 * 128 * 2);
    entmax_dash_desc dbad = dd;
    dbad.chunk = 96;
    EXPECT(entmax_dash_fwd(&dbad, p, p, p, p, p, NULL, NULL, p, p, p, big, NULL) == ENTMAX_ERR_UNSUPPORTED);
    EXPECT(entmax_dash_fwd(&dd, p, p, p, NULL, p, NULL, NULL, p, p, p, big, NULL) == ENTMAX_ERR_NULL);
    /* the backward: a workspace of at least the fp32 dQ, the per-sub-block dS sums and the
       routing-logit gradient; every tensor required; the forward's argument errors */
    const size_t bws = entmax_dash_bwd_workspace_bytes(&dd);
    EXPECT(bws >= (size_t)8 * 4096 * 128 * 4 + (size_t)8 * 128 * 4096 * 4 + (size_t)8 * 64 * 4096 * 4);
    EXPECT(entmax_dash_bwd_workspace_bytes(&dbad) == 0);
    EXPECT(entmax_dash_bwd(&dbad, p, p, p, p, p, p, p, p, p, p, p, p, p, p, p, big, NULL) == ENTMAX_ERR_UNSUPPORTED);
    EXPECT(entmax_dash_bwd(&dd, p, p, p, p, p, p, NULL, p, p, p, p, p, p, p, p, big, NULL) == ENTMAX_ERR_NULL);
    EXPECT(entmax_dash_bwd(&dd, p, p, p, p, p, p, p, p, p, p, p, p, p, p, p, bws - 1, NULL) == ENTMAX_ERR_WORKSPACE);

    printf("abi_check: ok\n");
    return 0;
}
