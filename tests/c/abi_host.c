/* The C ABI used from plain C99, with no GPU: the header compiles as C,
 * the library links and loads, sizing answers match direct counts, and bad
 * arguments are refused with an error code and a message before any device
 * work. Prints "ok" and exits 0 when every check holds. */
#include <math.h>
#include <stdio.h>
#include <string.h>

#include "fp_prefill.h"

static int failures = 0;

#define CHECK(cond)                                                              \
    do {                                                                         \
        if (!(cond)) {                                                           \
            printf("FAILED line %d: %s (last error: %s)\n", __LINE__, #cond,   \
                   fp_last_error());                                             \
            ++failures;                                                          \
        }                                                                        \
    } while (0)

static fp_problem fixed_problem(int S, int Hq, int Hkv, int block) {
    fp_problem p;
    memset(&p, 0, sizeof(p));
    p.batch = 1;
    p.seqlen = S;
    p.num_q_heads = Hq;
    p.num_kv_heads = Hkv;
    p.head_dim = 128;
    p.block = block;
    p.dtype = FP_DTYPE_BF16;
    p.softmax_scale = 0.f;
    p.q_stride[0] = (int64_t)S * Hq * 128; p.q_stride[1] = Hq * 128; p.q_stride[2] = 128;
    p.k_stride[0] = (int64_t)S * Hkv * 128; p.k_stride[1] = Hkv * 128; p.k_stride[2] = 128;
    memcpy(p.v_stride, p.k_stride, sizeof(p.k_stride));
    memcpy(p.o_stride, p.q_stride, sizeof(p.q_stride));
    return p;
}

int main(void) {
    const char* v = fp_version();
    CHECK(v != NULL && strlen(v) > 0);

    /* S = 2048, 64-token blocks: 32 query blocks, one KV head */
    fp_problem p = fixed_problem(2048, 4, 1, 64);
    CHECK(fp_num_rows(&p) == 32);
    CHECK(fp_max_nnz(&p) == 32 * 33 / 2);
    CHECK(fp_workspace_size(&p) > 0);
    CHECK(fp_prefill_workspace_size(&p) > 0);
    /* a ragged last block and 8 KV heads */
    p = fixed_problem(1000, 32, 8, 128);
    CHECK(fp_num_rows(&p) == 8 * 8);
    CHECK(fp_max_nnz(&p) == 8 * (8 * 9 / 2));

    /* unsupported shapes: code and message */
    p = fixed_problem(2048, 4, 1, 96);
    CHECK(fp_num_rows(&p) == FP_ERR_UNSUPPORTED && strlen(fp_last_error()) > 0);
    p = fixed_problem(2048, 4, 1, 64);
    p.head_dim = 64;
    CHECK(fp_num_rows(&p) == FP_ERR_UNSUPPORTED);
    p = fixed_problem(2048, 6, 4, 64);
    CHECK(fp_num_rows(&p) == FP_ERR_INVALID);

    /* invalid arguments are refused before any device work (no GPU here) */
    p = fixed_problem(2048, 4, 1, 64);
    float dummy[4];
    CHECK(fp_block_scores(&p, NULL, dummy, dummy, NULL, NULL, NULL, dummy, dummy, dummy, dummy, NULL) ==
          FP_ERR_INVALID);
    int32_t ibuf[4];
    CHECK(fp_select_blocks(&p, dummy, nanf(""), ibuf, ibuf, 1 << 20, NULL, dummy, 1 << 30, NULL) ==
          FP_ERR_INVALID);
    CHECK(fp_select_blocks(&p, dummy, 1.f, ibuf, ibuf, 10, NULL, dummy, 1 << 30, NULL) == FP_ERR_CAPACITY);

    /* paged varlen sizing: two sequences with cached prefixes, 64-token blocks */
    fp_varlen_problem vp;
    memset(&vp, 0, sizeof(vp));
    vp.num_seqs = 2;
    vp.num_q_heads = 4;
    vp.num_kv_heads = 2;
    vp.head_dim = 128;
    vp.block = 64;
    vp.page_size = 16;
    vp.dtype = FP_DTYPE_BF16;
    vp.max_pages_per_seq = 16;
    vp.q_stride[0] = 4 * 128; vp.q_stride[1] = 128;
    vp.kv_stride[0] = 16 * 2 * 128; vp.kv_stride[1] = 2 * 128; vp.kv_stride[2] = 128;
    vp.o_stride[0] = 4 * 128; vp.o_stride[1] = 128;
    const int32_t cu[3] = {0, 100, 160};     /* new rows: 100 and 60 */
    const int32_t lk[2] = {200, 60};         /* prefixes 100 and 0 */
    /* sequence 0: query blocks 1..3 (rows 100..199), sequence 1: blocks 0..0 */
    CHECK(fp_varlen_num_rows(&vp, cu, lk) == 2 * (3 + 1));
    CHECK(fp_varlen_max_nnz(&vp, cu, lk) == 2 * ((2 + 3 + 4) + 1));
    CHECK(fp_varlen_workspace_size(&vp, cu, lk) > 0);
    const int32_t bad_lk[2] = {50, 60};      /* fewer keys than new rows */
    CHECK(fp_varlen_num_rows(&vp, cu, bad_lk) == FP_ERR_INVALID);
    vp.page_size = 48;
    CHECK(fp_varlen_num_rows(&vp, cu, lk) == FP_ERR_UNSUPPORTED);

    /* every other entry point refuses bad arguments before any device work */
    p = fixed_problem(2048, 4, 1, 64);
    char* fake = (char*)dummy;               /* never dereferenced: the checks fail first */
    CHECK(fp_estimate_select_workspace_size(&p) > 0);
    CHECK(fp_estimate_select(&p, fake, fake, fake, NULL, NULL, NULL, nanf(""), dummy, dummy, dummy, ibuf, ibuf,
                             1 << 20, ibuf, fake, 1 << 30, NULL) == FP_ERR_INVALID);
    CHECK(fp_estimate_select(&p, fake, fake, fake, NULL, NULL, NULL, 1.f, dummy, dummy, dummy, ibuf, ibuf, 10, ibuf,
                             fake, 1 << 30, NULL) == FP_ERR_CAPACITY);
    CHECK(fp_sparse_prefill(&p, NULL, fake, fake, NULL, NULL, NULL, dummy, dummy, ibuf, ibuf, NULL, fake, NULL,
                            fake, 1 << 30, NULL) == FP_ERR_INVALID);
    CHECK(fp_sparse_prefill(&p, fake, fake, fake, NULL, NULL, NULL, dummy, dummy, ibuf, ibuf, NULL, fake, NULL,
                            fake, 1, NULL) == FP_ERR_CAPACITY);
    CHECK(fp_dense_prefill(&p, fake, NULL, fake, NULL, NULL, NULL, fake, NULL, NULL) == FP_ERR_INVALID);
    /* the block-score correction has its own entry point, and only it takes scores */
    CHECK(fp_sparse_prefill_scored(&p, fake, fake, fake, NULL, NULL, NULL, dummy, dummy, ibuf, ibuf, NULL, fake,
                                   NULL, fake, 1 << 30, NULL) == FP_ERR_INVALID);
    p.variant = FP_VARIANT_BLOCK_SCORE;
    CHECK(fp_sparse_prefill(&p, fake, fake, fake, NULL, NULL, NULL, dummy, dummy, ibuf, ibuf, NULL, fake, NULL,
                            fake, 1 << 30, NULL) == FP_ERR_INVALID);
    CHECK(fp_sparse_prefill_noalloc(&p, fake, fake, fake, NULL, NULL, NULL, dummy, dummy, ibuf, ibuf, NULL, fake,
                                    NULL, NULL) == FP_ERR_INVALID);
    /* the allocation-free entry point refuses problems beyond its static scratch */
    p = fixed_problem(1 << 20, 32, 8, 64);
    CHECK(fp_num_rows(&p) > 0);
    CHECK(fp_sparse_prefill_noalloc(&p, fake, fake, fake, NULL, NULL, NULL, dummy, dummy, ibuf, ibuf, NULL, fake,
                                    NULL, NULL) == FP_ERR_CAPACITY);
    /* paged: NaN tau, a short workspace, a missing pooled-KV cache */
    vp.page_size = 16;
    const int64_t vnnz = fp_varlen_max_nnz(&vp, cu, lk), vws = fp_varlen_workspace_size(&vp, cu, lk);
    CHECK(fp_sparse_prefill_paged(&vp, fake, cu, lk, fake, fake, ibuf, NULL, NULL, NULL, nanf(""), ibuf, ibuf, vnnz,
                                  fake, NULL, fake, (size_t)vws, NULL) == FP_ERR_INVALID);
    CHECK(fp_sparse_prefill_paged(&vp, fake, cu, lk, fake, fake, ibuf, NULL, NULL, NULL, 1.f, ibuf, ibuf, vnnz,
                                  fake, NULL, fake, (size_t)vws - 1, NULL) == FP_ERR_CAPACITY);
    CHECK(fp_sparse_prefill_paged_cached(&vp, fake, cu, lk, fake, fake, ibuf, NULL, NULL, NULL, NULL, dummy, 1.f,
                                         ibuf, ibuf, vnnz, fake, NULL, fake, (size_t)vws, NULL) == FP_ERR_INVALID);

    if (failures) return 1;
    printf("ok\n");
    return 0;
}
