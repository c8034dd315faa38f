/* The whole fixed-shape path driven from plain C99 through the C ABI:
 * device buffers from hipMalloc, a stream of its own (default priority),
 * fp_block_scores -> fp_select_blocks -> fp_sparse_prefill, results copied
 * back and written as raw files for comparison with the Python binding.
 *
 *   abi_run DIR         reads DIR/meta.txt ("S Hq Hkv block tau") and DIR/q.bin,
 *                       k.bin, v.bin (bf16, contiguous [S, H, 128]); writes
 *                       DIR/o.bin (bf16 [S, Hq, 128]), lse.bin (fp32 [Hq, S]),
 *                       row_ptr.bin, col_idx.bin (int32, nnz entries), sched.bin.
 *   abi_run paged DIR   fp_sparse_prefill_paged on a bf16 paged batch: reads
 *                       DIR/meta.txt ("num_seqs Hq Hkv block page_size n_pages
 *                       max_pages tau"), cu_seqlens_q.bin, seqlens_k.bin (int32),
 *                       q.bin (bf16 [sum q, Hq, 128]), k_cache.bin, v_cache.bin
 *                       (bf16 [n_pages, page_size, Hkv, 128]), block_table.bin
 *                       (int32 [num_seqs, max_pages]); writes o.bin, lse.bin
 *                       (fp32 [Hq, sum q]), row_ptr.bin, col_idx.bin.
 * Prints "ok" and exits 0 on success; any error is printed and exits 1. */
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "fp_prefill.h"

#define HIP_OK(call)                                                                 \
    do {                                                                             \
        hipError_t e_ = (call);                                                      \
        if (e_ != hipSuccess) {                                                      \
            printf("HIP error %s at line %d: %s\n", hipGetErrorString(e_), __LINE__, \
                   #call);                                                           \
            exit(1);                                                                 \
        }                                                                            \
    } while (0)

#define FP_OK_(call)                                                                            \
    do {                                                                                        \
        int r_ = (call);                                                                        \
        if (r_ != FP_OK) {                                                                      \
            printf("fp error %d at line %d: %s: %s\n", r_, __LINE__, #call, fp_last_error()); \
            exit(1);                                                                            \
        }                                                                                       \
    } while (0)

static char path_buf[4096];

static const char* path(const char* dir, const char* name) {
    snprintf(path_buf, sizeof(path_buf), "%s/%s", dir, name);
    return path_buf;
}

static void* read_file(const char* dir, const char* name, size_t bytes) {
    FILE* f = fopen(path(dir, name), "rb");
    if (!f) { printf("cannot open %s\n", path_buf); exit(1); }
    void* h = malloc(bytes ? bytes : 1);
    if (!h || fread(h, 1, bytes, f) != bytes) { printf("short read %s\n", path_buf); exit(1); }
    fclose(f);
    return h;
}

static void write_file(const char* dir, const char* name, const void* h, size_t bytes) {
    FILE* f = fopen(path(dir, name), "wb");
    if (!f || fwrite(h, 1, bytes, f) != bytes) { printf("cannot write %s\n", path_buf); exit(1); }
    fclose(f);
}

static void* to_device(const void* h, size_t bytes) {
    void* d = NULL;
    HIP_OK(hipMalloc(&d, bytes ? bytes : 1));
    if (bytes) HIP_OK(hipMemcpy(d, h, bytes, hipMemcpyHostToDevice));
    return d;
}

static void* device(size_t bytes) {
    void* d = NULL;
    HIP_OK(hipMalloc(&d, bytes ? bytes : 1));
    return d;
}

static int run_paged(const char* dir) {
    int nseq, Hq, Hkv, block, page, npages, maxp;
    float tau;
    FILE* mf = fopen(path(dir, "meta.txt"), "r");
    if (!mf || fscanf(mf, "%d %d %d %d %d %d %d %f", &nseq, &Hq, &Hkv, &block, &page, &npages, &maxp, &tau) != 8) {
        printf("bad meta.txt\n");
        return 1;
    }
    fclose(mf);
    int32_t* cu = (int32_t*)read_file(dir, "cu_seqlens_q.bin", (size_t)(nseq + 1) * 4);
    int32_t* lk = (int32_t*)read_file(dir, "seqlens_k.bin", (size_t)nseq * 4);
    const int64_t nq = cu[nseq];

    fp_varlen_problem p;
    memset(&p, 0, sizeof(p));
    p.num_seqs = nseq;
    p.num_q_heads = Hq;
    p.num_kv_heads = Hkv;
    p.head_dim = 128;
    p.block = block;
    p.page_size = page;
    p.dtype = FP_DTYPE_BF16;
    p.max_pages_per_seq = maxp;
    p.q_stride[0] = Hq * 128; p.q_stride[1] = 128;
    p.kv_stride[0] = (int64_t)page * Hkv * 128; p.kv_stride[1] = Hkv * 128; p.kv_stride[2] = 128;
    p.o_stride[0] = Hq * 128; p.o_stride[1] = 128;
    const int64_t rows = fp_varlen_num_rows(&p, cu, lk), cap = fp_varlen_max_nnz(&p, cu, lk);
    const int64_t wsb = fp_varlen_workspace_size(&p, cu, lk);
    if (rows < 0 || cap < 0 || wsb < 0) { printf("sizing: %s\n", fp_last_error()); return 1; }

    const size_t qb = (size_t)nq * Hq * 128 * 2, cb = (size_t)npages * page * Hkv * 128 * 2;
    const size_t btb = (size_t)nseq * maxp * 4;
    void* hq = read_file(dir, "q.bin", qb);
    void* hk = read_file(dir, "k_cache.bin", cb);
    void* hv = read_file(dir, "v_cache.bin", cb);
    void* hbt = read_file(dir, "block_table.bin", btb);
    void* dq = to_device(hq, qb);
    void* dk = to_device(hk, cb);
    void* dv = to_device(hv, cb);
    void* dbt = to_device(hbt, btb);
    int32_t* row_ptr = (int32_t*)device((size_t)(rows + 1) * 4);
    int32_t* col_idx = (int32_t*)device((size_t)(cap > 0 ? cap : 1) * 4);
    void* o = device(qb);
    float* lse = (float*)device((size_t)Hq * nq * 4);
    void* ws = device((size_t)wsb);

    hipStream_t st;
    HIP_OK(hipStreamCreate(&st));
    FP_OK_(fp_sparse_prefill_paged(&p, dq, cu, lk, dk, dv, (const int32_t*)dbt, NULL, NULL, NULL, tau, row_ptr,
                                   col_idx, cap, o, lse, ws, (size_t)wsb, st));
    HIP_OK(hipStreamSynchronize(st));

    int32_t* h_rp = (int32_t*)malloc((size_t)(rows + 1) * 4);
    HIP_OK(hipMemcpy(h_rp, row_ptr, (size_t)(rows + 1) * 4, hipMemcpyDeviceToHost));
    const int32_t nnz = h_rp[rows];
    if (nnz < rows || nnz > cap) { printf("bad nnz %d\n", nnz); return 1; }
    int32_t* h_ci = (int32_t*)malloc((size_t)(nnz > 0 ? nnz : 1) * 4);
    void* h_o = malloc(qb ? qb : 1);
    float* h_lse = (float*)malloc((size_t)Hq * nq * 4 + 4);
    HIP_OK(hipMemcpy(h_ci, col_idx, (size_t)nnz * 4, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(h_o, o, qb, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(h_lse, lse, (size_t)Hq * nq * 4, hipMemcpyDeviceToHost));
    write_file(dir, "row_ptr.bin", h_rp, (size_t)(rows + 1) * 4);
    write_file(dir, "col_idx.bin", h_ci, (size_t)nnz * 4);
    write_file(dir, "o.bin", h_o, qb);
    write_file(dir, "lse.bin", h_lse, (size_t)Hq * nq * 4);

    HIP_OK(hipStreamDestroy(st));
    void* bufs[] = {dq, dk, dv, dbt, row_ptr, col_idx, o, lse, ws};
    for (size_t i = 0; i < sizeof(bufs) / sizeof(bufs[0]); ++i) HIP_OK(hipFree(bufs[i]));
    free(cu); free(lk); free(hq); free(hk); free(hv); free(hbt); free(h_rp); free(h_ci); free(h_o); free(h_lse);
    printf("ok nnz=%d\n", nnz);
    return 0;
}

int main(int argc, char** argv) {
    if (argc == 3 && strcmp(argv[1], "paged") == 0) return run_paged(argv[2]);
    if (argc != 2) { printf("usage: abi_run DIR | abi_run paged DIR\n"); return 1; }
    const char* dir = argv[1];
    int S, Hq, Hkv, block;
    float tau;
    FILE* mf = fopen(path(dir, "meta.txt"), "r");
    if (!mf || fscanf(mf, "%d %d %d %d %f", &S, &Hq, &Hkv, &block, &tau) != 5) {
        printf("bad meta.txt\n");
        return 1;
    }
    fclose(mf);

    fp_problem p;
    memset(&p, 0, sizeof(p));
    p.batch = 1;
    p.seqlen = S;
    p.num_q_heads = Hq;
    p.num_kv_heads = Hkv;
    p.head_dim = 128;
    p.block = block;
    p.dtype = FP_DTYPE_BF16;
    p.q_stride[0] = (int64_t)S * Hq * 128; p.q_stride[1] = Hq * 128; p.q_stride[2] = 128;
    p.k_stride[0] = (int64_t)S * Hkv * 128; p.k_stride[1] = Hkv * 128; p.k_stride[2] = 128;
    memcpy(p.v_stride, p.k_stride, sizeof(p.k_stride));
    memcpy(p.o_stride, p.q_stride, sizeof(p.q_stride));

    const int64_t rows = fp_num_rows(&p), cap = fp_max_nnz(&p);
    const int64_t ws_sel = fp_workspace_size(&p), ws_pre = fp_prefill_workspace_size(&p);
    if (rows < 0 || cap < 0 || ws_sel < 0 || ws_pre < 0) { printf("sizing: %s\n", fp_last_error()); return 1; }
    const int nb = (S + block - 1) / block;
    const size_t qb = (size_t)S * Hq * 128 * 2, kvb = (size_t)S * Hkv * 128 * 2;

    void* hq = read_file(dir, "q.bin", qb);
    void* hk = read_file(dir, "k.bin", kvb);
    void* hv = read_file(dir, "v.bin", kvb);
    void* dq = to_device(hq, qb);
    void* dk = to_device(hk, kvb);
    void* dv = to_device(hv, kvb);
    float* qbar = (float*)device((size_t)Hq * nb * 128 * 4);
    float* kbar = (float*)device((size_t)Hkv * nb * 128 * 4);
    float* vbar = (float*)device((size_t)Hkv * nb * 128 * 4);
    float* scores = (float*)device((size_t)Hq * nb * nb * 4);
    int32_t* row_ptr = (int32_t*)device((size_t)(rows + 1) * 4);
    int32_t* col_idx = (int32_t*)device((size_t)cap * 4);
    int32_t* sched = (int32_t*)device((size_t)rows * 4);
    void* ws = device((size_t)(ws_sel > ws_pre ? ws_sel : ws_pre));
    void* o = device(qb);
    float* lse = (float*)device((size_t)Hq * S * 4);

    hipStream_t st;
    HIP_OK(hipStreamCreate(&st));
    FP_OK_(fp_block_scores(&p, dq, dk, dv, NULL, NULL, NULL, qbar, kbar, vbar, scores, st));
    FP_OK_(fp_select_blocks(&p, scores, tau, row_ptr, col_idx, cap, sched, ws,
                            (size_t)(ws_sel > ws_pre ? ws_sel : ws_pre), st));
    FP_OK_(fp_sparse_prefill(&p, dq, dk, dv, NULL, NULL, NULL, kbar, vbar, row_ptr, col_idx, sched, o, lse,
                             ws, (size_t)(ws_sel > ws_pre ? ws_sel : ws_pre), st));
    HIP_OK(hipStreamSynchronize(st));

    int32_t* h_rp = (int32_t*)malloc((size_t)(rows + 1) * 4);
    HIP_OK(hipMemcpy(h_rp, row_ptr, (size_t)(rows + 1) * 4, hipMemcpyDeviceToHost));
    const int32_t nnz = h_rp[rows];
    if (nnz < rows || nnz > cap) { printf("bad nnz %d\n", nnz); return 1; }
    int32_t* h_ci = (int32_t*)malloc((size_t)nnz * 4);
    int32_t* h_sc = (int32_t*)malloc((size_t)rows * 4);
    void* h_o = malloc(qb);
    float* h_lse = (float*)malloc((size_t)Hq * S * 4);
    HIP_OK(hipMemcpy(h_ci, col_idx, (size_t)nnz * 4, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(h_sc, sched, (size_t)rows * 4, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(h_o, o, qb, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(h_lse, lse, (size_t)Hq * S * 4, hipMemcpyDeviceToHost));
    write_file(dir, "row_ptr.bin", h_rp, (size_t)(rows + 1) * 4);
    write_file(dir, "col_idx.bin", h_ci, (size_t)nnz * 4);
    write_file(dir, "sched.bin", h_sc, (size_t)rows * 4);
    write_file(dir, "o.bin", h_o, qb);
    write_file(dir, "lse.bin", h_lse, (size_t)Hq * S * 4);

    HIP_OK(hipStreamDestroy(st));
    void* bufs[] = {dq, dk, dv, qbar, kbar, vbar, scores, row_ptr, col_idx, sched, ws, o, lse};
    for (size_t i = 0; i < sizeof(bufs) / sizeof(bufs[0]); ++i) HIP_OK(hipFree(bufs[i]));
    free(hq); free(hk); free(hv); free(h_rp); free(h_ci); free(h_sc); free(h_o); free(h_lse);
    printf("ok nnz=%d\n", nnz);
    return 0;
}
