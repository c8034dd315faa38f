/*
 * fp_prefill.h -- C ABI of a block-sparse causal GQA prefill-attention library
 * for AMD Instinct MI355X (gfx950).
 *
 * The method is FlashPrefill V2's prefill path as the pages describe it:
 *   - a block-level score estimate per (query block, key block) pair
 *     (aipulsen.com article body; lode.cx page, "How It Works");
 *   - a max-based dynamic threshold that keeps the key blocks whose estimate
 *     lies within tau of the query block's row maximum (lode.cx page, "How It
 *     Works"; aimodeling.com page, "From Prototype to Production");
 *   - a sparse flash-attention pass over the kept blocks with online softmax
 *     (lode.cx page, implementation paragraph and bullet list);
 *   - a mean-correction term standing in for the pruned blocks (lode.cx page,
 *     "How It Works"; aimodeling.com page, "Error correction" bullet);
 *   - FP8 inputs, paged KV cache and continuous (varlen) batching (lode.cx
 *     page, implementation paragraph; aimodeling.com page, "Operator alignment"
 *     and "Framework integration" bullets).
 * The pages print no formulas. This library computes exactly these equations
 * (B = block size, c = softmax scale, G = Hq/Hkv, g(h) = h / G):
 *   E1  Qbar[h,i] = mean of q over the present rows of query block i;
 *       Kbar[g,j], Vbar[g,j] = mean of k, v over key block j.
 *   E2  S[h,i,j] = c <Qbar[h,i], Kbar[g(h),j]>, j <= i   (-inf for j > i).
 *   E3  M[h,i] = max_{j<=i} S[h,i,j].
 *   E4  R[g,i,j] = max over the G heads h of group g of (S[h,i,j] - M[h,i]).
 *   E5  kept(g,i) = {0, i} U { j <= i : R[g,i,j] >= -tau }.
 *   E6  row t of query block i, head h: softmax over (a) the causal tokens
 *       s <= t of the kept blocks with logit c<q_t,k_s> and (b) one
 *       pseudo-token per pruned block j with key Kbar[g,j], value Vbar[g,j]
 *       and logit c<q_t,Kbar[g,j]> + ln|block j|; o = weighted value sum,
 *       lse = natural log of the softmax denominator.
 *
 * Conventions (every entry point):
 *   - Pointers marked (device) are HIP device pointers, (host) host pointers.
 *     Every buffer is owned by the caller. The library allocates, frees and
 *     synchronises nothing and keeps no state between calls.
 *   - Work is enqueued on `stream` (a hipStream_t; NULL = default stream) and
 *     the call returns without waiting. Device faults surface at the caller's
 *     next synchronisation.
 *   - Return value: FP_OK, or a negative FP_ERR_* code with a message in
 *     fp_last_error() (thread-local). Arguments are validated before any HIP
 *     call, so an error return means nothing was enqueued (FP_ERR_HIP aside).
 *   - head_dim must be 128; block must be 64 or 128; Hq % Hkv == 0 and
 *     Hq / Hkv <= 16; block count per sequence <= 16384.
 *   - Strides are in elements; the last (head_dim) dimension is contiguous.
 *     Fixed shape: k and v token strides x block x element size < 2 GiB.
 *   - Inputs are post-RoPE and finite (non-finite inputs: undefined results).
 *   - Kept-block lists are CSR over rows ordered (sequence b, KV head g, query
 *     block i ascending); columns strictly ascending absolute key-block
 *     indices within [0, i]. A caller's list that breaks this gives
 *     unspecified results, but the attention never loads a tile outside the
 *     row's blocks 0 .. i.
 */
#ifndef FP_PREFILL_H
#define FP_PREFILL_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define FP_OK 0
#define FP_ERR_INVALID (-1)      /* null pointer, bad size, NaN tau, ...        */
#define FP_ERR_UNSUPPORTED (-2)  /* head_dim != 128, block not 64/128, ...      */
#define FP_ERR_CAPACITY (-3)     /* col_idx capacity or workspace too small      */
#define FP_ERR_HIP (-4)          /* a HIP launch reported an error              */

#define FP_DTYPE_BF16 0          /* bfloat16 Q/K/V                               */
#define FP_DTYPE_FP8_E4M3 1      /* OCP E4M3FN codes (uint8) + fp32 scales       */
#define FP_OUT_BF16 0            /* fp_sparse_prefill output o in bfloat16        */
#define FP_OUT_FP32 2            /* ... in float32 (diagnostic: no output rounding) */
#define FP_VARIANT_MEAN_CORRECTION 0   /* E6 as specified: pruned blocks as pooled pseudo-tokens */
#define FP_VARIANT_NO_CORRECTION 1     /* ablation: pruned blocks simply dropped        */
#define FP_VARIANT_PER_HEAD_LISTS 2    /* ablation: one kept list per query head (E4 without the
                                          GQA union); kept-list rows are (b, query head, i)  */
#define FP_VARIANT_BLOCK_SCORE 3       /* ablation: a pruned block's pseudo-token takes the block
                                          score S[h,i,j] + ln|block| as logit for every row of
                                          query block i (fp_sparse_prefill_scored)            */
#define FP_SPLIT_OFF 0           /* each (row, slice) runs in one workgroup: a row's results do not
                                    depend on the other rows of the batch (default)            */
#define FP_SPLIT_SMALL_GRIDS 1   /* a problem of at most 128 (row, 256-row slice) work units, too
                                    few for the chip's 256 compute units, splits each row's tile
                                    sequence over up to 8 workgroups and merges their partial
                                    results: lower latency for short prompts; the rounding then
                                    depends on the problem's size                              */

/* Fixed-shape batch: `batch` sequences of `seqlen` tokens each, one-shot
 * prefill (no cached prefix). q [batch, seqlen, Hq, 128], k and v
 * [batch, seqlen, Hkv, 128], o like q; strides given per tensor (o strides
 * in elements of out_dtype; fp32 o rows 16-byte aligned). */
typedef struct fp_problem {
    int32_t batch;
    int32_t seqlen;
    int32_t num_q_heads;
    int32_t num_kv_heads;
    int32_t head_dim;        /* 128 */
    int32_t block;           /* 64 or 128 (square blocks) */
    int32_t dtype;           /* FP_DTYPE_* */
    float softmax_scale;     /* c; 0 means 1/sqrt(head_dim) */
    int64_t q_stride[3];     /* batch, token, head */
    int64_t k_stride[3];
    int64_t v_stride[3];
    int64_t o_stride[3];
    int32_t out_dtype;       /* FP_OUT_BF16 (0, default) or FP_OUT_FP32: diagnostic fp32 o */
    int32_t variant;         /* FP_VARIANT_MEAN_CORRECTION (0, default) or an ablation: NO_CORRECTION
                                and BLOCK_SCORE change E6 only; PER_HEAD_LISTS changes the kept
                                lists (sizes, selection and attention rows) */
    int32_t split;           /* FP_SPLIT_OFF (0, default) or FP_SPLIT_SMALL_GRIDS (E6 only) */
    int32_t reserved_;       /* must be 0 */
} fp_problem;

/* Paged varlen batch (continuous batching with cached prefixes). Sequence b
 * has L_b = seqlens_k[b] keys in the cache (new chunk included) and
 * q_len_b = cu_seqlens_q[b+1] - cu_seqlens_q[b] present query rows, the
 * positions [L_b - q_len_b, L_b). Blocks sit on the absolute-position grid. */
typedef struct fp_varlen_problem {
    int32_t num_seqs;        /* 1 .. 4096 */
    int32_t num_q_heads;
    int32_t num_kv_heads;
    int32_t head_dim;        /* 128 */
    int32_t block;           /* 64 or 128 */
    int32_t page_size;       /* power of two in [16, 256] */
    int32_t dtype;           /* FP_DTYPE_BF16 or FP_DTYPE_FP8_E4M3 */
    float softmax_scale;     /* 0 means 1/sqrt(head_dim) */
    int32_t max_pages_per_seq;  /* row length of block_table */
    int32_t pad_;
    int64_t q_stride[2];     /* packed q: token, head */
    int64_t kv_stride[3];    /* k_cache / v_cache: page, token-in-page, head */
    int64_t o_stride[2];     /* packed o: token, head */
} fp_varlen_problem;

const char* fp_version(void);
const char* fp_last_error(void);

/* Sizing (host only, no HIP call). Return < 0 with fp_last_error() set on an
 * invalid problem. With FP_VARIANT_PER_HEAD_LISTS, Hq replaces Hkv below. */
int64_t fp_num_rows(const fp_problem* p);       /* batch * Hkv * nb           */
int64_t fp_max_nnz(const fp_problem* p);        /* batch * Hkv * nb(nb+1)/2   */
int64_t fp_workspace_size(const fp_problem* p); /* bytes for fp_select_blocks */
/* bytes for fp_sparse_prefill: the bf16 summary operands and, with
 * split = FP_SPLIT_SMALL_GRIDS on a problem of at most 128 (row, 256-row
 * slice) work units, room for the partial results (unnormalised O, max,
 * sum) of the up to 8 workgroups each row's tile sequence is split over,
 * which a merge pass combines. The split is a function of the problem alone,
 * so fp_sparse_prefill, fp_sparse_prefill_scored and fp_sparse_prefill_noalloc
 * compute identical results on one problem. */
int64_t fp_prefill_workspace_size(const fp_problem* p);

/* E1-E2: the block-level score estimate (aipulsen.com article body: scores
 * estimated per block pair instead of per token; lode.cx page, "How It
 * Works": a small sample of attention scores decides the kept blocks).
 * Pools Q, K, V per block (float32 accumulation) and writes the block
 * scores. q, k, v (device, read-only): bf16, or E4M3FN codes with q_scale,
 * k_scale, v_scale (device, fp32 [batch, H, ceil(seqlen/128)], one scale per
 * 128-token block; NULL for bf16). Outputs (device, fp32, fully overwritten):
 * qbar [batch, Hq, nb, 128], kbar and vbar [batch, Hkv, nb, 128],
 * scores [batch, Hq, nb, nb] with -inf above the diagonal. */
int fp_block_scores(const fp_problem* p, const void* q, const void* k, const void* v,
                    const float* q_scale, const float* k_scale, const float* v_scale,
                    float* qbar, float* kbar, float* vbar, float* scores, void* stream);

/* E3-E5 plus compaction: the max-based dynamic threshold (lode.cx page, "How
 * It Works"; aimodeling.com page, "From Prototype to Production") with the G
 * query heads of a KV head sharing one list (lode.cx page, implementation
 * bullet list: PackGQA). scores (device) as written by fp_block_scores.
 * tau: +inf keeps everything, tau < 0 keeps only the sink and diagonal
 * blocks, NaN is an error. Outputs (device): row_ptr int32 [rows + 1],
 * col_idx int32 [capacity] (capacity >= fp_max_nnz checked on the host),
 * sched int32 [rows] or NULL: the work order for fp_sparse_prefill. The
 * (sequence, KV head) pairs, in row order, form groups by where each pair's
 * K/V starts, in units of 128 MiB of K and V (widened so that groups x
 * (key blocks + 1) stays within 32768); groups come in order, rows inside a
 * group by kept count descending (heavy-row-first), ties by row id ascending.
 * workspace (device) of ws_bytes >= fp_workspace_size(p). */
int fp_select_blocks(const fp_problem* p, const float* scores, float tau,
                     int32_t* row_ptr, int32_t* col_idx, int64_t capacity,
                     int32_t* sched, void* workspace, size_t ws_bytes, void* stream);

/* E1-E5 in one call, without a score matrix: pools Q, K, V per block (as
 * fp_block_scores), then computes each row's block scores from the pooled
 * rows inside the selection and emits the kept lists and schedule (as
 * fp_select_blocks). The estimate has to be cheap next to the attention it
 * prunes (aipulsen.com article body: the search latency of earlier sparse
 * methods). The scores are summed in the same order as fp_block_scores, so
 * the kept lists equal those of fp_block_scores + fp_select_blocks bit for
 * bit. Sequences of more than 1024 key blocks fall back to a score matrix in
 * the workspace. Outputs: qbar, kbar, vbar (device, as fp_block_scores),
 * row_ptr, col_idx (capacity >= fp_max_nnz), sched (nullable); workspace of
 * ws_bytes >= fp_estimate_select_workspace_size(p), 256-byte aligned. */
int64_t fp_estimate_select_workspace_size(const fp_problem* p);
int fp_estimate_select(const fp_problem* p, const void* q, const void* k, const void* v,
                       const float* q_scale, const float* k_scale, const float* v_scale, float tau,
                       float* qbar, float* kbar, float* vbar, int32_t* row_ptr, int32_t* col_idx,
                       int64_t capacity, int32_t* sched, void* workspace, size_t ws_bytes, void* stream);

/* E6: the sparse flash-attention operator over the kept blocks (lode.cx
 * page, implementation paragraph and bullet list; aimodeling.com page,
 * "Operator alignment" bullet) plus the mean correction for the pruned
 * blocks (lode.cx page, "How It Works"; aimodeling.com page, "Error
 * correction" bullet). Sparse attention over the kept blocks of (row_ptr, col_idx) -- any
 * valid kept list whose rows contain the sink and diagonal blocks, e.g. the
 * one fp_select_blocks wrote -- plus the mean-correction pseudo-tokens of the
 * pruned blocks, taken from kbar and vbar (device, as fp_block_scores wrote
 * them). sched (device, NULL = row order) only orders the work. workspace
 * (device, ws_bytes >= fp_prefill_workspace_size, 256-byte aligned) receives
 * bf16 copies of kbar and vbar for the correction; its contents need not be
 * preserved between calls. Outputs (device): o (o_stride; bf16 with 8-byte
 * aligned rows, or fp32 with 16-byte aligned rows when out_dtype is
 * FP_OUT_FP32), lse fp32
 * [batch, Hq, seqlen] or NULL. */
int fp_sparse_prefill(const fp_problem* p, const void* q, const void* k, const void* v,
                      const float* q_scale, const float* k_scale, const float* v_scale,
                      const float* kbar, const float* vbar,
                      const int32_t* row_ptr, const int32_t* col_idx, const int32_t* sched,
                      void* o, float* lse, void* workspace, size_t ws_bytes, void* stream);

/* E6 under the block-score correction (FP_VARIANT_BLOCK_SCORE, an ablation
 * of the mean correction of the lode.cx page, "How It Works", and the
 * aimodeling.com page, "Error correction" bullet): a pruned block j stands in
 * as one pseudo-token with value Vbar[g,j] and logit scores[b,h,i,j] +
 * ln|block j| for every row of query block i. scores (device) as written by
 * fp_block_scores; no pooled keys are read. Other arguments as for
 * fp_sparse_prefill; the problem's variant must be FP_VARIANT_BLOCK_SCORE. */
int fp_sparse_prefill_scored(const fp_problem* p, const void* q, const void* k, const void* v,
                             const float* q_scale, const float* k_scale, const float* v_scale,
                             const float* scores, const float* vbar,
                             const int32_t* row_ptr, const int32_t* col_idx, const int32_t* sched,
                             void* o, float* lse, void* workspace, size_t ws_bytes, void* stream);

/* Dense causal attention with the same kernel: every key block j <= i of
 * every row is attended (no estimate, no selection, no correction), tiles in
 * order, rows longest first. It is the dense baseline the sparse path is
 * measured against (the pages quote their speedups against dense
 * FlashAttention kernels: lode.cx page, "Why It Matters"; aimodeling.com
 * page, "The Numbers That Matter") and equals fp_sparse_prefill on the
 * lists of tau = +inf bit for bit. Arguments as for fp_sparse_prefill (the
 * problem's variant is ignored); no kept lists, no workspace. */
int fp_dense_prefill(const fp_problem* p, const void* q, const void* k, const void* v,
                     const float* q_scale, const float* k_scale, const float* v_scale,
                     void* o, float* lse, void* stream);

/* Allocation-free variant of fp_sparse_prefill, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc): the same kernels and results,
 * with the workspace replaced by a static device array of
 * FP_NOALLOC_SCRATCH_BYTES that each GPU holds from the library's load
 * until the process ends. It accepts problems with batch x num_kv_heads x
 * ceil(seqlen / block) <= FP_NOALLOC_MAX_POOLED_ROWS pooled rows and returns
 * FP_ERR_CAPACITY above that. It calls no hipMalloc or hipFree; the first
 * call on a device looks the array's address up there (hipGetSymbolAddress),
 * with that device current, which must be the device of `stream`. Every call
 * on one GPU uses that GPU's one array: calls that overlap in time on the same
 * GPU (other streams, other threads) race and must be serialised by the
 * caller. Arguments as for fp_sparse_prefill. */
#define FP_NOALLOC_MAX_POOLED_ROWS 32768
/* The array holds the bf16 summary operands (3 x 256 bytes per pooled row)
 * and, for a problem of at most 128 workgroups, whose rows are split over
 * several workgroups (see fp_prefill_workspace_size), the parts' partial
 * results (at most 256 parts of 133,120 bytes). */
#define FP_NOALLOC_SCRATCH_BYTES (36 << 20)
int fp_sparse_prefill_noalloc(const fp_problem* p, const void* q, const void* k, const void* v,
                              const float* q_scale, const float* k_scale, const float* v_scale,
                              const float* kbar, const float* vbar,
                              const int32_t* row_ptr, const int32_t* col_idx, const int32_t* sched,
                              void* o, float* lse, void* stream);

/* Sizing of a paged varlen call (host only). cu_seqlens_q int32 [num_seqs+1]
 * and seqlens_k int32 [num_seqs] are HOST arrays. */
int64_t fp_varlen_num_rows(const fp_varlen_problem* p, const int32_t* cu_seqlens_q,
                           const int32_t* seqlens_k);
int64_t fp_varlen_max_nnz(const fp_varlen_problem* p, const int32_t* cu_seqlens_q,
                          const int32_t* seqlens_k);
int64_t fp_varlen_workspace_size(const fp_varlen_problem* p, const int32_t* cu_seqlens_q,
                                 const int32_t* seqlens_k);

/* E1-E6 for a paged varlen batch in one call (the pages' paged KV cache and
 * continuous batching: aimodeling.com page, "Framework integration" bullet;
 * lode.cx page, implementation paragraph). When no sequence has present rows
 * (every one fully cached) q and o may be NULL and only row_ptr[0] = 0 is
 * written.
 * q (device) packed [sum q_len, Hq, 128]; k_cache, v_cache (device)
 * [pages, page_size, Hkv, 128]; bf16, or E4M3FN codes when dtype is
 * FP_DTYPE_FP8_E4M3. block_table (device) int32 [num_seqs, max_pages_per_seq]
 * (token s of sequence b lives in page block_table[b][s / page_size], slot
 * s % page_size; the new chunk's keys must already be in the cache). Every
 * entry a sequence uses (its first ceil(seqlens_k[b] / page_size)) must name
 * a page of the caches: the library does not know the pool's size and does
 * not check them; unused entries are never read.
 * q_scale, k_scale, v_scale (device, fp8 only, else NULL): fp32
 * [num_seqs, H, nsb] with nsb = ceil(max_pages_per_seq * page_size / 128),
 * one scale per 128 positions of each sequence (the query row at position t
 * of sequence b uses q_scale[b][h][t / 128]; keys and values likewise).
 * cu_seqlens_q, seqlens_k: HOST arrays, read during the call only.
 * Outputs (device): row_ptr [rows+1] and col_idx [capacity] (the kept lists,
 * capacity >= fp_varlen_max_nnz), o packed like q in bf16, lse fp32
 * [Hq, sum q_len] or NULL. workspace (device) >= fp_varlen_workspace_size
 * bytes. */
int fp_sparse_prefill_paged(const fp_varlen_problem* p, const void* q,
                            const int32_t* cu_seqlens_q, const int32_t* seqlens_k,
                            const void* k_cache, const void* v_cache,
                            const int32_t* block_table,
                            const float* q_scale, const float* k_scale, const float* v_scale,
                            float tau, int32_t* row_ptr, int32_t* col_idx, int64_t capacity,
                            void* o, float* lse, void* workspace, size_t ws_bytes,
                            void* stream);

/* fp_sparse_prefill_paged with a pooled-KV cache for chunked prefill: the
 * block means of K and V (E1) are kept beside the page cache, so a chunk
 * pools only the blocks its new keys fall in (the pages' chunked prefill over
 * a paged KV cache with continuous batching: lode.cx page, "How It Works",
 * implementation paragraph; aimodeling.com page, "Framework integration"
 * bullet).
 * kbar_cache, vbar_cache (device, 16-byte aligned): fp32 [slots, Hkv, 128],
 * slots = (pages of the cache) * spp with spp = max(1, page_size / block).
 * The complete key block j of sequence b (tokens [j*block, (j+1)*block)) has
 * slot block_table[b][e / page_size] * spp + (e % page_size) / block, where
 * e = (j+1)*block - 1 is its last token: the slot travels with the page that
 * holds the block's last token, so sequences that share that page share the
 * block's tokens and its slot.
 * Read: each block complete within the cached prefix ((j+1)*block <= L_b -
 * q_len_b) is taken from its slot and its keys are not re-read. Its slot
 * must hold what an earlier call of this entry point wrote when the block
 * was complete (that call's chunk ended at or past the block's last token);
 * a slot never written holds garbage, which the call cannot detect.
 * Write: every complete block this call pools ((j+1)*block > L_b - q_len_b
 * and <= L_b) is written to its slot. A block still partial at the chunk's
 * end is pooled from the page cache on each call and never written.
 * Sequences without present rows read and write nothing. Every other
 * argument, output and error is as for fp_sparse_prefill_paged; the outputs
 * are bit-identical to its own on the same call when the read slots hold
 * what this entry point wrote. Calls that overlap on the same slots race. */
int fp_sparse_prefill_paged_cached(const fp_varlen_problem* p, const void* q,
                                   const int32_t* cu_seqlens_q, const int32_t* seqlens_k,
                                   const void* k_cache, const void* v_cache,
                                   const int32_t* block_table,
                                   const float* q_scale, const float* k_scale, const float* v_scale,
                                   float* kbar_cache, float* vbar_cache,
                                   float tau, int32_t* row_ptr, int32_t* col_idx, int64_t capacity,
                                   void* o, float* lse, void* workspace, size_t ws_bytes,
                                   void* stream);

#ifdef __cplusplus
}
#endif

#endif /* FP_PREFILL_H */
