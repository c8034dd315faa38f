// C ABI of the block-sparse prefill library (declared in include/fp_prefill.h).
//
// Host side only: argument validation (always before the first HIP call),
// workspace sizing and carving, and launch sequencing on the caller's stream.
// Nothing here allocates, frees or synchronises.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <mutex>
#include <vector>

#include "../../include/fp_prefill.h"
#include "attn_geom.h"

using namespace fp;

namespace {

thread_local char g_err[512] = "";

int fail(int code, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof(g_err), fmt, ap);
    va_end(ap);
    return code;
}

int ok() {
    g_err[0] = 0;
    return FP_OK;
}

constexpr size_t ALIGN = 256;
size_t align_up(size_t x) { return (x + ALIGN - 1) / ALIGN * ALIGN; }

float default_scale(float sc, int d) { return sc == 0.f ? 1.f / sqrtf((float)d) : sc; }

int check_heads(int Hq, int Hkv, int d, int blk) {
    if (Hq <= 0 || Hkv <= 0) return fail(FP_ERR_INVALID, "head counts must be positive (Hq=%d, Hkv=%d)", Hq, Hkv);
    if (Hq % Hkv) return fail(FP_ERR_INVALID, "num_q_heads %% num_kv_heads != 0 (%d, %d)", Hq, Hkv);
    if (Hq / Hkv > MAX_G) return fail(FP_ERR_UNSUPPORTED, "Hq/Hkv = %d exceeds %d", Hq / Hkv, MAX_G);
    if (d != D) return fail(FP_ERR_UNSUPPORTED, "head_dim %d unsupported (only 128)", d);
    if (blk != 64 && blk != 128) return fail(FP_ERR_UNSUPPORTED, "block %d unsupported (64 or 128)", blk);
    return FP_OK;
}

int check_fixed(const fp_problem* p) {
    if (!p) return fail(FP_ERR_INVALID, "problem is NULL");
    int rc = check_heads(p->num_q_heads, p->num_kv_heads, p->head_dim, p->block);
    if (rc) return rc;
    if (p->batch <= 0 || p->seqlen <= 0) return fail(FP_ERR_INVALID, "batch and seqlen must be positive");
    if (p->dtype != FP_DTYPE_BF16 && p->dtype != FP_DTYPE_FP8_E4M3)
        return fail(FP_ERR_UNSUPPORTED, "dtype %d unsupported", p->dtype);
    if (!(p->softmax_scale >= 0.f) || isinf(p->softmax_scale))
        return fail(FP_ERR_INVALID, "softmax_scale must be finite and >= 0");
    const int nb = cdiv(p->seqlen, p->block);
    if (nb > MAX_NB) return fail(FP_ERR_UNSUPPORTED, "%d blocks per sequence exceed %d", nb, MAX_NB);
    const long long rows = (long long)p->batch * p->num_kv_heads * nb;
    if ((long long)p->batch * nb * p->num_q_heads * nb > (1LL << 40) || rows > (1LL << 30))
        return fail(FP_ERR_UNSUPPORTED, "problem too large");
    const int64_t* st[4] = {p->q_stride, p->k_stride, p->v_stride, p->o_stride};
    for (int t = 0; t < 4; ++t)
        for (int e = 0; e < 3; ++e)
            if (st[t][e] < 0) return fail(FP_ERR_INVALID, "negative stride");
    const int esz = p->dtype == FP_DTYPE_BF16 ? 2 : 1;
    // 16-byte vector loads of whole rows need 16-byte aligned row starts
    for (int t = 0; t < 3; ++t)
        for (int e = 0; e < 3; ++e)
            if ((st[t][e] * esz) % 16) return fail(FP_ERR_INVALID, "strides must be multiples of 16 bytes");
    if (p->out_dtype != FP_OUT_BF16 && p->out_dtype != FP_OUT_FP32)
        return fail(FP_ERR_UNSUPPORTED, "out_dtype %d unsupported", p->out_dtype);
    if (p->variant < FP_VARIANT_MEAN_CORRECTION || p->variant > FP_VARIANT_BLOCK_SCORE)
        return fail(FP_ERR_UNSUPPORTED, "variant %d unsupported", p->variant);
    if (p->split != FP_SPLIT_OFF && p->split != FP_SPLIT_SMALL_GRIDS)
        return fail(FP_ERR_UNSUPPORTED, "split %d unsupported", p->split);
    if (p->reserved_ != 0) return fail(FP_ERR_INVALID, "fp_problem.reserved_ must be 0");
    const int osz = p->out_dtype == FP_OUT_FP32 ? 4 : 2;
    for (int e = 0; e < 3; ++e)
        if ((p->o_stride[e] * osz) % (osz == 4 ? 16 : 8))
            return fail(FP_ERR_INVALID, "o strides must be multiples of %d bytes", osz == 4 ? 16 : 8);
    // a K/V tile's per-lane load offsets are 32-bit byte offsets
    if (p->k_stride[1] * esz * p->block >= (1LL << 31) || p->v_stride[1] * esz * p->block >= (1LL << 31))
        return fail(FP_ERR_UNSUPPORTED, "k/v token stride x block must stay below 2 GiB");
    return FP_OK;
}

GeoFixed geo_fixed(const fp_problem* p) {
    GeoFixed g;
    g.nseq = p->batch;
    g.S = p->seqlen;
    g.Hq = p->num_q_heads;
    g.Hkv = p->num_kv_heads;
    g.blk = p->block;
    g.nb = cdiv(p->seqlen, p->block);
    g.ntile = score_tiles(g.nb, g.nb);
    return g;
}

bool misaligned(const void* ptr, size_t a) { return ((uintptr_t)ptr) % a != 0; }

// Schedule groups: consecutive (sequence, KV head) pairs whose K/V together
// fit SCHED_GROUP_BYTES run one group after another (heavy rows first within
// a group), so the K/V that the running rows read stays within the
// memory-side cache (256 MiB on this part) instead of spanning every head of
// the batch. Measured at S = 131072, 32/8 heads: 3% less attention time than
// one heavy-first order over all heads; groups of 4 heads (256 MiB) were 10%
// slower. The histogram of the schedule sort holds ngrp * (max_nbk + 1) bins
// and is kept within SORT_MAX_BINS by widening the groups.
constexpr long long SCHED_GROUP_BYTES = 128LL << 20;
constexpr int SORT_MAX_BINS = 32768;

struct SortPlan {
    int ngrp;
    long long grp_units;   // key blocks x KV heads per group
};

SortPlan sort_plan(long long total_units, int max_nbk, int blk, int esz) {
    const long long unit_bytes = (long long)blk * D * esz * 2;          // one key block of K and V, one head
    long long units = std::max(SCHED_GROUP_BYTES / unit_bytes, 1LL);
    long long ng = std::max((total_units + units - 1) / units, 1LL);
    const long long nmax = std::max(SORT_MAX_BINS / (max_nbk + 1), 1);
    if (ng > nmax) {
        units = (total_units + nmax - 1) / nmax;
        ng = std::max((total_units + units - 1) / units, 1LL);
    }
    return SortPlan{(int)ng, units};
}

struct SelectWs {
    size_t counts, bits, keys, maxc, hist, total;
    int nbw;
};

SelectWs select_ws(long long rows, int max_nbk, int ngrp) {
    SelectWs w;
    w.nbw = cdiv(max_nbk, 32) + 1;
    w.counts = 0;
    w.bits = align_up((size_t)rows * 4);
    w.keys = w.bits + align_up((size_t)rows * w.nbw * 4);
    w.maxc = w.keys + align_up((size_t)rows * 4);
    w.hist = w.maxc + align_up(4);
    w.total = w.hist + align_up((size_t)((rows + SORT_CHUNK - 1) / SORT_CHUNK) * ngrp * (max_nbk + 1) * 4);
    return w;
}

// The kept lists' view of a problem: one list per (sequence, KV head, query
// block), or per (sequence, query head, query block) for the per-head
// variant -- there each query head is its own group of one.
fp_problem lists_of(const fp_problem* p) {
    fp_problem v = *p;
    if (p->variant == FP_VARIANT_PER_HEAD_LISTS) v.num_kv_heads = p->num_q_heads;
    return v;
}

SortPlan fixed_sort_plan(const fp_problem* p) {
    const int nb = cdiv(p->seqlen, p->block);
    return sort_plan((long long)p->batch * p->num_kv_heads * nb, nb, p->block,
                     p->dtype == FP_DTYPE_FP8_E4M3 ? 1 : 2);
}

// bf16 copies of the pooled keys (hi, lo) and values used by the summary tiles
size_t summary_ws_bytes(long long pooled_rows) { return 3 * align_up((size_t)pooled_rows * D * 2); }

// Split rows (small grids, fixed shape): parts per row and the bytes of their partial results.
int fixed_split(const fp_problem* p) {
    if (p->split != FP_SPLIT_SMALL_GRIDS) return 1;
    const fp_problem lv = lists_of(p);
    const int rows = p->batch * lv.num_kv_heads * cdiv(p->seqlen, p->block);
    return split_count(rows, attn_slices(p->num_q_heads / lv.num_kv_heads, p->block));
}
size_t split_ws_bytes(const fp_problem* p) {
    const int ns = fixed_split(p);
    if (ns < 2) return 0;
    const fp_problem lv = lists_of(p);
    const int rows = p->batch * lv.num_kv_heads * cdiv(p->seqlen, p->block);
    return align_up((size_t)split_floats(split_parts(rows, attn_slices(p->num_q_heads / lv.num_kv_heads, p->block),
                                                     ns)) * 4);
}

}  // namespace

// ---------------------------------------------------------------------------
// descriptor-table copy: the table rides in kernel arguments (by value), so no
// host buffer has to outlive the call and no memcpy is queued
// ---------------------------------------------------------------------------
namespace fp {
constexpr int TABLE_CHUNK = 64;
struct TableChunk {
    SeqDesc e[TABLE_CHUNK];
};
__global__ void table_copy_kernel(TableChunk c, int n, SeqDesc* dst) {
    const int t = threadIdx.x;
    if (t < n) dst[t] = c.e[t];
}
// row_ptr[0] = 0 for a batch without present rows (a kernel rather than a
// memset node, so the call stays capturable in a graph)
__global__ void zero_first_kernel(int32_t* p) { *p = 0; }
hipError_t launch_zero_first(int32_t* p, hipStream_t st) {
    zero_first_kernel<<<1, 1, 0, st>>>(p);
    return hipGetLastError();
}
hipError_t launch_table_copy(const SeqDesc* host, int n, SeqDesc* dev, hipStream_t st) {
    for (int base = 0; base < n; base += TABLE_CHUNK) {
        TableChunk c;
        const int m = std::min(TABLE_CHUNK, n - base);
        memcpy(c.e, host + base, sizeof(SeqDesc) * m);
        table_copy_kernel<<<1, TABLE_CHUNK, 0, st>>>(c, m, dev + base);
    }
    return hipGetLastError();
}
}  // namespace fp

extern "C" {

const char* fp_version(void) { return "fp_prefill 0.1.0 (gfx950)"; }
const char* fp_last_error(void) { return g_err; }

int64_t fp_num_rows(const fp_problem* p) {
    int rc = check_fixed(p);
    if (rc) return rc;
    return (int64_t)p->batch * lists_of(p).num_kv_heads * cdiv(p->seqlen, p->block);
}

int64_t fp_max_nnz(const fp_problem* p) {
    int rc = check_fixed(p);
    if (rc) return rc;
    const int64_t nb = cdiv(p->seqlen, p->block);
    return (int64_t)p->batch * lists_of(p).num_kv_heads * nb * (nb + 1) / 2;
}

int64_t fp_prefill_workspace_size(const fp_problem* p) {
    int rc = check_fixed(p);
    if (rc) return rc;
    return (int64_t)(summary_ws_bytes((long long)p->batch * p->num_kv_heads * cdiv(p->seqlen, p->block)) +
                     split_ws_bytes(p));
}

int64_t fp_workspace_size(const fp_problem* p) {
    int rc = check_fixed(p);
    if (rc) return rc;
    const fp_problem lv = lists_of(p);
    const int nb = cdiv(p->seqlen, p->block);
    return (int64_t)select_ws((long long)p->batch * lv.num_kv_heads * nb, nb, fixed_sort_plan(&lv).ngrp).total;
}

}  // extern "C"

namespace {

// Pooling (E1) of a checked fixed-shape problem.
hipError_t fixed_pool(const fp_problem* p, const void* q, const void* k, const void* v, const float* q_scale,
                      const float* k_scale, const float* v_scale, float* qbar, float* kbar, float* vbar,
                      hipStream_t st) {
    GeoFixed geo = geo_fixed(p);
    const int nsb = cdiv(p->seqlen, SCALE_TOK);
    PoolArgs a{};
    a.q = q; a.k = k; a.v = v;
    a.qa = RowAddr{p->q_stride[0], p->q_stride[1], p->q_stride[2]};
    a.ka = KVAddr{p->k_stride[0], p->k_stride[1], p->k_stride[2], 0, nullptr, 0, 0};
    a.va = KVAddr{p->v_stride[0], p->v_stride[1], p->v_stride[2], 0, nullptr, 0, 0};
    a.qs = ScaleAddr{q_scale, (long long)p->num_q_heads * nsb, nsb};
    a.ks = ScaleAddr{k_scale, (long long)p->num_kv_heads * nsb, nsb};
    a.vs = ScaleAddr{v_scale, (long long)p->num_kv_heads * nsb, nsb};
    a.qbar = qbar; a.kbar = kbar; a.vbar = vbar;
    a.Hq = p->num_q_heads; a.Hkv = p->num_kv_heads; a.blk = p->block;
    a.fp8 = p->dtype == FP_DTYPE_FP8_E4M3; a.paged = 0;
    a.total_qblocks = a.total_kblocks = p->batch * geo.nb;
    return launch_pool(&geo, nullptr, a, st);
}

// Block scores (E2) of a checked fixed-shape problem into `scores`.
hipError_t fixed_scores(const fp_problem* p, const float* qbar, const float* kbar, float* scores, hipStream_t st) {
    GeoFixed geo = geo_fixed(p);
    ScoreArgs sa;
    sa.qbar = qbar; sa.kbar = kbar; sa.scores = scores;
    sa.Hq = p->num_q_heads; sa.Hkv = p->num_kv_heads;
    sa.total_tiles = p->batch * geo.ntile;
    sa.scale = default_scale(p->softmax_scale, p->head_dim);
    return launch_scores(&geo, nullptr, sa, st);
}

// Shared checks of the pooled-input arguments.
int check_pool_args(const char* fn, const fp_problem* p, const void* q, const void* k, const void* v,
                    const float* q_scale, const float* k_scale, const float* v_scale, const float* qbar,
                    const float* kbar, const float* vbar) {
    if (!q || !k || !v || !qbar || !kbar || !vbar) return fail(FP_ERR_INVALID, "%s: NULL tensor pointer", fn);
    if (p->dtype == FP_DTYPE_FP8_E4M3 && (!q_scale || !k_scale || !v_scale))
        return fail(FP_ERR_INVALID, "%s: fp8 needs q_scale, k_scale and v_scale", fn);
    if (misaligned(q, 16) || misaligned(k, 16) || misaligned(v, 16) || misaligned(qbar, 16) ||
        misaligned(kbar, 16) || misaligned(vbar, 16))
        return fail(FP_ERR_INVALID, "%s: tensors must be 16-byte aligned", fn);
    return FP_OK;
}

// Checks of the kept-list outputs and workspace of a selection; fills the
// workspace carve.
int check_select_args(const char* fn, const fp_problem* p, float tau, const int32_t* row_ptr,
                      const int32_t* col_idx, int64_t capacity, const void* workspace, size_t ws_bytes,
                      size_t ws_need) {
    if (!row_ptr || !col_idx || !workspace) return fail(FP_ERR_INVALID, "%s: NULL pointer", fn);
    if (isnan(tau)) return fail(FP_ERR_INVALID, "%s: tau is NaN", fn);
    const int nb = cdiv(p->seqlen, p->block);
    const long long rows = (long long)p->batch * lists_of(p).num_kv_heads * nb;
    const long long need = rows * (nb + 1) / 2;
    if (capacity < need)
        return fail(FP_ERR_CAPACITY, "%s: capacity %lld < max nnz %lld", fn, (long long)capacity, need);
    if (ws_bytes < ws_need) return fail(FP_ERR_CAPACITY, "%s: workspace %zu < %zu bytes", fn, ws_bytes, ws_need);
    if (misaligned(workspace, ALIGN)) return fail(FP_ERR_INVALID, "workspace must be 256-byte aligned");
    return FP_OK;
}

// Selection arguments over the kept lists' view (lists_of) of a problem.
SelectArgs fixed_select_args(const fp_problem* p, const SelectWs& w, const SortPlan& sp, void* workspace,
                             float tau, int32_t* row_ptr, int32_t* col_idx, int32_t* sched) {
    const int nb = cdiv(p->seqlen, p->block);
    const int Hkv_pool = p->num_kv_heads;
    const fp_problem lv = lists_of(p);
    p = &lv;
    SelectArgs a{};
    a.Hkv_pool = Hkv_pool;
    a.kv_div = p->num_kv_heads / Hkv_pool;
    a.counts = (int32_t*)((char*)workspace + w.counts);
    a.bits = (uint32_t*)((char*)workspace + w.bits);
    a.keys = (int32_t*)((char*)workspace + w.keys);
    a.maxc = (int32_t*)((char*)workspace + w.maxc);
    a.hist = (int32_t*)((char*)workspace + w.hist);
    a.nbw = w.nbw;
    a.row_ptr = row_ptr; a.col_idx = col_idx; a.sched = sched;
    a.Hq = p->num_q_heads; a.Hkv = p->num_kv_heads;
    a.rows = p->batch * p->num_kv_heads * nb; a.max_nbk = nb;
    a.ngrp = sp.ngrp; a.grp_units = sp.grp_units;
    a.neg_tau = -tau;
    a.scale = default_scale(p->softmax_scale, p->head_dim);
    return a;
}

SelectWs fixed_select_ws(const fp_problem* p) {
    const fp_problem lv = lists_of(p);
    const int nb = cdiv(p->seqlen, p->block);
    return select_ws((long long)p->batch * lv.num_kv_heads * nb, nb, fixed_sort_plan(&lv).ngrp);
}

// Workspace of fp_estimate_select: the selection's, plus the score matrix
// when the sequence is too long for the fused kernel.
size_t estimate_select_ws(const fp_problem* p) {
    const int nb = cdiv(p->seqlen, p->block);
    size_t total = fixed_select_ws(p).total;
    if (nb > FUSED_MAX_NBK) total = align_up(total) + (size_t)p->batch * p->num_q_heads * nb * nb * 4;
    return total;
}

}  // namespace

extern "C" {

int64_t fp_estimate_select_workspace_size(const fp_problem* p) {
    int rc = check_fixed(p);
    if (rc) return rc;
    return (int64_t)estimate_select_ws(p);
}

int fp_block_scores(const fp_problem* p, const void* q, const void* k, const void* v,
                    const float* q_scale, const float* k_scale, const float* v_scale,
                    float* qbar, float* kbar, float* vbar, float* scores, void* stream) {
    int rc = check_fixed(p);
    if (rc) return rc;
    rc = check_pool_args("fp_block_scores", p, q, k, v, q_scale, k_scale, v_scale, qbar, kbar, vbar);
    if (rc) return rc;
    if (!scores) return fail(FP_ERR_INVALID, "fp_block_scores: NULL tensor pointer");
    hipStream_t st = (hipStream_t)stream;
    hipError_t e = fixed_pool(p, q, k, v, q_scale, k_scale, v_scale, qbar, kbar, vbar, st);
    if (e != hipSuccess) return fail(FP_ERR_HIP, "pool launch: %s", hipGetErrorString(e));
    e = fixed_scores(p, qbar, kbar, scores, st);
    if (e != hipSuccess) return fail(FP_ERR_HIP, "scores launch: %s", hipGetErrorString(e));
    return ok();
}

int fp_select_blocks(const fp_problem* p, const float* scores, float tau, int32_t* row_ptr,
                     int32_t* col_idx, int64_t capacity, int32_t* sched, void* workspace,
                     size_t ws_bytes, void* stream) {
    int rc = check_fixed(p);
    if (rc) return rc;
    if (!scores) return fail(FP_ERR_INVALID, "fp_select_blocks: NULL pointer");
    const SelectWs w = fixed_select_ws(p);
    rc = check_select_args("fp_select_blocks", p, tau, row_ptr, col_idx, capacity, workspace, ws_bytes, w.total);
    if (rc) return rc;
    const fp_problem lv = lists_of(p);
    GeoFixed geo = geo_fixed(&lv);
    SelectArgs a = fixed_select_args(p, w, fixed_sort_plan(&lv), workspace, tau, row_ptr, col_idx, sched);
    a.scores = scores;
    hipError_t e = launch_select(&geo, nullptr, a, (hipStream_t)stream);
    if (e != hipSuccess) return fail(FP_ERR_HIP, "select launch: %s", hipGetErrorString(e));
    return ok();
}

int fp_estimate_select(const fp_problem* p, const void* q, const void* k, const void* v,
                       const float* q_scale, const float* k_scale, const float* v_scale, float tau,
                       float* qbar, float* kbar, float* vbar, int32_t* row_ptr, int32_t* col_idx,
                       int64_t capacity, int32_t* sched, void* workspace, size_t ws_bytes, void* stream) {
    int rc = check_fixed(p);
    if (rc) return rc;
    rc = check_pool_args("fp_estimate_select", p, q, k, v, q_scale, k_scale, v_scale, qbar, kbar, vbar);
    if (rc) return rc;
    rc = check_select_args("fp_estimate_select", p, tau, row_ptr, col_idx, capacity, workspace, ws_bytes,
                           estimate_select_ws(p));
    if (rc) return rc;
    hipStream_t st = (hipStream_t)stream;
    hipError_t e = fixed_pool(p, q, k, v, q_scale, k_scale, v_scale, qbar, kbar, vbar, st);
    if (e != hipSuccess) return fail(FP_ERR_HIP, "pool launch: %s", hipGetErrorString(e));
    const SelectWs w = fixed_select_ws(p);
    const fp_problem lv = lists_of(p);
    GeoFixed geo = geo_fixed(&lv);
    SelectArgs a = fixed_select_args(p, w, fixed_sort_plan(&lv), workspace, tau, row_ptr, col_idx, sched);
    if (geo.nb <= FUSED_MAX_NBK) {
        a.qbar = qbar; a.kbar = kbar;
        e = launch_select_fused(geo, a, st);
        if (e != hipSuccess) return fail(FP_ERR_HIP, "fused select launch: %s", hipGetErrorString(e));
        return ok();
    }
    // longer sequences: the score rows do not fit the fused kernel's LDS
    float* scores = (float*)((char*)workspace + align_up(w.total));
    e = fixed_scores(p, qbar, kbar, scores, st);
    if (e != hipSuccess) return fail(FP_ERR_HIP, "scores launch: %s", hipGetErrorString(e));
    a.scores = scores;
    e = launch_select(&geo, nullptr, a, st);
    if (e != hipSuccess) return fail(FP_ERR_HIP, "select launch: %s", hipGetErrorString(e));
    return ok();
}

}  // extern "C"

namespace {

// Argument checks of fp_sparse_prefill and its allocation-free variant (no HIP call).
int check_prefill(const char* fn, const fp_problem* p, const void* q, const void* k, const void* v,
                  const float* q_scale, const float* k_scale, const float* v_scale, const float* kbar,
                  const float* vbar, const int32_t* row_ptr, const int32_t* col_idx, const void* o) {
    int rc = check_fixed(p);
    if (rc) return rc;
    if (!q || !k || !v || !kbar || !vbar || !row_ptr || !col_idx || !o)
        return fail(FP_ERR_INVALID, "%s: NULL pointer", fn);
    const bool fp8 = p->dtype == FP_DTYPE_FP8_E4M3;
    if (fp8 && (!q_scale || !k_scale || !v_scale))
        return fail(FP_ERR_INVALID, "%s: fp8 needs q_scale, k_scale and v_scale", fn);
    // fp32 o rows are written with 16-byte stores, bf16 rows with 8-byte stores
    if (misaligned(q, 16) || misaligned(k, 16) || misaligned(v, 16) || misaligned(kbar, 16) ||
        misaligned(vbar, 16) || misaligned(o, p->out_dtype == FP_OUT_FP32 ? 16 : 8))
        return fail(FP_ERR_INVALID, "%s: misaligned tensor", fn);
    return FP_OK;
}

long long fixed_pooled_rows(const fp_problem* p) {
    return (long long)p->batch * p->num_kv_heads * cdiv(p->seqlen, p->block);
}

// Launches of E6 on a checked problem; `workspace` (256-byte aligned) holds
// the bf16 summary operands, summary_ws_bytes(pooled rows) bytes.
int launch_prefill(const fp_problem* p, const void* q, const void* k, const void* v, const float* q_scale,
                   const float* k_scale, const float* v_scale, const float* kbar, const float* vbar,
                   const int32_t* row_ptr, const int32_t* col_idx, const int32_t* sched, void* o, float* lse,
                   void* workspace, hipStream_t st, const float* scores = nullptr) {
    const long long prow = fixed_pooled_rows(p);
    const bool fp8 = p->dtype == FP_DTYPE_FP8_E4M3;
    // rows of the kept lists: (sequence, KV head, query block), or per query head
    const fp_problem lv = lists_of(p);
    GeoFixed geo = geo_fixed(&lv);
    const int nsb = cdiv(p->seqlen, SCALE_TOK);
    const int G = p->num_q_heads / lv.num_kv_heads;   // query heads sharing one list
    AttnArgs a{};
    a.kv_div = lv.num_kv_heads / p->num_kv_heads;
    a.scores = scores;
    a.q = q; a.k = k; a.v = v;
    a.qa = RowAddr{p->q_stride[0], p->q_stride[1], p->q_stride[2]};
    a.oa = RowAddr{p->o_stride[0], p->o_stride[1], p->o_stride[2]};
    a.o_f32 = p->out_dtype == FP_OUT_FP32;
    a.no_correction = p->variant == FP_VARIANT_NO_CORRECTION;
    a.ka = KVAddr{p->k_stride[0], p->k_stride[1], p->k_stride[2], 0, nullptr, 0, 0};
    a.va = KVAddr{p->v_stride[0], p->v_stride[1], p->v_stride[2], 0, nullptr, 0, 0};
    a.qs = ScaleAddr{q_scale, (long long)p->num_q_heads * nsb, nsb};
    a.ks = ScaleAddr{k_scale, (long long)p->num_kv_heads * nsb, nsb};
    a.vs = ScaleAddr{v_scale, (long long)p->num_kv_heads * nsb, nsb};
    a.kbar = kbar; a.vbar = vbar;
    {
        const size_t part = align_up((size_t)prow * D * 2);
        a.kbar_hi = (const __bf16*)workspace;
        a.kbar_lo = (const __bf16*)((char*)workspace + part);
        a.vbar_bf = (const __bf16*)((char*)workspace + 2 * part);
    }
    a.row_ptr = row_ptr; a.col_idx = col_idx; a.sched = sched;
    a.o = o; a.lse = lse;
    a.la = RowAddr{(long long)p->num_q_heads * p->seqlen, 1, p->seqlen};
    a.Hq = p->num_q_heads; a.Hkv = p->num_kv_heads; a.G = G;
    a.rows = p->batch * lv.num_kv_heads * geo.nb;
    a.slices = attn_slices(G, p->block);
    // a grid too small for the chip splits each row's tiles; the parts' results follow the summary operands
    a.nsplit = fixed_split(p);
    if (a.nsplit > 1) {
        const long long parts = split_parts(a.rows, a.slices, a.nsplit);
        a.part_o = (float*)((char*)workspace + summary_ws_bytes(prow));
        a.part_ml = a.part_o + split_o_floats(parts);
    }
    a.scale_log2 = default_scale(p->softmax_scale, p->head_dim) * 1.4426950408889634f;
    // the block-score correction needs no pooled keys (kbar may be null)
    hipError_t e = launch_summary_prep(scores ? nullptr : kbar, vbar, (__bf16*)a.kbar_hi, (__bf16*)a.kbar_lo,
                                       (__bf16*)a.vbar_bf, prow * D, st);
    if (e != hipSuccess) return fail(FP_ERR_HIP, "summary prep launch: %s", hipGetErrorString(e));
    e = launch_attn(&geo, nullptr, a, p->block, fp8, 0, st);
    if (e != hipSuccess) return fail(FP_ERR_HIP, "attention launch: %s", hipGetErrorString(e));
    return ok();
}

}  // namespace

// ---------------------------------------------------------------------------
// Scratch of the allocation-free entry point: the bf16 summary operands live
// in this device array instead of a caller workspace. Each GPU the library
// runs on holds its own copy until the process ends. In host code the name
// is only a handle: its device address on the current device comes from
// hipGetSymbolAddress, looked up once per device on the first call there.
// ---------------------------------------------------------------------------
__device__ __align__(256) uint8_t scratch[FP_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int MAX_DEVICES = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[MAX_DEVICES] = {};

int scratch_address(void** out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(FP_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
    if (dev < 0 || dev >= MAX_DEVICES) return fail(FP_ERR_UNSUPPORTED, "device %d beyond %d", dev, MAX_DEVICES);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* ptr = nullptr;
        e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !ptr)
            return fail(FP_ERR_HIP, "hipGetSymbolAddress(scratch): %s", hipGetErrorString(e));
        g_scratch_ptr[dev] = ptr;
    }
    *out = g_scratch_ptr[dev];
    return FP_OK;
}
}  // namespace

extern "C" {

int fp_sparse_prefill(const fp_problem* p, const void* q, const void* k, const void* v,
                      const float* q_scale, const float* k_scale, const float* v_scale,
                      const float* kbar, const float* vbar, const int32_t* row_ptr,
                      const int32_t* col_idx, const int32_t* sched, void* o, float* lse,
                      void* workspace, size_t ws_bytes, void* stream) {
    int rc = check_prefill("fp_sparse_prefill", p, q, k, v, q_scale, k_scale, v_scale, kbar, vbar, row_ptr,
                           col_idx, o);
    if (rc) return rc;
    if (p->variant == FP_VARIANT_BLOCK_SCORE)
        return fail(FP_ERR_INVALID, "fp_sparse_prefill: the block-score variant takes the block scores "
                                    "(fp_sparse_prefill_scored)");
    if (!workspace) return fail(FP_ERR_INVALID, "fp_sparse_prefill: NULL workspace");
    const size_t need = summary_ws_bytes(fixed_pooled_rows(p)) + split_ws_bytes(p);
    if (ws_bytes < need)
        return fail(FP_ERR_CAPACITY, "fp_sparse_prefill: workspace %zu < %zu bytes", ws_bytes, need);
    if (misaligned(workspace, ALIGN)) return fail(FP_ERR_INVALID, "workspace must be 256-byte aligned");
    return launch_prefill(p, q, k, v, q_scale, k_scale, v_scale, kbar, vbar, row_ptr, col_idx, sched, o, lse,
                          workspace, (hipStream_t)stream);
}

int fp_dense_prefill(const fp_problem* p, const void* q, const void* k, const void* v, const float* q_scale,
                     const float* k_scale, const float* v_scale, void* o, float* lse, void* stream) {
    int rc = check_fixed(p);
    if (rc) return rc;
    if (!q || !k || !v || !o) return fail(FP_ERR_INVALID, "fp_dense_prefill: NULL pointer");
    const bool fp8 = p->dtype == FP_DTYPE_FP8_E4M3;
    if (fp8 && (!q_scale || !k_scale || !v_scale))
        return fail(FP_ERR_INVALID, "fp_dense_prefill: fp8 needs q_scale, k_scale and v_scale");
    if (misaligned(q, 16) || misaligned(k, 16) || misaligned(v, 16) ||
        misaligned(o, p->out_dtype == FP_OUT_FP32 ? 16 : 8))
        return fail(FP_ERR_INVALID, "fp_dense_prefill: misaligned tensor");
    GeoFixed geo = geo_fixed(p);
    const int nsb = cdiv(p->seqlen, SCALE_TOK);
    const int G = p->num_q_heads / p->num_kv_heads;
    AttnArgs a{};
    a.q = q; a.k = k; a.v = v;
    a.qa = RowAddr{p->q_stride[0], p->q_stride[1], p->q_stride[2]};
    a.oa = RowAddr{p->o_stride[0], p->o_stride[1], p->o_stride[2]};
    a.o_f32 = p->out_dtype == FP_OUT_FP32;
    a.no_correction = 1;                 // nothing is pruned
    a.dense = 1;
    a.kv_div = 1;
    a.ka = KVAddr{p->k_stride[0], p->k_stride[1], p->k_stride[2], 0, nullptr, 0, 0};
    a.va = KVAddr{p->v_stride[0], p->v_stride[1], p->v_stride[2], 0, nullptr, 0, 0};
    a.qs = ScaleAddr{q_scale, (long long)p->num_q_heads * nsb, nsb};
    a.ks = ScaleAddr{k_scale, (long long)p->num_kv_heads * nsb, nsb};
    a.vs = ScaleAddr{v_scale, (long long)p->num_kv_heads * nsb, nsb};
    a.o = o; a.lse = lse;
    a.la = RowAddr{(long long)p->num_q_heads * p->seqlen, 1, p->seqlen};
    a.Hq = p->num_q_heads; a.Hkv = p->num_kv_heads; a.G = G;
    a.rows = p->batch * p->num_kv_heads * geo.nb;
    a.scale_log2 = default_scale(p->softmax_scale, p->head_dim) * 1.4426950408889634f;
    hipError_t e = launch_attn(&geo, nullptr, a, p->block, fp8, 0, (hipStream_t)stream);
    if (e != hipSuccess) return fail(FP_ERR_HIP, "attention launch: %s", hipGetErrorString(e));
    return ok();
}

int fp_sparse_prefill_scored(const fp_problem* p, const void* q, const void* k, const void* v,
                             const float* q_scale, const float* k_scale, const float* v_scale,
                             const float* scores, const float* vbar, const int32_t* row_ptr,
                             const int32_t* col_idx, const int32_t* sched, void* o, float* lse,
                             void* workspace, size_t ws_bytes, void* stream) {
    int rc = check_prefill("fp_sparse_prefill_scored", p, q, k, v, q_scale, k_scale, v_scale, vbar, vbar,
                           row_ptr, col_idx, o);
    if (rc) return rc;
    if (p->variant != FP_VARIANT_BLOCK_SCORE)
        return fail(FP_ERR_INVALID, "fp_sparse_prefill_scored: the problem's variant must be "
                                    "FP_VARIANT_BLOCK_SCORE");
    if (!scores || misaligned(scores, 16)) return fail(FP_ERR_INVALID, "fp_sparse_prefill_scored: scores");
    if (!workspace) return fail(FP_ERR_INVALID, "fp_sparse_prefill_scored: NULL workspace");
    const size_t need = summary_ws_bytes(fixed_pooled_rows(p)) + split_ws_bytes(p);
    if (ws_bytes < need)
        return fail(FP_ERR_CAPACITY, "fp_sparse_prefill_scored: workspace %zu < %zu bytes", ws_bytes, need);
    if (misaligned(workspace, ALIGN)) return fail(FP_ERR_INVALID, "workspace must be 256-byte aligned");
    return launch_prefill(p, q, k, v, q_scale, k_scale, v_scale, nullptr, vbar, row_ptr, col_idx, sched, o, lse,
                          workspace, (hipStream_t)stream, scores);
}

int fp_sparse_prefill_noalloc(const fp_problem* p, const void* q, const void* k, const void* v,
                              const float* q_scale, const float* k_scale, const float* v_scale,
                              const float* kbar, const float* vbar, const int32_t* row_ptr,
                              const int32_t* col_idx, const int32_t* sched, void* o, float* lse,
                              void* stream) {
    int rc = check_prefill("fp_sparse_prefill_noalloc", p, q, k, v, q_scale, k_scale, v_scale, kbar, vbar,
                           row_ptr, col_idx, o);
    if (rc) return rc;
    if (p->variant == FP_VARIANT_BLOCK_SCORE)
        return fail(FP_ERR_INVALID, "fp_sparse_prefill_noalloc: the block-score variant takes the block scores "
                                    "(fp_sparse_prefill_scored)");
    const size_t need = summary_ws_bytes(fixed_pooled_rows(p)) + split_ws_bytes(p);
    if (fixed_pooled_rows(p) > FP_NOALLOC_MAX_POOLED_ROWS || need > (size_t)FP_NOALLOC_SCRATCH_BYTES)
        return fail(FP_ERR_CAPACITY,
                    "fp_sparse_prefill_noalloc: the problem has %lld pooled rows (batch x KV heads x blocks, at "
                    "most %d) and needs %zu bytes of the %d-byte static array", fixed_pooled_rows(p),
                    FP_NOALLOC_MAX_POOLED_ROWS, need, FP_NOALLOC_SCRATCH_BYTES);
    void* ws = nullptr;
    rc = scratch_address(&ws);
    if (rc) return rc;
    return launch_prefill(p, q, k, v, q_scale, k_scale, v_scale, kbar, vbar, row_ptr, col_idx, sched, o, lse,
                          ws, (hipStream_t)stream);
}

// ---------------------------------------------------------------------------
// paged varlen
// ---------------------------------------------------------------------------
namespace {

struct VarPlan {
    std::vector<SeqDesc> table;      // nseq + 1 (last: totals)
    long long rows = 0, max_nnz = 0, sum_q = 0;
    int max_nbk = 0, total_qblocks = 0, total_kblocks = 0, total_tiles = 0;
    long long total_scores = 0;
    // workspace carve (byte offsets)
    size_t o_table = 0, o_qbar = 0, o_kbar = 0, o_vbar = 0, o_scores = 0, o_sched = 0, o_sel = 0, o_sum = 0,
           total = 0;
    SelectWs sel;
    SortPlan sort;
};

int check_varlen(const fp_varlen_problem* p, const int32_t* cu, const int32_t* lk, VarPlan& plan) {
    if (!p) return fail(FP_ERR_INVALID, "problem is NULL");
    int rc = check_heads(p->num_q_heads, p->num_kv_heads, p->head_dim, p->block);
    if (rc) return rc;
    if (p->num_seqs <= 0 || p->num_seqs > 4096) return fail(FP_ERR_INVALID, "num_seqs must be in [1, 4096]");
    if (p->dtype != FP_DTYPE_BF16 && p->dtype != FP_DTYPE_FP8_E4M3)
        return fail(FP_ERR_UNSUPPORTED, "dtype %d unsupported", p->dtype);
    const int esz = p->dtype == FP_DTYPE_FP8_E4M3 ? 1 : 2;
    if (p->page_size < 16 || p->page_size > 256 || (p->page_size & (p->page_size - 1)))
        return fail(FP_ERR_UNSUPPORTED, "page_size %d unsupported (power of two in [16, 256])", p->page_size);
    if (p->max_pages_per_seq <= 0) return fail(FP_ERR_INVALID, "max_pages_per_seq must be positive");
    if (!(p->softmax_scale >= 0.f) || isinf(p->softmax_scale))
        return fail(FP_ERR_INVALID, "softmax_scale must be finite and >= 0");
    if (!cu || !lk) return fail(FP_ERR_INVALID, "cu_seqlens_q and seqlens_k (host arrays) are required");
    if (cu[0] != 0) return fail(FP_ERR_INVALID, "cu_seqlens_q[0] must be 0");
    for (int e = 0; e < 2; ++e)
        if (p->q_stride[e] < 0 || p->o_stride[e] < 0) return fail(FP_ERR_INVALID, "negative stride");
    for (int e = 0; e < 3; ++e)
        if (p->kv_stride[e] < 0 || (p->kv_stride[e] * esz) % 16) return fail(FP_ERR_INVALID, "bad kv stride");
    if ((p->q_stride[0] * esz) % 16 || (p->q_stride[1] * esz) % 16 || (p->o_stride[0] * 2) % 8 ||
        (p->o_stride[1] * 2) % 8)
        return fail(FP_ERR_INVALID, "q/o strides must be multiples of 16/8 bytes");
    const int B = p->block;
    plan.table.assign(p->num_seqs + 1, SeqDesc{});
    long long qb = 0, kb = 0, tiles = 0, sc = 0;
    for (int b = 0; b < p->num_seqs; ++b) {
        const int ql = cu[b + 1] - cu[b];
        const int L = lk[b];
        if (ql < 0) return fail(FP_ERR_INVALID, "cu_seqlens_q not non-decreasing at %d", b);
        if (L < ql) return fail(FP_ERR_INVALID, "seqlens_k[%d] = %d < q_len %d", b, L, ql);
        const int nbk = cdiv(L, B);
        if (nbk > MAX_NB) return fail(FP_ERR_UNSUPPORTED, "sequence %d has %d blocks (max %d)", b, nbk, MAX_NB);
        if ((long long)cdiv(L, p->page_size) > p->max_pages_per_seq)
            return fail(FP_ERR_INVALID, "sequence %d needs %d pages > max_pages_per_seq", b, cdiv(L, p->page_size));
        SeqDesc& s = plan.table[b];
        s.L = L;
        s.P = L - ql;
        s.i0 = ql ? s.P / B : 0;
        s.nq = ql ? (L - 1) / B - s.i0 + 1 : 0;
        s.nbk = ql ? nbk : 0;      // a sequence with no new rows needs no pooled keys
        s.q0 = cu[b];
        s.qb0 = (int)qb;
        s.kb0 = (int)kb;
        s.row0 = (int)(qb * p->num_kv_heads);
        s.tile0 = (int)tiles;
        s.sc0 = sc;
        for (int il = 0; il < s.nq; ++il) plan.max_nnz += (long long)p->num_kv_heads * (s.i0 + il + 1);
        plan.max_nbk = std::max(plan.max_nbk, s.nbk);
        qb += s.nq;
        kb += s.nbk;
        tiles += ql ? score_tiles(s.nq, s.nbk) : 0;
        sc += (long long)p->num_q_heads * s.nq * s.nbk;
        plan.sum_q += ql;
    }
    SeqDesc& e = plan.table[p->num_seqs];
    e.qb0 = (int)qb; e.kb0 = (int)kb; e.row0 = (int)(qb * p->num_kv_heads); e.tile0 = (int)tiles; e.sc0 = sc;
    if (qb > (1 << 28) || kb > (1 << 28) || sc > (1LL << 40)) return fail(FP_ERR_UNSUPPORTED, "batch too large");
    plan.rows = qb * p->num_kv_heads;
    plan.total_qblocks = (int)qb;
    plan.total_kblocks = (int)kb;
    plan.total_tiles = (int)tiles;
    plan.total_scores = sc;
    size_t off = 0;
    plan.o_table = off; off = align_up(off + sizeof(SeqDesc) * (p->num_seqs + 1));
    plan.o_qbar = off; off = align_up(off + (size_t)qb * p->num_q_heads * D * 4);
    plan.o_kbar = off; off = align_up(off + (size_t)kb * p->num_kv_heads * D * 4);
    plan.o_vbar = off; off = align_up(off + (size_t)kb * p->num_kv_heads * D * 4);
    plan.o_scores = off; off = align_up(off + (size_t)sc * 4);
    plan.o_sched = off; off = align_up(off + (size_t)plan.rows * 4);
    plan.sort = sort_plan(kb * p->num_kv_heads, std::max(plan.max_nbk, 1), B, esz);
    plan.sel = select_ws(plan.rows, std::max(plan.max_nbk, 1), plan.sort.ngrp);
    plan.o_sel = off; off = align_up(off + plan.sel.total);
    plan.o_sum = off; off += summary_ws_bytes(kb * p->num_kv_heads);
    plan.total = off;
    return FP_OK;
}

}  // namespace

int64_t fp_varlen_num_rows(const fp_varlen_problem* p, const int32_t* cu, const int32_t* lk) {
    VarPlan plan;
    int rc = check_varlen(p, cu, lk, plan);
    return rc ? rc : plan.rows;
}

int64_t fp_varlen_max_nnz(const fp_varlen_problem* p, const int32_t* cu, const int32_t* lk) {
    VarPlan plan;
    int rc = check_varlen(p, cu, lk, plan);
    return rc ? rc : plan.max_nnz;
}

int64_t fp_varlen_workspace_size(const fp_varlen_problem* p, const int32_t* cu, const int32_t* lk) {
    VarPlan plan;
    int rc = check_varlen(p, cu, lk, plan);
    return rc ? rc : (int64_t)plan.total;
}

}  // extern "C"

namespace {

// The paged varlen path; kc / vc: the pooled-KV cache (both NULL: none).
int paged_impl(const char* who, const fp_varlen_problem* p, const void* q, const int32_t* cu,
               const int32_t* lk, const void* k_cache, const void* v_cache,
               const int32_t* block_table, const float* q_scale, const float* k_scale,
               const float* v_scale, float* kc, float* vc, float tau, int32_t* row_ptr, int32_t* col_idx,
               int64_t capacity, void* o, float* lse, void* workspace, size_t ws_bytes, void* stream) {
    VarPlan plan;
    int rc = check_varlen(p, cu, lk, plan);
    if (rc) return rc;
    if (!k_cache || !v_cache || !block_table || !row_ptr || !col_idx || !workspace)
        return fail(FP_ERR_INVALID, "%s: NULL pointer", who);
    // q and o hold sum q_len rows: they may be empty (NULL) when every sequence is fully cached
    if (plan.sum_q > 0 && (!q || !o)) return fail(FP_ERR_INVALID, "%s: NULL q or o", who);
    const bool fp8 = p->dtype == FP_DTYPE_FP8_E4M3;
    if (fp8 && (!q_scale || !k_scale || !v_scale))
        return fail(FP_ERR_INVALID, "%s: fp8 needs q_scale, k_scale and v_scale", who);
    // fp8 scales: [num_seqs, H, nsb], one per 128 positions of each sequence
    const long long nsb = ((long long)p->max_pages_per_seq * p->page_size + SCALE_TOK - 1) / SCALE_TOK;
    if (isnan(tau)) return fail(FP_ERR_INVALID, "%s: tau is NaN", who);
    if (capacity < plan.max_nnz)
        return fail(FP_ERR_CAPACITY, "%s: capacity %lld < max nnz %lld", who, (long long)capacity, plan.max_nnz);
    if (ws_bytes < plan.total)
        return fail(FP_ERR_CAPACITY, "%s: workspace %zu < %zu bytes", who, ws_bytes, plan.total);
    if (misaligned(workspace, ALIGN)) return fail(FP_ERR_INVALID, "workspace must be 256-byte aligned");
    if (misaligned(q, 16) || misaligned(k_cache, 16) || misaligned(v_cache, 16) || misaligned(o, 8) ||
        misaligned(kc, 16) || misaligned(vc, 16))
        return fail(FP_ERR_INVALID, "%s: misaligned tensor", who);
    if (plan.rows == 0) {
        // nothing to attend: the kept lists are empty, row_ptr = {0}
        hipError_t e = launch_zero_first(row_ptr, (hipStream_t)stream);
        if (e != hipSuccess) return fail(FP_ERR_HIP, "row_ptr write: %s", hipGetErrorString(e));
        return ok();
    }

    char* ws = (char*)workspace;
    SeqDesc* dtable = (SeqDesc*)(ws + plan.o_table);
    float* qbar = (float*)(ws + plan.o_qbar);
    float* kbar = (float*)(ws + plan.o_kbar);
    float* vbar = (float*)(ws + plan.o_vbar);
    float* scores = (float*)(ws + plan.o_scores);
    int32_t* sched = (int32_t*)(ws + plan.o_sched);
    char* selws = ws + plan.o_sel;
    hipStream_t st = (hipStream_t)stream;

    GeoTable geo;
    geo.t = dtable;
    geo.nseq = p->num_seqs;
    geo.Hq = p->num_q_heads;
    geo.Hkv = p->num_kv_heads;
    geo.blk = p->block;
    int shift = 0;
    while ((1 << shift) < p->page_size) ++shift;
    const KVAddr kva{0, p->kv_stride[1], p->kv_stride[2], p->kv_stride[0], block_table,
                     p->max_pages_per_seq, shift};

    hipError_t e = launch_table_copy(plan.table.data(), p->num_seqs + 1, dtable, st);
    if (e != hipSuccess) return fail(FP_ERR_HIP, "table copy: %s", hipGetErrorString(e));

    PoolArgs pa{};
    pa.q = q; pa.k = k_cache; pa.v = v_cache;
    pa.qa = RowAddr{0, p->q_stride[0], p->q_stride[1]};
    pa.ka = kva; pa.va = kva;
    pa.qs = ScaleAddr{q_scale, p->num_q_heads * nsb, nsb};
    pa.ks = ScaleAddr{k_scale, p->num_kv_heads * nsb, nsb};
    pa.vs = ScaleAddr{v_scale, p->num_kv_heads * nsb, nsb};
    pa.qbar = qbar; pa.kbar = kbar; pa.vbar = vbar;
    pa.Hq = p->num_q_heads; pa.Hkv = p->num_kv_heads; pa.blk = p->block;
    pa.fp8 = fp8; pa.paged = 1;
    pa.total_qblocks = plan.total_qblocks; pa.total_kblocks = plan.total_kblocks;
    pa.kc = kc; pa.vc = vc;
    pa.spp = std::max(1, p->page_size / p->block);
    e = launch_pool(nullptr, &geo, pa, st);
    if (e != hipSuccess) return fail(FP_ERR_HIP, "pool launch: %s", hipGetErrorString(e));

    ScoreArgs sa;
    sa.qbar = qbar; sa.kbar = kbar; sa.scores = scores;
    sa.Hq = p->num_q_heads; sa.Hkv = p->num_kv_heads;
    sa.total_tiles = plan.total_tiles;
    sa.scale = default_scale(p->softmax_scale, p->head_dim);
    e = launch_scores(nullptr, &geo, sa, st);
    if (e != hipSuccess) return fail(FP_ERR_HIP, "scores launch: %s", hipGetErrorString(e));

    SelectArgs se;
    se.scores = scores;
    se.counts = (int32_t*)(selws + plan.sel.counts);
    se.bits = (uint32_t*)(selws + plan.sel.bits);
    se.keys = (int32_t*)(selws + plan.sel.keys);
    se.maxc = (int32_t*)(selws + plan.sel.maxc);
    se.hist = (int32_t*)(selws + plan.sel.hist);
    se.nbw = plan.sel.nbw;
    se.row_ptr = row_ptr; se.col_idx = col_idx; se.sched = sched;
    se.Hq = p->num_q_heads; se.Hkv = p->num_kv_heads;
    se.rows = (int)plan.rows; se.max_nbk = std::max(plan.max_nbk, 1);
    se.ngrp = plan.sort.ngrp; se.grp_units = plan.sort.grp_units;
    se.neg_tau = -tau;
    se.kv_div = 1; se.Hkv_pool = p->num_kv_heads;
    e = launch_select(nullptr, &geo, se, st);
    if (e != hipSuccess) return fail(FP_ERR_HIP, "select launch: %s", hipGetErrorString(e));

    const int G = p->num_q_heads / p->num_kv_heads;
    AttnArgs a{};
    a.q = q; a.k = k_cache; a.v = v_cache;
    a.qa = RowAddr{0, p->q_stride[0], p->q_stride[1]};
    a.oa = RowAddr{0, p->o_stride[0], p->o_stride[1]};
    a.ka = kva; a.va = kva;
    a.kv_div = 1;
    // per-lane in-page offsets of a tile are kept in 24 bits
    a.paged_fast = (long long)std::min(p->page_size, p->block) * p->kv_stride[1] * (fp8 ? 1 : 2) < (1LL << 24);
    a.qs = pa.qs; a.ks = pa.ks; a.vs = pa.vs;
    a.kbar = kbar; a.vbar = vbar;
    {
        const size_t part = align_up((size_t)plan.total_kblocks * p->num_kv_heads * D * 2);
        a.kbar_hi = (const __bf16*)(ws + plan.o_sum);
        a.kbar_lo = (const __bf16*)(ws + plan.o_sum + part);
        a.vbar_bf = (const __bf16*)(ws + plan.o_sum + 2 * part);
    }
    a.row_ptr = row_ptr; a.col_idx = col_idx; a.sched = sched;
    a.o = o; a.lse = lse;
    a.la = RowAddr{0, 1, plan.sum_q};
    a.Hq = p->num_q_heads; a.Hkv = p->num_kv_heads; a.G = G;
    a.rows = (int)plan.rows;
    a.slices = cdiv(G * p->block, 128);
    a.scale_log2 = default_scale(p->softmax_scale, p->head_dim) * 1.4426950408889634f;
    e = launch_summary_prep(kbar, vbar, (__bf16*)a.kbar_hi, (__bf16*)a.kbar_lo, (__bf16*)a.vbar_bf,
                            (long long)plan.total_kblocks * p->num_kv_heads * D, st);
    if (e != hipSuccess) return fail(FP_ERR_HIP, "summary prep launch: %s", hipGetErrorString(e));
    e = launch_attn(nullptr, &geo, a, p->block, fp8, 1, st);
    if (e != hipSuccess) return fail(FP_ERR_HIP, "attention launch: %s", hipGetErrorString(e));
    return ok();
}

}  // namespace

extern "C" {

int fp_sparse_prefill_paged(const fp_varlen_problem* p, const void* q, const int32_t* cu,
                            const int32_t* lk, const void* k_cache, const void* v_cache,
                            const int32_t* block_table, const float* q_scale, const float* k_scale,
                            const float* v_scale, float tau, int32_t* row_ptr, int32_t* col_idx,
                            int64_t capacity, void* o, float* lse, void* workspace, size_t ws_bytes,
                            void* stream) {
    return paged_impl("fp_sparse_prefill_paged", p, q, cu, lk, k_cache, v_cache, block_table, q_scale, k_scale,
                      v_scale, nullptr, nullptr, tau, row_ptr, col_idx, capacity, o, lse, workspace, ws_bytes,
                      stream);
}

int fp_sparse_prefill_paged_cached(const fp_varlen_problem* p, const void* q, const int32_t* cu,
                                   const int32_t* lk, const void* k_cache, const void* v_cache,
                                   const int32_t* block_table, const float* q_scale, const float* k_scale,
                                   const float* v_scale, float* kbar_cache, float* vbar_cache, float tau,
                                   int32_t* row_ptr, int32_t* col_idx, int64_t capacity, void* o, float* lse,
                                   void* workspace, size_t ws_bytes, void* stream) {
    if (!kbar_cache || !vbar_cache)
        return fail(FP_ERR_INVALID, "fp_sparse_prefill_paged_cached: NULL kbar_cache or vbar_cache");
    return paged_impl("fp_sparse_prefill_paged_cached", p, q, cu, lk, k_cache, v_cache, block_table, q_scale,
                      k_scale, v_scale, kbar_cache, vbar_cache, tau, row_ptr, col_idx, capacity, o, lse, workspace,
                      ws_bytes, stream);
}

}  // extern "C"
