// Internal declarations shared by the HIP kernels and the C-ABI host code.
// gfx950 (CDNA4) only: wave64, MFMA, 160 KiB LDS per CU.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

// Index arithmetic is callable from host code too (FP_HD), so host programs
// can replay a launch's addresses and check them against buffer extents.
#define FP_HD __host__ __device__ __forceinline__

namespace fp {

constexpr int D = 128;            // head dim
constexpr int MAX_G = 16;         // query heads per KV head
constexpr int MAX_NB = 16384;     // key blocks per sequence
constexpr int SCALE_TOK = 128;    // tokens per fp8 scale

// ---------------------------------------------------------------------------
// Sequence geometry. Blocks live on the absolute-position grid of each
// sequence: query block i covers present rows [max(iB, P), min((i+1)B, L)),
// key block j covers [jB, min((j+1)B, L)).
// ---------------------------------------------------------------------------
struct SeqDesc {
    int L;        // keys (cache + new chunk)
    int P;        // cached prefix (first present query row)
    int i0;       // first query block
    int nq;       // query blocks
    int nbk;      // key blocks
    int q0;       // packed row of token P in q / o / lse (varlen); 0 for fixed
    int qb0;      // query blocks of earlier sequences (pooled-Q offset)
    int kb0;      // key blocks of earlier sequences (pooled-K/V offset)
    int row0;     // kept-list rows of earlier sequences (= Hkv * qb0)
    int tile0;    // score tiles of earlier sequences
    long long sc0;  // score-matrix elements of earlier sequences
};

constexpr int SC_TILE = 64;       // score tile edge (query blocks x key blocks)

__host__ __device__ inline int cdiv(int a, int b) { return (a + b - 1) / b; }
__host__ __device__ inline int score_tiles(int nq, int nbk) {
    return cdiv(nq, SC_TILE) * cdiv(nbk, SC_TILE);
}

// Fixed shape: every sequence has S tokens and no prefix. Everything is
// arithmetic; no table in memory.
struct GeoFixed {
    static constexpr bool PAGED_KV = false;   // contiguous K/V
    int nseq, S, Hq, Hkv, blk, nb, ntile;
    FP_HD SeqDesc seq(int b) const {
        SeqDesc s;
        s.L = S; s.P = 0; s.i0 = 0; s.nq = nb; s.nbk = nb; s.q0 = 0;
        s.qb0 = b * nb; s.kb0 = b * nb; s.row0 = b * Hkv * nb; s.tile0 = b * ntile;
        s.sc0 = (long long)b * Hq * nb * nb;
        return s;
    }
    FP_HD int seq_of_qblock(int u) const { return u / nb; }
    FP_HD int seq_of_kblock(int u) const { return u / nb; }
    FP_HD int seq_of_row(int r) const { return r / (Hkv * nb); }
    FP_HD int seq_of_tile(int u) const { return u / ntile; }
};

// Varlen: a table of nseq descriptors in device memory, entry nseq holding
// the running totals (qb0, kb0, row0, tile0, sc0) past the last sequence.
struct GeoTable {
    static constexpr bool PAGED_KV = true;    // K/V in the paged cache
    const SeqDesc* t;
    int nseq, Hq, Hkv, blk;
    FP_HD SeqDesc seq(int b) const { return t[b]; }
    // largest b in [0, nseq) with field(b) <= u (empty sequences share the
    // next one's offset, so ties resolve to the last, non-empty, one)
#define FP_SEARCH(FIELD)                                              \
    int lo = 0, hi = nseq;                                            \
    while (hi - lo > 1) {                                             \
        int mid = (lo + hi) >> 1;                                     \
        if (t[mid].FIELD <= u) lo = mid; else hi = mid;               \
    }                                                                 \
    return lo;
    FP_HD int seq_of_qblock(int u) const { FP_SEARCH(qb0) }
    FP_HD int seq_of_kblock(int u) const { FP_SEARCH(kb0) }
    FP_HD int seq_of_row(int r) const { int u = r; FP_SEARCH(row0) }
    FP_HD int seq_of_tile(int u) const { FP_SEARCH(tile0) }
#undef FP_SEARCH
};

// Token addressing (element offsets; the head dim is contiguous).
// q / o / lse rows: b * sb + (q0 + t - P) * st + h * sh   (varlen: sb = 0)
struct RowAddr {
    long long sb, st, sh;
    FP_HD long long off(int b, const SeqDesc& s, int t, int h) const {
        return (long long)b * sb + (long long)(s.q0 + t - s.P) * st + (long long)h * sh;
    }
};

// k / v: contiguous  b * sb + s * st + g * sh
//        paged       table[b * maxp + s / page] * spage + (s % page) * st + g * sh
struct KVAddr {
    long long sb, st, sh, spage;
    const int* table;
    int maxp, page_shift;
    template <bool PAGED>
    FP_HD long long off(int b, int s, int g) const {
        if (PAGED) {
            int pg = table[(long long)b * maxp + (s >> page_shift)];
            return (long long)pg * spage + (long long)(s & ((1 << page_shift) - 1)) * st +
                   (long long)g * sh;
        }
        return (long long)b * sb + (long long)s * st + (long long)g * sh;
    }
    // paged offset with the page id already looked up
    FP_HD long long off_page(int pg, int s, int g) const {
        return (long long)pg * spage + (long long)(s & ((1 << page_shift) - 1)) * st + (long long)g * sh;
    }
};

// Pooled tensors: Qbar [qb0*Hq + h*nq + il], Kbar/Vbar [kb0*Hkv + g*nbk + j], rows of D floats.
FP_HD long long qbar_row(const SeqDesc& s, int Hq, int h, int il) {
    return (long long)s.qb0 * Hq + (long long)h * s.nq + il;
}
FP_HD long long kbar_row(const SeqDesc& s, int Hkv, int g, int j) {
    return (long long)s.kb0 * Hkv + (long long)g * s.nbk + j;
}
// Scores: [sc0 + (h*nq + il) * nbk + j]
FP_HD long long score_off(const SeqDesc& s, int h, int il, int j) {
    return s.sc0 + ((long long)h * s.nq + il) * s.nbk + j;
}

// fp8 scales: [b][H][nsb] with nsb = scale_stride_h, b stride = scale_stride_b
struct ScaleAddr {
    const float* p;
    long long sb, sh;
    FP_HD float at(int b, int h, int t) const {
        return p[(long long)b * sb + (long long)h * sh + (t >> 7)];
    }
};

// ---------------------------------------------------------------------------
// launchers (defined in the .hip files); all return hipError_t of the launch
// ---------------------------------------------------------------------------
struct PoolArgs {
    const void* q; const void* k; const void* v;
    RowAddr qa; KVAddr ka, va;
    ScaleAddr qs, ks, vs;
    float* qbar; float* kbar; float* vbar;
    int Hq, Hkv, blk, fp8, paged;
    int total_qblocks, total_kblocks;
    // pooled-KV cache beside the page cache (NULL: none): fp32 [slots, Hkv, D]
    float* kc; float* vc;
    int spp;                                    // slots per page: max(1, page / blk)
    // slot of complete key block j of sequence b: the page of its last token
    FP_HD long long cache_row(int b, int j, int head) const {
        const int e = (j + 1) * blk - 1;
        const long long pg = ka.table[(long long)b * ka.maxp + (e >> ka.page_shift)];
        const int in_page = (e & ((1 << ka.page_shift) - 1)) / blk;
        return ((pg * spp + in_page) * Hkv + head) * D;
    }
};

struct ScoreArgs {
    const float* qbar; const float* kbar; float* scores;
    int Hq, Hkv, total_tiles;
    float scale;
};

constexpr int SORT_CHUNK = 256;    // rows per chunk of the schedule sort

struct SelectArgs {
    const float* scores;
    int32_t* counts; uint32_t* bits; int nbw;   // bitmask row stride (u32 words)
    int32_t* keys;                              // [rows] schedule group of the row
    int32_t* maxc;                              // largest kept count (written by the scan)
    int32_t* hist;                              // [chunks][ngrp * (largest count + 1)] sort histograms / offsets
    int32_t* row_ptr; int32_t* col_idx; int32_t* sched;
    int Hq, Hkv, rows, max_nbk;
    int ngrp;                                   // schedule groups (rows sharing a K/V working set)
    long long grp_units;                        // group size in (key block x KV head) units
    float neg_tau;
    // fused estimate + threshold (scores == nullptr): pooled rows and the softmax scale
    const float* qbar; const float* kbar; float scale;
    int kv_div, Hkv_pool;                       // pooled keys of list group g: KV head g / kv_div of Hkv_pool
};

// Fused block scores + threshold: the workgroup's S columns (query block x
// query head) and the largest key-block count whose S rows fit its LDS.
constexpr int FUSED_COLS = 32;
constexpr int FUSED_MAX_NBK = 1024;

// Schedule group of the rows of (sequence s, KV head g): the (sequence, KV
// head) pairs in row order are cut into groups of grp_units key blocks' worth
// of K/V, by where the pair's K/V starts.
__host__ __device__ inline int row_group(const SeqDesc& s, int g, int Hkv, long long grp_units, int ngrp) {
    const long long start = (long long)Hkv * s.kb0 + (long long)g * s.nbk;
    const long long grp = start / grp_units;
    return (int)(grp < ngrp - 1 ? grp : ngrp - 1);
}

struct AttnArgs {
    const void* q; const void* k; const void* v;
    RowAddr qa, oa; KVAddr ka, va;
    ScaleAddr qs, ks, vs;
    const float* kbar; const float* vbar;
    const __bf16* kbar_hi; const __bf16* kbar_lo; const __bf16* vbar_bf;   // summary operands
    const int32_t* row_ptr; const int32_t* col_idx; const int32_t* sched;
    void* o; float* lse; RowAddr la;   // lse offset: b*sb + (q0+t-P)*st + h*sh
    int Hq, Hkv, G, rows, slices;
    float scale_log2;                  // c * log2(e)
    int o_f32;                         // o in fp32 (diagnostic) instead of bf16
    int paged_fast;                    // paged: in-page offsets of a tile fit 24 bits (precomputed per lane)
    int no_correction;                 // ablation: pruned blocks dropped (no summary tiles)
    int dense;                         // every block j <= i kept, no kept lists read (dense causal attention)
    int kv_div;                        // KV head of kept-list row group g: g / kv_div (G with per-head lists, else 1)
    const float* scores;               // block-score correction: pseudo-token logit S[b,h,i,j] + ln|J| (else null)
    int nsplit;                        // parts per row's tile sequence (split_count; 0 or 1: off)
    float* part_o; float* part_ml;     // split: per-part unnormalised O and (m, l), merged afterwards
};

hipError_t launch_pool(const GeoFixed* gf, const GeoTable* gt, const PoolArgs& a, hipStream_t st);
hipError_t launch_scores(const GeoFixed* gf, const GeoTable* gt, const ScoreArgs& a, hipStream_t st);
hipError_t launch_select(const GeoFixed* gf, const GeoTable* gt, const SelectArgs& a, hipStream_t st);
// E2-E5 without a score matrix (fixed shape, key blocks <= FUSED_MAX_NBK), then the same compaction
hipError_t launch_select_fused(const GeoFixed& gf, const SelectArgs& a, hipStream_t st);
hipError_t launch_attn(const GeoFixed* gf, const GeoTable* gt, const AttnArgs& a, int blk,
                       int fp8, int paged, hipStream_t st);
hipError_t launch_summary_prep(const float* kbar, const float* vbar, __bf16* hi, __bf16* lo,
                               __bf16* vb, long long nfloats, hipStream_t st);
hipError_t launch_table_copy(const SeqDesc* host, int n, SeqDesc* dev, hipStream_t st);
hipError_t launch_zero_first(int32_t* p, hipStream_t st);

}  // namespace fp
