// Address arithmetic of the sparse attention kernel (k_attn.hip), callable
// from host code as well: the kernel computes every global and LDS address
// through these functions, and a host replay (tests/c/attn_replay.cpp) runs
// the same functions over whole launches to check each access against the
// extents of the buffers and of the LDS allocation.
#pragma once

#include "fp_internal.h"

#if defined(__HIP_DEVICE_COMPILE__)
#define FP_UNIFORM(x) __builtin_amdgcn_readfirstlane(x)
#else
#define FP_UNIFORM(x) (x)
#endif

namespace fp {

// ---------------------------------------------------------------------------
// Tile layouts in LDS (128 dims per row). The LDS banks repeat every 256
// bytes; reads that would land on one bank group are spread either by
// padding the rows or by rotating each row's bytes:
//   bf16 K rows every 272 bytes: the QK^T operand read (16 lanes = 16 rows
//     at one 16-byte chunk) lands on 16 distinct 4-bank groups;
//   bf16 V rows every 256 bytes (no padding), row r's bytes rotated by
//     64 (r mod 4): a transpose read covers 8 rows x 64 bytes, served 32 lanes
//     (4 rows, r mod 4 = 0..3) at a time, on 4 disjoint 64-byte bank groups;
//   fp8 K rows every 144 bytes (16 mod 256, as bf16 K);
//   fp8 V rows every 128 bytes, keys permuted inside each 64-key step (bits 2
//     and 3 swapped) so that each 32-lane half of a transpose read covers 8
//     consecutive rows x 32 bytes, and row r's bytes rotated by
//     32 ((r / 2) mod 4): those 8 rows land on 8 disjoint 32-byte bank groups.
// Padding keeps an operand address lane_base + immediate; a rotation needs
// one lane base per 32-dim block of V (4), which the V reads can afford, and
// it saves the direct loads of the padding (V: 20% of its pieces).
// Summary tiles (pooled keys hi/lo and pooled values) use the bf16 layouts.
// ---------------------------------------------------------------------------
constexpr int KSTR = 272;
constexpr int VSTR = 256;
constexpr int KSTR8 = 144;
constexpr int VSTR8 = 128;
constexpr int PIECE = 1024;                 // LDS bytes one wavefront load instruction fills

// swap bits 2 and 3 of a key index
FP_HD int vt_slot(int key) { return (key & ~0xC) | ((key >> 1) & 4) | ((key << 1) & 8); }

template <int BLK, bool FP8>
struct TileGeom {
    static constexpr int ESZ = FP8 ? 1 : 2;
    static constexpr int KS = FP8 ? KSTR8 : KSTR;
    static constexpr int VS = FP8 ? VSTR8 : VSTR;
    static constexpr int NKB = BLK / 32;             // 32-key blocks per tile
    static constexpr int SUMC = BLK / 2;             // pooled columns per summary sub-tile
    static constexpr int SB = NKB / 2;               // 32-column blocks per summary sub-tile
    static constexpr int KTILE = BLK * KSTR;         // bytes: a bf16 or fp8 K tile, or a summary K tile
    static constexpr int VTILE_KEPT = BLK * VS;
    static constexpr int VTILE_SUM = SUMC * VSTR;
    static constexpr int VTILE = VTILE_KEPT > VTILE_SUM ? VTILE_KEPT : VTILE_SUM;
    static constexpr int KPIECES = BLK * KS / PIECE;
    static constexpr int VPIECES = BLK * VS / PIECE;
    static constexpr int SKPIECES = BLK * KSTR / PIECE;   // summary K: hi rows then lo rows
    static constexpr int SVPIECES = SUMC * VSTR / PIECE;
    static_assert(BLK * KS % PIECE == 0 && BLK * VS % PIECE == 0 && SUMC * VSTR % PIECE == 0, "whole pieces");
};

// Lane `lane` of the load of piece t (stride STR) fills LDS bytes
// t * 1024 + 16 lane .. + 15: tile row `row`, 16-byte data chunk `ch` of it.
// Padded rows: chunks past the row's data (the padding, never read) take a
// copy of the row's last data chunk, so the lane's source shares a cache line
// with its neighbour's and no lane of a load has to be masked off. Rotated
// rows (the V layouts): LDS chunk position p of row r holds data chunk
// p - rot(r), modulo the chunks per row.
struct PieceLoc {
    int row, ch;
};
FP_HD PieceLoc piece_loc(int STR, int t, int lane, int data_chunks) {
    const int pb = t * PIECE + lane * 16;
    const int row = pb / STR;
    const int ch = (pb - row * STR) >> 4;
    if (STR == VSTR) return PieceLoc{row, (ch - 4 * (row & 3)) & 15};
    if (STR == VSTR8) return PieceLoc{row, (ch - 2 * ((row >> 1) & 3)) & 7};
    return PieceLoc{row, ch < data_chunks ? ch : data_chunks - 1};
}

// Per-lane byte offsets (from the tile's first key row) of the pieces this
// lane loads for contiguous K/V, computed once per workgroup; wavefront w of
// NW loads pieces w, w + NW, ... (piece k * NW + w exists for k < NP - 1 on
// every wavefront, for the last k only when has(k, w)). Unsigned 32-bit
// offsets from a uniform base let each load use the scalar-base form.
template <int STR, int BLK, int ESZ, bool PERM, int NW>
struct TileOffs {
    static constexpr int PIECES = BLK * STR / PIECE;
    static constexpr int NP = (PIECES + NW - 1) / NW;
    uint32_t off[NP];
    // whether wavefront `wave` loads a k-th piece (uniform; compile-time true but for the last k)
    static FP_HD bool has(int k, int wave) { return k < NP - 1 || PIECES % NW == 0 || k * NW + wave < PIECES; }
    FP_HD void init(long long tok_stride, int wave, int lane) {
#pragma unroll
        for (int k = 0; k < NP; ++k) {
            const PieceLoc pl = piece_loc(STR, k * NW + wave, lane, 8 * ESZ);
            const int key = PERM ? vt_slot(pl.row) : pl.row;
            off[k] = has(k, wave) ? (uint32_t)(key * tok_stride * ESZ + pl.ch * 16) : 0u;
        }
    }
    // Paged K/V: key `key` of a tile lies in page slot key >> lshift of the
    // tile (lshift = log2 min(page, BLK)) at in-page row key & (2^lshift - 1);
    // off packs the in-page byte offset (low 24 bits) with the slot.
    FP_HD void init_paged(long long tok_stride, int lshift, int wave, int lane) {
#pragma unroll
        for (int k = 0; k < NP; ++k) {
            const PieceLoc pl = piece_loc(STR, k * NW + wave, lane, 8 * ESZ);
            const int key = PERM ? vt_slot(pl.row) : pl.row;
            const uint32_t inpage = (uint32_t)((key & ((1 << lshift) - 1)) * tok_stride * ESZ + pl.ch * 16);
            off[k] = has(k, wave) ? (inpage | ((uint32_t)(key >> lshift) << 24)) : 0u;
        }
    }
    // byte address, relative to the tensor base, of piece k of a full
    // contiguous tile whose first key row is at byte tile_base
    FP_HD long long src_full(long long tile_base, int k) const { return tile_base + off[k]; }
    // paged: the page slot of piece k within the tile and its in-page byte offset
    FP_HD int page_slot(int k) const { return (int)(off[k] >> 24); }
    FP_HD uint32_t in_page(int k) const { return off[k] & 0xFFFFFFu; }
};

// Byte offset (relative to the tensor base) of the 16 bytes lane `lane`
// loads for piece t (< the tile's pieces) of key block j in the generic path
// (ragged tile, or a paged tile without the fast offsets). Rows past the
// sequence repeat its last key. pages: the sequence's page ids (staged), or
// have_pages false to read the block table.
template <int STR, int BLK, int ESZ, bool PERM, bool PAGED, typename PageFn>
FP_HD long long tile_src(const KVAddr& ka, int b, int L, int g, int j, int t, int lane, PageFn pages,
                         bool have_pages) {
    const PieceLoc pl = piece_loc(STR, t, lane, 8 * ESZ);
    const int key = PERM ? vt_slot(pl.row) : pl.row;
    const int rmax = L - 1 - j * BLK;
    const int sk = j * BLK + (key < rmax ? key : rmax);
    const long long off = PAGED && have_pages ? ka.off_page(pages(sk >> ka.page_shift), sk, g)
                                              : ka.template off<PAGED>(b, sk, g);
    return off * ESZ + pl.ch * 16;
}

// Summary sub-tile m (pooled columns [SUMC m, SUMC m + SUMC)): lane `lane`
// of piece t of the K (w = 0) or V (w = 1) part. K rows 0 .. SUMC-1 hold the
// bf16 hi parts of those pooled keys, rows SUMC .. BLK-1 the lo parts; V rows
// the bf16 pooled values. Returns the element offset into the hi / lo / V
// array (which = 0, 1, 2). Columns past the sequence's last block repeat it
// (they are masked out).
struct SummarySrc {
    int which;
    long long off;
};
template <int BLK>
FP_HD SummarySrc summary_src(const SeqDesc& s, int Hkv, int g, int m, int w, int t, int lane) {
    constexpr int SUMC = BLK / 2;
    const PieceLoc pl = piece_loc(w == 0 ? KSTR : VSTR, t, lane, 16);
    const int part = w == 0 && pl.row >= SUMC;          // 0 hi / 1 lo (K rows)
    const int jc = SUMC * m + pl.row - part * SUMC;
    const int jp = jc < s.nbk - 1 ? jc : s.nbk - 1;
    return SummarySrc{w == 0 ? part : 2, kbar_row(s, Hkv, g, jp) * D + pl.ch * 8};
}

// Per-lane byte offsets of a whole summary sub-tile's loads (every pooled
// column of it inside the sequence, so none repeats), computed once per
// workgroup. Relative to the sub-tile's first hi row in the hi array, K piece
// k * NW + w (wavefront w) reads at k_off[k]: its lo rows sit lo_delta bytes
// further (the distance from the hi array to the lo array). The V pieces repeat
// one pattern (4 rows of 256 bytes per piece, rotation period 4 rows): piece t
// reads at v_off + t * PIECE from the sub-tile's first row in the V array.
// summary_src gives the same addresses for these sub-tiles.
template <int BLK, int NW>
struct SumOffs {
    using TG = TileGeom<BLK, false>;
    static constexpr int NPK = (TG::SKPIECES + NW - 1) / NW;
    static constexpr int NPV = (TG::SVPIECES + NW - 1) / NW;
    uint32_t k_off[NPK];
    uint32_t v_off;
    static FP_HD bool has_k(int k, int wave) { return k * NW + wave < TG::SKPIECES; }
    static FP_HD bool has_v(int k, int wave) { return k * NW + wave < TG::SVPIECES; }
    FP_HD void init(uint32_t lo_delta, int wave, int lane) {
#pragma unroll
        for (int k = 0; k < NPK; ++k) {
            const PieceLoc pl = piece_loc(KSTR, k * NW + wave, lane, 16);
            const int part = pl.row >= TG::SUMC;
            k_off[k] = has_k(k, wave) ? (part ? lo_delta : 0u) + (uint32_t)((pl.row - part * TG::SUMC) * D * 2 +
                                                                           pl.ch * 16)
                                      : 0u;
        }
        const PieceLoc pv = piece_loc(VSTR, 0, lane, 16);
        v_off = (uint32_t)(pv.row * D * 2 + pv.ch * 16);
    }
    // sub-tile m of a sequence with nbk key blocks takes these offsets when all its columns exist
    static FP_HD bool whole(int m, int nbk) { return (m + 1) * TG::SUMC <= nbk; }
};

// ---------------------------------------------------------------------------
// Work units. Unit u of the grid runs one 256-row slice of one kept-list row,
// or, when the row's tiles are split, one part of that slice's tile sequence:
// u % 8 picks the XCD, and the slices and parts of a row sit on one XCD so
// they share its L2 copy of the K/V tiles.
// ---------------------------------------------------------------------------
struct UnitMap {
    int pidx, slice, split;
};
FP_HD UnitMap unit_map(int u, int slices, int nsplit = 1) {
    const int xcd = u & 7, k8 = u >> 3, per = slices * nsplit;
    const int rem = k8 % per;
    return UnitMap{8 * (k8 / per) + xcd, rem % slices, rem / slices};
}

// 256-row slices per kept-list row: G query heads x BLK tokens, packed
constexpr int SLICE_ROWS = 256;
FP_HD int attn_slices(int G, int blk) { return (G * blk + SLICE_ROWS - 1) / SLICE_ROWS; }

// Split rows: a grid with fewer units than the chip's 256 compute units
// splits each row's tile sequence into parts run by separate workgroups, as
// many as bring the grid to about 256 units (at most SPLIT_MAX); each part
// leaves its unnormalised (O, m, l) and a merge pass combines them. 1 = off.
constexpr int SPLIT_MAX = 8;
constexpr int SPLIT_TARGET_UNITS = 256;
FP_HD int split_count(int rows, int slices) {
    const long long units = (long long)((rows + 7) / 8) * 8 * slices;
    const long long n = units > 0 ? SPLIT_TARGET_UNITS / units : 1;
    return n < 2 ? 1 : (n > SPLIT_MAX ? SPLIT_MAX : (int)n);
}
// floats of the partial results: O [parts][256][128], then (m, l) [parts][256][2]
FP_HD long long split_parts(int rows, int slices, int nsplit) { return (long long)rows * slices * nsplit; }
FP_HD long long split_o_floats(long long parts) { return parts * SLICE_ROWS * D; }
FP_HD long long split_floats(long long parts) { return parts * SLICE_ROWS * (D + 2); }
FP_HD long long split_part(int pidx, int slices, int slice, int nsplit, int split) {
    return ((long long)pidx * slices + slice) * nsplit + split;
}
// tiles [first, first + count) of a sequence of T tiles for part `split`
struct SplitRange {
    int first, count;
};
FP_HD SplitRange split_range(int T, int split, int nsplit) {
    const int a = (int)((long long)T * split / nsplit), z = (int)((long long)T * (split + 1) / nsplit);
    return SplitRange{a, z - a};
}

// Packed query row of (slice, wavefront, row group, lane): NW wavefronts x RG
// groups x 32 rows = 256 rows per slice, token-major over the G heads.
template <int NW>
FP_HD int packed_row(int slice, int wave, int rg, int n) {
    constexpr int RG = 8 / NW;
    return slice * 256 + wave * (32 * RG) + rg * 32 + n;
}

// ---------------------------------------------------------------------------
// Tile sequence of a row: the kept blocks in column order (codes >= 0 are
// block indices), then the summary sub-tiles holding at least one pruned
// column (code -1 - m for sub-tile m), then NONE. `kept` is the row's kept
// bitmap (bit j of word j / 32), i the row's diagonal block.
// ---------------------------------------------------------------------------
constexpr int TILE_NONE = -0x7fffffff;

FP_HD uint32_t range_bits(int c0, int lo, int hi) {
    const int a = lo - c0 > 0 ? lo - c0 : 0, z = hi - c0 < 31 ? hi - c0 : 31;
    if (a > z) return 0u;
    return (0xFFFFFFFFu >> (31 - z)) & (0xFFFFFFFFu << a);
}

template <int SUMC, typename Bits>
FP_HD int next_summary(const Bits& kept, int i, int m0, bool no_correction) {
    if (no_correction) return TILE_NONE;                  // ablation: no pseudo-tokens
    for (int mm = m0; mm * SUMC <= i - 1; ++mm) {
        const int c_lo = mm * SUMC > 1 ? mm * SUMC : 1;
        const int c_hi = mm * SUMC + SUMC - 1 < i - 1 ? mm * SUMC + SUMC - 1 : i - 1;
        uint32_t anyw = 0u;
        for (int wd = c_lo >> 5; wd <= (c_hi >> 5); ++wd) anyw |= ~kept[wd] & range_bits(wd * 32, c_lo, c_hi);
        if (anyw) return -1 - mm;
    }
    return TILE_NONE;
}

// number of summary sub-tiles of a row, and the code of its k-th one (k < that number)
template <int SUMC, typename Bits>
FP_HD int count_summary(const Bits& kept, int i, bool no_correction) {
    int n = 0;
    for (int c = next_summary<SUMC>(kept, i, 0, no_correction); c != TILE_NONE;
         c = next_summary<SUMC>(kept, i, -c, no_correction))
        ++n;
    return n;
}
template <int SUMC, typename Bits>
FP_HD int nth_summary(const Bits& kept, int i, int k, bool no_correction) {
    int c = next_summary<SUMC>(kept, i, 0, no_correction);
    for (int e = 0; e < k && c != TILE_NONE; ++e) c = next_summary<SUMC>(kept, i, -c, no_correction);
    return c;
}

template <int SUMC, typename Bits>
FP_HD int next_code(const Bits& kept, int i, int code, bool no_correction) {
    if (code >= 0) {
        int wd = (code + 1) >> 5;
        uint32_t w = code + 1 <= i ? kept[wd] & (~0u << ((code + 1) & 31)) : 0u;
        while (w == 0u && wd < (i >> 5)) w = kept[++wd];
        w = FP_UNIFORM(w);
        wd = FP_UNIFORM(wd);
        if (w != 0u) return wd * 32 + __builtin_ctz(w);
        return next_summary<SUMC>(kept, i, 0, no_correction);
    }
    return next_summary<SUMC>(kept, i, -code, no_correction);
}

// ---------------------------------------------------------------------------
// LDS operand reads of the tile compute, as byte offsets within a tile
// buffer, for lane (n = lane & 31, lh = lane >> 5).
// ---------------------------------------------------------------------------
// bf16 K operand of key block kb, dim step ks: 16 bytes.
// DORD 0: dims 16 ks + 8 lh .. +8; DORD 1: dims 64 (ks / 4) + 32 lh + 8 (ks % 4) .. +8
template <int DORD>
FP_HD int k_read_off(int kb, int ks, int n, int lh) {
    const int d0 = DORD ? 64 * (ks >> 2) + 32 * lh + 8 * (ks & 3) : 16 * ks + 8 * lh;
    return (kb * 32 + n) * KSTR + d0 * 2;
}
// bf16 V^T transpose read aa (0, 1) of key block kb, 16-key step s2, dim block db: 8 bytes
// (row kb * 32 + 16 s2 + 8 aa + rsub, whose rotation is 64 (rsub mod 4) bytes)
FP_HD int v_read_off(int kb, int s2, int aa, int db, int lane) {
    const int jj = lane & 15, q = lane >> 4;
    const int rsub = 4 * (q >> 1) + (jj >> 2);
    const int dsub = 16 * (q & 1) + 4 * (jj & 3);
    return (kb * 32 + 16 * s2 + 8 * aa + rsub) * VSTR + 64 * ((db + rsub) & 3) + 2 * dsub;
}
// fp8 K operand of key block kb, 64-dim step ks: 32 bytes (two 16-byte reads)
FP_HD int k8_read_off(int kb, int ks, int n, int lh) { return (kb * 32 + n) * KSTR8 + ks * 64 + lh * 32; }
// fp8 V^T transpose read c (0..3) of 64-key step s2, dim block db: 8 bytes
// (row s2 * 64 + 16 c + 8 lh + a / 2, whose rotation is 32 (a / 4) bytes)
FP_HD int v8_read_off(int s2, int c, int db, int lane) {
    const int a = lane & 15, half = (lane >> 4) & 1, lh = lane >> 5;
    return (s2 * 64 + 16 * c + 8 * lh + (a >> 1)) * VSTR8 + 32 * ((db + (a >> 2)) & 3) + 16 * half + 8 * (a & 1);
}

}  // namespace fp
