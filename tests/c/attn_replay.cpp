// Host replay of the sparse attention kernel's memory accesses.
//
// The kernel computes every global and LDS address with the functions of
// csrc/attn_geom.h and fp_internal.h; this program runs the same functions
// over every workgroup, wavefront, lane, piece and tile of whole launches
// (fixed-shape and paged, bf16 and fp8, both block sizes, ragged tails, tiny
// sequences, cached prefixes, random kept lists and schedules) and checks each
// access against the extent of its buffer and of its LDS allocation. It is
// built for the host with AddressSanitizer and UndefinedBehaviorSanitizer by
// a CPU test. Prints "ok" and exits 0 when every access is in bounds.
#include <algorithm>
#include <cstdio>
#include <cstdlib>
#include <random>
#include <vector>

#include "../../block_sparse_long_estimate_amd/csrc/attn_geom.h"

using namespace fp;

static long long g_checks = 0;
static int g_fail = 0;
static const char* g_case = "";

#define CHECK(cond, ...)                                                  \
    do {                                                                  \
        ++g_checks;                                                       \
        if (!(cond)) {                                                    \
            fprintf(stderr, "[%s] out of bounds: ", g_case);              \
            fprintf(stderr, __VA_ARGS__);                                 \
            fputc('\n', stderr);                                          \
            if (++g_fail > 20) exit(1);                                   \
        }                                                                 \
    } while (0)

// One launch's buffers, as element extents.
struct Launch {
    bool paged = false;
    int nseq = 0, Hq = 0, Hkv = 0, G = 0, blk = 128;
    int kv_div = 1;                  // per-head lists: list groups are query heads, KV head = g / kv_div
    int Hlist = 0;                   // list groups per sequence (Hkv, or Hq with per-head lists)
    std::vector<SeqDesc> table;      // nseq + 1 (the last entry: totals)
    RowAddr qa{}, oa{}, la{};
    KVAddr ka{}, va{};
    long long q_elems = 0, o_elems = 0, lse_elems = 0, k_elems = 0, v_elems = 0;
    long long pooled_rows = 0;       // kbar rows (x 128 elements) of the summary operands
    long long qs_elems = 0, kvs_elems = 0;
    ScaleAddr qs{}, ks{}, vs{};
    std::vector<int> block_table;
    int n_pages = 0;
    bool paged_fast = false;
    int rows = 0;
    std::vector<int> row_ptr, col_idx, sched;
};

static int seq_of_row(const Launch& L, int r) {
    int b = 0;
    while (b + 1 < L.nseq && L.table[b + 1].row0 <= r) ++b;
    return b;
}

// The kernel's last-column clamp of a summary sub-tile needs nbk >= 1; and
// each row's list holds its sink and diagonal.
static void make_lists(Launch& L, std::mt19937_64& rng, double density) {
    std::uniform_real_distribution<double> U(0, 1);
    L.row_ptr.assign(1, 0);
    L.col_idx.clear();
    for (int b = 0; b < L.nseq; ++b) {
        const SeqDesc& s = L.table[b];
        for (int g = 0; g < L.Hlist; ++g)
            for (int il = 0; il < s.nq; ++il) {
                const int i = s.i0 + il;
                for (int j = 0; j <= i; ++j)
                    if (j == 0 || j == i || U(rng) < density) L.col_idx.push_back(j);
                L.row_ptr.push_back((int)L.col_idx.size());
            }
    }
    L.rows = (int)L.row_ptr.size() - 1;
    L.sched.resize(L.rows);
    for (int r = 0; r < L.rows; ++r) L.sched[r] = r;
    std::shuffle(L.sched.begin(), L.sched.end(), rng);
}

// Sequence table of a fixed batch or a varlen batch, as the C ABI builds it.
static void make_table(Launch& L, const std::vector<int>& Ls, const std::vector<int>& Ps) {
    const int B = L.blk;
    L.table.assign(L.nseq + 1, SeqDesc{});
    long long qb = 0, kb = 0, qrows = 0;
    for (int b = 0; b < L.nseq; ++b) {
        SeqDesc& s = L.table[b];
        const int ql = Ls[b] - Ps[b];
        s.L = Ls[b];
        s.P = Ps[b];
        s.i0 = ql ? s.P / B : 0;
        s.nq = ql ? (s.L - 1) / B - s.i0 + 1 : 0;
        s.nbk = ql ? cdiv(s.L, B) : 0;
        s.q0 = L.paged ? (int)qrows : 0;
        s.qb0 = (int)qb;
        s.kb0 = (int)kb;
        s.row0 = (int)(qb * L.Hlist);
        qb += s.nq;
        kb += s.nbk;
        qrows += ql;
    }
    L.table[L.nseq].qb0 = (int)qb;
    L.table[L.nseq].kb0 = (int)kb;
    L.table[L.nseq].row0 = (int)(qb * L.Hlist);
    L.pooled_rows = kb * L.Hkv;
}

template <int BLK, bool FP8, bool PAGED, int NW>
static void replay(const Launch& L, bool split_small) {
    using TG = TileGeom<BLK, FP8>;
    constexpr int RG = 8 / NW, ESZ = TG::ESZ;
    const int slices = cdiv(L.G * BLK, 256);
    const int units = cdiv(L.rows, 8) * 8 * slices;
    const long long kbytes = L.k_elems * ESZ, vbytes = L.v_elems * ESZ;
    // the kernel reads the block table through KVAddr (ASan watches these reads)
    KVAddr ka = L.ka, va = L.va;
    ka.table = va.table = L.block_table.empty() ? nullptr : L.block_table.data();
    const long long nnz = (long long)L.col_idx.size();
    constexpr int PAGE_CAP = 2048;
    std::vector<uint32_t> kept(MAX_NB / 32);

    // LDS operand reads of the tile compute (independent of the data)
    for (int lane = 0; lane < 64; ++lane) {
        const int n = lane & 31, lh = lane >> 5;
        for (int kb = 0; kb < TG::NKB; ++kb) {
            if (FP8) {
                for (int ks = 0; ks < 2; ++ks)
                    CHECK(k8_read_off(kb, ks, n, lh) + 32 <= TG::KTILE, "fp8 K read");
                for (int s2 = 0; s2 < TG::NKB / 2; ++s2)
                    for (int c = 0; c < 4; ++c)
                        for (int db = 0; db < 4; ++db)
                            CHECK(v8_read_off(s2, c, db, lane) + 8 <= TG::VTILE_KEPT, "fp8 V read");
            } else {
                for (int ks = 0; ks < 8; ++ks) CHECK(k_read_off<0>(kb, ks, n, lh) + 16 <= TG::KTILE, "K read");
                for (int s2 = 0; s2 < 2; ++s2)
                    for (int aa = 0; aa < 2; ++aa)
                        for (int db = 0; db < 4; ++db)
                            CHECK(v_read_off(kb, s2, aa, db, lane) + 8 <= TG::VTILE_KEPT, "V read");
            }
        }
        // summary sub-tiles: hi rows (key blocks 0 .. SB-1), lo rows (SB .. 2 SB - 1), V rows
        for (int kb = 0; kb < 2 * TG::SB; ++kb)
            for (int ks = 0; ks < 8; ++ks) {
                CHECK(k_read_off<0>(kb, ks, n, lh) + 16 <= TG::KTILE, "summary K read");
                CHECK(k_read_off<1>(kb, ks, n, lh) + 16 <= TG::KTILE, "summary K read (fp8 order)");
            }
        for (int kb = 0; kb < TG::SB; ++kb)
            for (int s2 = 0; s2 < 2; ++s2)
                for (int aa = 0; aa < 2; ++aa)
                    for (int db = 0; db < 4; ++db)
                        CHECK(v_read_off(kb, s2, aa, db, lane) + 8 <= TG::VTILE_SUM, "summary V read");
    }

    // a grid too small for the chip splits the rows of a fixed-shape launch
    const int nsplit = PAGED || !split_small ? 1 : split_count(L.rows, slices);
    const long long parts = split_parts(L.rows, slices, nsplit);
    {
        // the unit map covers each (row, slice, part) once
        std::vector<int> seen((size_t)cdiv(L.rows, 8) * 8 * slices * nsplit, 0);
        for (int u = 0; u < units * nsplit; ++u) {
            const UnitMap um = unit_map(u, slices, nsplit);
            CHECK(um.slice >= 0 && um.slice < slices && um.split >= 0 && um.split < nsplit && um.pidx >= 0,
                  "unit %d", u);
            const long long key = ((long long)um.pidx * slices + um.slice) * nsplit + um.split;
            if (key >= 0 && key < (long long)seen.size()) ++seen[key];
        }
        for (size_t k = 0; k < seen.size(); ++k) CHECK(seen[k] == 1, "unit key %zu seen %d times", k, seen[k]);
    }
    for (int u = 0; u < units * nsplit; ++u) {
        const UnitMap um = unit_map(u, slices, nsplit);
        if (um.split != 0) continue;                 // all parts of a (row, slice) are replayed together
        if (um.pidx >= L.rows) continue;
        CHECK(um.pidx >= 0 && um.pidx < (int)L.sched.size(), "sched[%d]", um.pidx);
        const int r = L.sched[um.pidx];
        CHECK(r >= 0 && r < L.rows, "row %d", r);
        const int b = seq_of_row(L, r);
        const SeqDesc s = L.table[b];
        const int rl = r - s.row0;
        const int g = rl / s.nq, il = rl % s.nq;
        const int gk = g / L.kv_div;
        const int i = s.i0 + il;
        const int t_lo = std::max(i * BLK, s.P), t_hi = std::min((i + 1) * BLK, s.L);
        const int npk = L.G * (t_hi - t_lo);
        if (um.slice * 256 >= npk) continue;
        CHECK(r + 1 < (int)L.row_ptr.size(), "row_ptr[%d]", r + 1);
        const int rp0 = L.row_ptr[r], nr = L.row_ptr[r + 1] - rp0;
        CHECK(rp0 >= 0 && rp0 + nr <= nnz && nr >= 1, "col_idx[%d..%d)", rp0, rp0 + nr);

        // query rows: q loads, o stores (bf16 or fp32), lse stores, fp8 q
        // scales; the slice's 256 packed rows are each owned by one lane
        int owned[256] = {};
        for (int wave = 0; wave < NW; ++wave)
            for (int rg = 0; rg < RG; ++rg)
                for (int n = 0; n < 32; ++n) {
                    const int prow = packed_row<NW>(um.slice, wave, rg, n);
                    CHECK(prow >= um.slice * 256 && prow < um.slice * 256 + 256, "packed row %d", prow);
                    if (prow >= um.slice * 256 && prow < um.slice * 256 + 256) ++owned[prow - um.slice * 256];
                    if (prow >= npk) continue;
                    const int tl = prow / L.G;
                    const int t = t_lo + tl, h = g * L.G + prow - tl * L.G;
                    CHECK(t >= s.P && t < s.L && h >= 0 && h < L.Hq, "row t=%d h=%d", t, h);
                    const long long qo = L.qa.off(b, s, t, h), oo = L.oa.off(b, s, t, h);
                    CHECK(qo >= 0 && qo + D <= L.q_elems, "q row %lld", qo);
                    CHECK(oo >= 0 && oo + D <= L.o_elems, "o row %lld", oo);
                    const long long lo = L.la.off(b, s, t, h);
                    CHECK(lo >= 0 && lo < L.lse_elems, "lse %lld", lo);
                    if (FP8) {
                        const long long qsi = (long long)b * L.qs.sb + (long long)h * L.qs.sh + (t >> 7);
                        CHECK(qsi >= 0 && qsi < L.qs_elems, "q scale %lld", qsi);
                    }
                }

        for (int e = 0; e < 256; ++e) CHECK(owned[e] == 1, "packed row %d of the slice owned %d times", e, owned[e]);

        // kept bitmap of the row
        std::fill(kept.begin(), kept.end(), 0u);
        for (int e = 0; e < nr; ++e) {
            const int j = L.col_idx[rp0 + e];
            CHECK(j >= 0 && j <= i && (j >> 5) < MAX_NB / 32, "kept column %d of row %d", j, i);
            kept[j >> 5] |= 1u << (j & 31);
        }
        const int j0 = L.col_idx[rp0];

        // staged page ids
        std::vector<int> pages;
        bool have_pages = false;
        if (PAGED) {
            const int npg = (s.L + (1 << ka.page_shift) - 1) >> ka.page_shift;
            if (npg <= PAGE_CAP) {
                have_pages = true;
                for (int p = 0; p < npg; ++p) {
                    const long long bi = (long long)b * ka.maxp + p;
                    CHECK(bi >= 0 && bi < (long long)L.block_table.size(), "block_table[%lld]", bi);
                    pages.push_back(L.block_table[bi]);
                }
            }
        }
        auto page_of = [&](int slot) {
            CHECK(slot >= 0 && slot < (int)pages.size(), "staged page slot %d of %zu", slot, pages.size());
            return pages[slot];
        };
        auto check_kv = [&](long long off, long long bytes, const char* what) {
            CHECK(off >= 0 && off + 16 <= bytes, "%s bytes [%lld, %lld) of %lld", what, off, off + 16, bytes);
        };

        // tile sequence of the row; the first tile is issued before the page
        // ids are staged, so it reads the block table directly
        const bool no_corr = false;
        std::vector<char> visited(i + 1, 0), sub_visited(i / TG::SUMC + 1, 0);
        auto visit = [&](int code, bool staged) {
            if (code >= 0 && code <= i) ++visited[code];
            if (code < 0 && -1 - code <= i / TG::SUMC) ++sub_visited[-1 - code];
            if (code >= 0) {
                CHECK(code <= i, "kept code %d > %d", code, i);
                if (FP8) {
                    const long long ksi = (long long)b * L.ks.sb + (long long)gk * L.ks.sh + ((code * BLK) >> 7);
                    CHECK(ksi >= 0 && ksi < L.kvs_elems, "k scale %lld", ksi);
                }
                const bool full = (code + 1) * BLK <= s.L;
                for (int wave = 0; wave < NW; ++wave)
                    for (int lane = 0; lane < 64; ++lane) {
                        TileOffs<TG::KS, BLK, ESZ, false, NW> ko;
                        TileOffs<TG::VS, BLK, ESZ, FP8, NW> vo;
                        if (!PAGED && full) {
                            ko.init(ka.st, wave, lane);
                            vo.init(va.st, wave, lane);
                            const long long k0 = ka.template off<false>(b, code * BLK, gk) * ESZ;
                            const long long v0 = va.template off<false>(b, code * BLK, gk) * ESZ;
                            for (int k = 0; k < ko.NP; ++k)
                                if (ko.has(k, wave)) {
                                    check_kv(ko.src_full(k0, k), kbytes, "K tile");
                                    CHECK((k * NW + wave) * PIECE + 16 * lane + 16 <= TG::KTILE, "K LDS piece");
                                }
                            for (int k = 0; k < vo.NP; ++k)
                                if (vo.has(k, wave)) {
                                    check_kv(vo.src_full(v0, k), vbytes, "V tile");
                                    CHECK((k * NW + wave) * PIECE + 16 * lane + 16 <= TG::VTILE, "V LDS piece");
                                }
                        } else if (PAGED && staged && L.paged_fast && full) {
                            const int lshift = std::min(ka.page_shift, BLK == 128 ? 7 : 6);
                            ko.init_paged(ka.st, lshift, wave, lane);
                            vo.init_paged(va.st, lshift, wave, lane);
                            const int sh = ka.page_shift;
                            const long long ub =
                                (long long)((code * BLK) & ((1 << sh) - 1)) * ka.st + (long long)gk * ka.sh;
                            const int slot0 = (code * BLK) >> sh;
                            for (int k = 0; k < ko.NP; ++k)
                                if (ko.has(k, wave)) {
                                    const int pg = page_of(slot0 + ko.page_slot(k));
                                    check_kv(ub * ESZ + (long long)pg * ka.spage * ESZ + ko.in_page(k), kbytes,
                                             "K paged tile");
                                    CHECK((k * NW + wave) * PIECE + 16 * lane + 16 <= TG::KTILE, "K LDS piece");
                                }
                            for (int k = 0; k < vo.NP; ++k)
                                if (vo.has(k, wave)) {
                                    const int pg = page_of(slot0 + vo.page_slot(k));
                                    check_kv(ub * ESZ + (long long)pg * va.spage * ESZ + vo.in_page(k), vbytes,
                                             "V paged tile");
                                    CHECK((k * NW + wave) * PIECE + 16 * lane + 16 <= TG::VTILE, "V LDS piece");
                                }
                        } else {
                            auto pf = [&](int slot) { return page_of(slot); };
                            for (int k = 0; k < ko.NP; ++k) {
                                if (!ko.has(k, wave)) continue;
                                const long long src = tile_src<TG::KS, BLK, ESZ, false, PAGED>(
                                    ka, b, s.L, gk, code, k * NW + wave, lane, pf, staged);
                                {
                                    check_kv(src, kbytes, "K generic tile");
                                    CHECK((k * NW + wave) * PIECE + 16 * lane + 16 <= TG::KTILE, "K LDS piece");
                                }
                            }
                            for (int k = 0; k < vo.NP; ++k) {
                                if (!vo.has(k, wave)) continue;
                                const long long src = tile_src<TG::VS, BLK, ESZ, FP8, PAGED>(
                                    va, b, s.L, gk, code, k * NW + wave, lane, pf, staged);
                                {
                                    check_kv(src, vbytes, "V generic tile");
                                    CHECK((k * NW + wave) * PIECE + 16 * lane + 16 <= TG::VTILE, "V LDS piece");
                                }
                            }
                        }
                    }
            } else {
                const int m = -1 - code;
                CHECK(m * TG::SUMC <= i - 1, "summary sub-tile %d of row %d", m, i);
                for (int w = 0; w < 2; ++w) {
                    const int P = w == 0 ? TG::SKPIECES : TG::SVPIECES;
                    for (int wave = 0; wave < NW; ++wave)
                        for (int t0 = 0; t0 < P; t0 += NW) {
                            const int t = t0 + wave;
                            if (t >= P) continue;
                            for (int lane = 0; lane < 64; ++lane) {
                                const SummarySrc src = summary_src<BLK>(s, L.Hkv, gk, m, w, t, lane);
                                CHECK(src.which >= 0 && src.which <= 2, "summary array %d", src.which);
                                CHECK(src.off >= 0 && src.off + 8 <= L.pooled_rows * D, "summary source %lld",
                                      src.off);
                                CHECK(t * PIECE + 16 * lane + 16 <= (w == 0 ? TG::KTILE : TG::VTILE),
                                      "summary LDS piece");
                                if (SumOffs<BLK, NW>::whole(m, s.nbk)) {
                                    // whole sub-tile: the per-lane offsets of the load
                                    // path read the same bytes (lo array lo_delta bytes
                                    // after the hi array, as the library lays them out)
                                    using SO = SumOffs<BLK, NW>;
                                    const long long lo_delta = (L.pooled_rows * D * 2 + 255) / 256 * 256;
                                    SO so;
                                    so.init((uint32_t)lo_delta, wave, lane);
                                    const long long r0 = kbar_row(s, L.Hkv, gk, TG::SUMC * m) * D * 2;
                                    const int k = t0 / NW;
                                    const long long fast = w == 0 ? (SO::has_k(k, wave) ? r0 + so.k_off[k] : -1)
                                                                  : (SO::has_v(k, wave) ? r0 + so.v_off + (long long)t * PIECE
                                                                                        : -1);
                                    const long long slow = (src.which == 1 ? lo_delta : 0) + src.off * 2;
                                    CHECK(fast == slow, "summary offsets: sub-tile %d piece %d lane %d: %lld vs %lld", m,
                                          t, lane, fast, slow);
                                }
                            }
                        }
                }
            }
        };
        if (nsplit < 2) {
            for (int code = j0; code != TILE_NONE; code = next_code<TG::SUMC>(kept, i, code, no_corr))
                visit(code, have_pages && code != j0);
        } else {
            // the parts of a split row: tiles [first, first + count) each, first
            // issued after the bitmap; partial results and their merge in bounds
            const int T = nr + count_summary<TG::SUMC>(kept, i, no_corr);
            int covered = 0;
            for (int sp = 0; sp < nsplit; ++sp) {
                const SplitRange sr = split_range(T, sp, nsplit);
                CHECK(sr.first == covered && sr.count >= 0, "part %d of row %d: tiles [%d, +%d)", sp, i, sr.first,
                      sr.count);
                covered = sr.first + sr.count;
                const long long pu = split_part(um.pidx, slices, um.slice, nsplit, sp);
                CHECK(pu >= 0 && pu < parts, "part index %lld of %lld", pu, parts);
                for (int pl = 0; pl < 256 && um.slice * 256 + pl < npk; ++pl) {
                    CHECK((pu * SLICE_ROWS + pl) * D + D <= split_o_floats(parts), "partial O row %d", pl);
                    CHECK((pu * SLICE_ROWS + pl) * 2 + 2 <= split_floats(parts) - split_o_floats(parts),
                          "partial (m, l) row %d", pl);
                }
                if (sr.count == 0) continue;
                int code = sr.first < nr ? L.col_idx[rp0 + sr.first]
                                         : nth_summary<TG::SUMC>(kept, i, sr.first - nr, no_corr);
                CHECK(code != TILE_NONE, "part %d of row %d starts past the sequence", sp, i);
                for (int remaining = sr.count; code != TILE_NONE;) {
                    visit(code, have_pages);
                    if (--remaining <= 0) break;
                    code = next_code<TG::SUMC>(kept, i, code, no_corr);
                    CHECK(code != TILE_NONE, "part %d of row %d ends early", sp, i);
                }
            }
            CHECK(covered == T, "parts of row %d cover %d of %d tiles", i, covered, T);
        }
        // every kept block visited once as a kept tile; every pruned column
        // (between the sink and the diagonal) inside a summary sub-tile that is
        // visited once; no sub-tile without a pruned column
        for (int j = 0; j <= i; ++j) {
            const bool k = (kept[j >> 5] >> (j & 31)) & 1u;
            CHECK(visited[j] == (k ? 1 : 0), "column %d of row %d visited %d times as a kept tile", j, i, visited[j]);
            if (!k && j >= 1 && j <= i - 1)
                CHECK(sub_visited[j / TG::SUMC] == 1, "pruned column %d of row %d: sub-tile visited %d times", j, i,
                      sub_visited[j / TG::SUMC]);
        }
        for (int m = 0; m <= i / TG::SUMC; ++m) {
            bool any = false;
            for (int j = std::max(1, m * TG::SUMC); j <= std::min(i - 1, m * TG::SUMC + TG::SUMC - 1); ++j)
                any |= !((kept[j >> 5] >> (j & 31)) & 1u);
            CHECK(sub_visited[m] == (any ? 1 : 0), "summary sub-tile %d of row %d visited %d times", m, i,
                  sub_visited[m]);
        }
    }
}

// ---------------------------------------------------------------------------
// problem builders
// ---------------------------------------------------------------------------
static Launch fixed_launch(int batch, int S, int Hq, int Hkv, int blk, bool fp8, double density, uint64_t seed,
                           bool fused_qkv, bool per_head = false) {
    Launch L;
    L.nseq = batch;
    L.Hq = Hq;
    L.Hkv = Hkv;
    L.G = per_head ? 1 : Hq / Hkv;
    L.kv_div = per_head ? Hq / Hkv : 1;
    L.Hlist = per_head ? Hq : Hkv;
    L.blk = blk;
    make_table(L, std::vector<int>(batch, S), std::vector<int>(batch, 0));
    // fixed shape: every sequence has nb query and key blocks; the descriptor
    // offsets are the same arithmetic GeoFixed uses (over the list groups)
    GeoFixed gf{batch, S, Hq, L.Hlist, blk, cdiv(S, blk), 0};
    for (int b = 0; b < batch; ++b) L.table[b] = gf.seq(b);
    long long qst = (long long)Hq * D, kst = (long long)Hkv * D;
    if (fused_qkv) qst = kst = (long long)(Hq + 2 * Hkv) * D;    // one [S, Hq + 2 Hkv, D] buffer
    L.qa = RowAddr{S * qst, qst, D};
    L.ka = KVAddr{S * kst, kst, D, 0, nullptr, 0, 0};
    L.va = L.ka;
    L.oa = RowAddr{(long long)S * Hq * D, (long long)Hq * D, D};
    L.la = RowAddr{(long long)Hq * S, 1, S};
    L.q_elems = batch * S * qst;
    L.k_elems = L.v_elems = batch * S * kst;
    L.o_elems = (long long)batch * S * Hq * D;
    L.lse_elems = (long long)batch * Hq * S;
    const int nsb = cdiv(S, SCALE_TOK);
    L.qs = ScaleAddr{nullptr, (long long)Hq * nsb, nsb};
    L.ks = ScaleAddr{nullptr, (long long)Hkv * nsb, nsb};
    L.vs = L.ks;
    L.qs_elems = (long long)batch * Hq * nsb;
    L.kvs_elems = (long long)batch * Hkv * nsb;
    L.pooled_rows = (long long)batch * Hkv * cdiv(S, blk);
    std::mt19937_64 rng(seed);
    make_lists(L, rng, density);
    (void)fp8;
    return L;
}

static Launch paged_launch(const std::vector<int>& Ls, const std::vector<int>& Ps, int Hq, int Hkv, int blk,
                           int page, double density, uint64_t seed) {
    Launch L;
    L.paged = true;
    L.nseq = (int)Ls.size();
    L.Hq = Hq;
    L.Hkv = Hkv;
    L.G = Hq / Hkv;
    L.Hlist = Hkv;
    L.blk = blk;
    make_table(L, Ls, Ps);
    int shift = 0;
    while ((1 << shift) < page) ++shift;
    int maxp = 0, total = 0;
    long long sum_q = 0;
    for (int b = 0; b < L.nseq; ++b) {
        maxp = std::max(maxp, cdiv(Ls[b], page));
        total += cdiv(Ls[b], page);
        sum_q += Ls[b] - Ps[b];
    }
    std::mt19937_64 rng(seed);
    std::vector<int> perm(total);
    for (int p = 0; p < total; ++p) perm[p] = p;
    std::shuffle(perm.begin(), perm.end(), rng);
    L.block_table.assign((size_t)L.nseq * maxp, 0);
    int off = 0;
    for (int b = 0; b < L.nseq; ++b)
        for (int p = 0; p < cdiv(Ls[b], page); ++p) L.block_table[(size_t)b * maxp + p] = perm[off++];
    L.n_pages = total;
    const long long st = (long long)Hkv * D, spage = page * st;
    L.ka = KVAddr{0, st, D, spage, nullptr, maxp, shift};
    L.va = L.ka;
    L.qa = RowAddr{0, (long long)Hq * D, D};
    L.oa = L.qa;
    L.la = RowAddr{0, 1, sum_q};
    L.q_elems = L.o_elems = sum_q * Hq * D;
    L.lse_elems = sum_q * Hq;
    L.k_elems = L.v_elems = (long long)total * spage;
    const int nsb = cdiv(maxp * page, SCALE_TOK);
    L.qs = ScaleAddr{nullptr, (long long)Hq * nsb, nsb};
    L.ks = ScaleAddr{nullptr, (long long)Hkv * nsb, nsb};
    L.vs = L.ks;
    L.qs_elems = (long long)L.nseq * Hq * nsb;
    L.kvs_elems = (long long)L.nseq * Hkv * nsb;
    L.paged_fast = (long long)std::min(page, blk) * st * 2 < (1LL << 24);
    make_lists(L, rng, density);
    return L;
}

// ---------------------------------------------------------------------------
// Operand layout: fill a tagged image of each LDS tile through the load
// functions (piece_loc, with the fp8 V key permutation; summary_src for the
// summary tiles), then emulate every operand read of the tile compute --
// plain 16/32-byte reads for K, the transpose reads for V^T with the lane
// semantics of ds_read_b64_tr_b16 (16-lane group: lane i's element e is
// element i mod 4 of the 8 bytes lane 4e + i / 4 addresses) and
// ds_read_b64_tr_b8 (lane i's byte e is byte i mod 8 of the 8 bytes lane
// 2e + i / 8 addresses) -- and check that each lane receives the (key, dim)
// the MFMA step expects: K[key kb*32 + n][dims of its k slot] for QK^T; for
// PV, the A operand's k index must hold the key that the P operand (taken in
// the order of the S^T accumulator, key 8 (v/4) + 4 lh + v mod 4 for
// accumulator element v of lane half lh) holds there.
// ---------------------------------------------------------------------------
struct Tag {
    int key = -1, dim = -1;          // dim: element index within the 128 dims
    bool operator==(const Tag& o) const { return key == o.key && dim == o.dim; }
};

static void tag_tile(std::vector<Tag>& img, int STR, int rows, int esz, bool perm, int key_of_row_lo = 0,
                     bool summary_k = false, int sumc = 0) {
    const int pieces = rows * STR / PIECE;
    img.assign((size_t)pieces * PIECE, Tag{});
    for (int t = 0; t < pieces; ++t)
        for (int lane = 0; lane < 64; ++lane) {
            const PieceLoc pl = piece_loc(STR, t, lane, 8 * esz);
            int key = perm ? vt_slot(pl.row) : pl.row;
            if (summary_k) key = pl.row >= sumc ? 1000000 + (pl.row - sumc) : pl.row;   // lo rows: tagged apart
            for (int b = 0; b < 16; ++b)
                img[(size_t)t * PIECE + lane * 16 + b] = Tag{key + key_of_row_lo, (pl.ch * 16 + b) / esz};
        }
}



#define LAYOUT(cond, ...)                                                 \
    do {                                                                  \
        ++g_checks;                                                       \
        if (!(cond)) {                                                    \
            fprintf(stderr, "[operand layout] ");                        \
            fprintf(stderr, __VA_ARGS__);                                 \
            fputc('\n', stderr);                                          \
            if (++g_fail > 20) exit(1);                                   \
        }                                                                 \
    } while (0)

// A kept K or V tile as the contiguous-tile loads fill it: the per-lane
// source offsets of TileOffs (rows of 128 elements) decoded back to (key, dim).
template <int STR, int BLK, int ESZ, bool PERM, int NW>
static void tag_loaded_tile(std::vector<Tag>& img) {
    using TO = TileOffs<STR, BLK, ESZ, PERM, NW>;
    img.assign((size_t)TO::PIECES * PIECE, Tag{});
    for (int wave = 0; wave < NW; ++wave)
        for (int lane = 0; lane < 64; ++lane) {
            TO o;
            o.init(128, wave, lane);
            for (int k = 0; k < TO::NP; ++k) {
                if (!TO::has(k, wave)) continue;
                if (k * NW + wave >= TO::PIECES) {
                    LAYOUT(false, "piece %d of wave %d lies past the %d-piece tile", k * NW + wave, wave, TO::PIECES);
                    continue;
                }
                const long long src = o.src_full(0, k);
                const int key = (int)(src / (128 * ESZ)), d0 = (int)(src % (128 * ESZ)) / ESZ;
                for (int b = 0; b < 16; ++b)
                    img[(size_t)(k * NW + wave) * PIECE + lane * 16 + b] = Tag{key, d0 + b / ESZ};
            }
        }
}

template <int BLK, bool FP8>
static void check_operand_layout() {
    using TG = TileGeom<BLK, FP8>;
    constexpr int ESZ = TG::ESZ;
    std::vector<Tag> K, V, SK, SV;
    tag_loaded_tile<TG::KS, BLK, ESZ, false, 8>(K);
    tag_loaded_tile<TG::VS, BLK, ESZ, FP8, 8>(V);
    tag_tile(SK, KSTR, BLK, 2, false, 0, true, TG::SUMC);
    tag_tile(SV, VSTR, TG::SUMC, 2, false);
    auto at = [](const std::vector<Tag>& img, int byte, int esz) -> Tag {
        if (byte < 0 || byte + esz > (int)img.size()) return Tag{-2, -2};
        return img[byte];
    };
    for (int lane = 0; lane < 64; ++lane) {
        const int n = lane & 31, lh = lane >> 5;
        for (int kb = 0; kb < TG::NKB; ++kb) {
            if (FP8) {
                for (int ks = 0; ks < 2; ++ks)
                    for (int e = 0; e < 32; ++e)
                        LAYOUT(at(K, k8_read_off(kb, ks, n, lh) + e, 1) == (Tag{kb * 32 + n, 64 * ks + 32 * lh + e}),
                               "fp8 K blk=%d kb=%d ks=%d lane=%d byte %d", BLK, kb, ks, lane, e);
            } else {
                for (int ks = 0; ks < 8; ++ks)
                    for (int e = 0; e < 8; ++e)
                        LAYOUT(at(K, k_read_off<0>(kb, ks, n, lh) + 2 * e, 2) == (Tag{kb * 32 + n, 16 * ks + 8 * lh + e}),
                               "bf16 K blk=%d kb=%d ks=%d lane=%d elem %d", BLK, kb, ks, lane, e);
            }
        }
        // summary K: row kb*32+n holds hi of column kb*32+n for kb < SB, lo of column (kb-SB)*32+n after
        for (int kb = 0; kb < 2 * TG::SB; ++kb)
            for (int dord = 0; dord < 2; ++dord)
                for (int ks = 0; ks < 8; ++ks) {
                    const int col = (kb % TG::SB) * 32 + n + (kb >= TG::SB ? 1000000 : 0);
                    const int d0 = dord ? 64 * (ks >> 2) + 32 * lh + 8 * (ks & 3) : 16 * ks + 8 * lh;
                    const int off = dord ? k_read_off<1>(kb, ks, n, lh) : k_read_off<0>(kb, ks, n, lh);
                    for (int e = 0; e < 8; ++e)
                        LAYOUT(at(SK, off + 2 * e, 2) == (Tag{col, d0 + e}), "summary K blk=%d kb=%d ks=%d lane=%d",
                               BLK, kb, ks, lane);
                }
    }
    // V^T transpose reads, whole wavefront at a time
    for (int db = 0; db < 4; ++db) {
        if (FP8) {
            for (int s2 = 0; s2 < TG::NKB / 2; ++s2)
                for (int c = 0; c < 4; ++c)
                    for (int lane = 0; lane < 64; ++lane) {
                        const int g = lane / 16, i = lane % 16;
                        for (int e = 0; e < 8; ++e) {
                            const int src = 16 * g + 2 * e + i / 8;
                            const Tag got = at(V, v8_read_off(s2, c, db, src) + i % 8, 1);
                            const int key = s2 * 64 + 16 * c + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
                            LAYOUT(got == (Tag{key, 32 * db + (lane & 31)}), "fp8 V blk=%d s2=%d c=%d db=%d lane=%d",
                                   BLK, s2, c, db, lane);
                        }
                    }
        }
        const int nkb_v = FP8 ? 0 : TG::NKB;
        for (int part = 0; part < 2; ++part) {          // 0: kept V tile (bf16), 1: summary V tile
            const std::vector<Tag>& img = part ? SV : V;
            for (int kb = 0; kb < (part ? TG::SB : nkb_v); ++kb)
                for (int s2 = 0; s2 < 2; ++s2)
                    for (int aa = 0; aa < 2; ++aa)
                        for (int lane = 0; lane < 64; ++lane) {
                            const int g = lane / 16, i = lane % 16;
                            for (int e4 = 0; e4 < 4; ++e4) {
                                const int src = 16 * g + 4 * e4 + i / 4;
                                const Tag got = at(img, v_read_off(kb, s2, aa, db, src) + 2 * (i % 4), 2);
                                const int e = 4 * aa + e4;
                                const int key = kb * 32 + 16 * s2 + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
                                LAYOUT(got == (Tag{key, 32 * db + (lane & 31)}),
                                       "%s V blk=%d kb=%d s2=%d aa=%d db=%d lane=%d", part ? "summary" : "bf16", BLK,
                                       kb, s2, aa, db, lane);
                            }
                        }
        }
    }
}

template <int NW>
static void replay_all(const Launch& L, bool fp8) {
    if (L.paged) {
        if (L.blk == 128) fp8 ? replay<128, true, true, NW>(L, false) : replay<128, false, true, NW>(L, false);
        else fp8 ? replay<64, true, true, NW>(L, false) : replay<64, false, true, NW>(L, false);
        return;
    }
    // fixed shape: as launched by default, and with the split of small grids when it applies
    const int slices = attn_slices(L.G, L.blk);
    for (int sp = 0; sp < (split_count(L.rows, slices) > 1 ? 2 : 1); ++sp) {
        if (L.blk == 128) fp8 ? replay<128, true, false, NW>(L, sp) : replay<128, false, false, NW>(L, sp);
        else fp8 ? replay<64, true, false, NW>(L, sp) : replay<64, false, false, NW>(L, sp);
    }
}

int main(int argc, char** argv) {
    // "quick": only the first case of each kind (used to check that planted
    // mistakes in the address functions are caught)
    const bool quick = argc > 1 && argv[1][0] == 'q';
    char name[256];
    uint64_t seed = 1;
    check_operand_layout<128, false>();
    check_operand_layout<128, true>();
    check_operand_layout<64, false>();
    check_operand_layout<64, true>();
    // a launch small enough to split its rows into parts (first, so the quick mode runs it too)
    for (int fp8 = 0; fp8 < 2; ++fp8) {
        snprintf(name, sizeof name, "fixed split rows S=700 4/1 blk=128 %s", fp8 ? "fp8" : "bf16");
        g_case = name;
        const Launch L = fixed_launch(1, 700, 4, 1, 128, fp8, 0.3, seed++, false);
        if (split_count(L.rows, attn_slices(L.G, 128)) < 2) {
            fprintf(stderr, "[%s] expected a split launch\n", name);
            return 1;
        }
        replay_all<8>(L, fp8);
    }
    // launches whose rows see whole summary sub-tiles (all their pooled
    // columns inside the sequence: the per-lane offset load path), first too
    for (int blk : {64, 128})
        for (int fp8 = 0; fp8 < 2; ++fp8) {
            const int S = blk == 64 ? 2600 : 8400;
            snprintf(name, sizeof name, "fixed whole summary sub-tiles S=%d 4/1 blk=%d %s", S, blk, fp8 ? "fp8" : "bf16");
            g_case = name;
            const Launch L = fixed_launch(1, S, 4, 1, blk, fp8, 0.0, seed++, false);
            replay_all<8>(L, fp8);
            replay_all<4>(L, fp8);
        }
    // fixed shapes: tiny and ragged lengths, GQA ratios, densities from
    // "sink and diagonal only" to "everything kept", fused q/k/v strides;
    // among them the launch that once faulted: S = 4173, 8/2 heads, block 128
    struct F { int batch, S, Hq, Hkv, blk; };
    const F fixed[] = {{1, 4173, 8, 2, 128}, {1, 1, 4, 1, 64}, {1, 5, 8, 8, 128}, {2, 127, 6, 2, 128},
                       {1, 129, 16, 1, 64}, {1, 1000, 3, 1, 128}, {1, 3000, 8, 2, 64}, {2, 2053, 8, 2, 128},
                       {1, 2048, 4, 1, 64}, {1, 700, 48, 16, 128}};
    for (const F& f : fixed)
        for (double dens : {0.0, 0.3, 1.0})
            for (int fp8 = 0; fp8 < 2; ++fp8)
                for (int fused = 0; fused < 2; ++fused) {
                    snprintf(name, sizeof name, "fixed B=%d S=%d %d/%d blk=%d dens=%.1f %s%s", f.batch, f.S, f.Hq,
                             f.Hkv, f.blk, dens, fp8 ? "fp8" : "bf16", fused ? " fused-qkv" : "");
                    g_case = name;
                    const Launch L = fixed_launch(f.batch, f.S, f.Hq, f.Hkv, f.blk, fp8, dens, seed++, fused);
                    replay_all<8>(L, fp8);
                    replay_all<4>(L, fp8);
                    if (quick) goto paged_cases;
                    if (fused == 0 && f.Hq != f.Hkv) {      // one kept list per query head
                        snprintf(name, sizeof name, "fixed per-head lists B=%d S=%d %d/%d blk=%d dens=%.1f %s",
                                 f.batch, f.S, f.Hq, f.Hkv, f.blk, dens, fp8 ? "fp8" : "bf16");
                        const Launch P = fixed_launch(f.batch, f.S, f.Hq, f.Hkv, f.blk, fp8, dens, seed++, false,
                                                      true);
                        replay_all<8>(P, fp8);
                    }
                }
paged_cases:
    // paged varlen: cached prefixes (mid-block, on a block boundary, one new
    // row, fully cached), one-token sequences, pages smaller than, equal to
    // and larger than a block, and a sequence with more pages than are staged
    struct P { std::vector<int> L, Pf; int Hq, Hkv, blk, page; };
    const P paged[] = {{{700, 1, 1324, 900, 2049}, {700, 0, 1024, 899, 0}, 8, 2, 128, 64},
                       {{300, 3500, 1200}, {0, 1700, 37}, 8, 2, 128, 16},
                       {{300, 3500, 1200}, {0, 1700, 37}, 8, 2, 64, 256},
                       {{2500, 900}, {1000, 0}, 6, 2, 64, 32},
                       {{40000}, {39000}, 4, 1, 128, 16},
                       {{5000, 7000}, {2500, 0}, 16, 1, 64, 128}};
    for (const P& p : paged)
        for (double dens : {0.0, 0.3, 1.0})
            for (int fp8 = 0; fp8 < 2; ++fp8) {
                snprintf(name, sizeof name, "paged n=%zu %d/%d blk=%d page=%d dens=%.1f %s", p.L.size(), p.Hq, p.Hkv,
                         p.blk, p.page, dens, fp8 ? "fp8" : "bf16");
                g_case = name;
                const Launch L = paged_launch(p.L, p.Pf, p.Hq, p.Hkv, p.blk, p.page, dens, seed++);
                replay_all<8>(L, fp8);
                replay_all<4>(L, fp8);
                if (quick) goto done;
            }
done:
    if (g_fail) {
        fprintf(stderr, "%d out-of-bounds accesses (%lld checks)\n", g_fail, g_checks);
        return 1;
    }
    printf("ok %lld checks\n", g_checks);
    return 0;
}
