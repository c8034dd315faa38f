// Sparse attention over the kept blocks plus the mean-correction pseudo-tokens
// (E6), bf16 and fp8-e4m3 inputs, contiguous or paged K/V.
//
// The pages describe a sparse flash-attention operator over the kept blocks
// (lode.cx page, implementation paragraph; aimodeling.com page, "Operator
// alignment" bullet) and a mean correction for the pruned blocks (lode.cx
// page, "How It Works"; aimodeling.com page, "Error correction" bullet). The
// H20 design they name (PackGQA, warp specialisation, pingpong) is prior art;
// this is a gfx950 design:
//
//  * Work unit = (kept-list row, 256-row slice). A row is (sequence, KV head
//    g, query block i); its G query heads share the row's list, so the slice
//    packs token-major rows (token, head) of all G heads into one M tile
//    (the PackGQA idea: one K/V tile load serves G heads).
//  * NW = 8 wavefronts x 32 packed rows (two wavefronts per SIMD); the
//    template is written for RG = 8 / NW row groups of 32 per wavefront (each
//    K or V^T operand read feeding RG MFMAs). S^T = K Q^T and O^T = V^T P^T on MFMA (bf16:
//    32x32x16; fp8: the scaled 32x32x64 f8f6f4 form with unit scales), so each
//    lane owns one query row per row group: row max and row sum are
//    lane-local plus one exchange with lane ^ 32, and the accumulator rescale
//    is a per-lane scalar.
//  * The online softmax is split in two: probabilities and sums without a
//    branch, then the rare rescale of the accumulators (the only branch).
//  * P never leaves registers: the PV contraction order over the keys of each
//    MFMA step is the order in which the QK^T accumulator already holds them.
//    V stays row-major in LDS and the V^T operand comes from transpose reads
//    (ds_read_b64_tr_b16 / _tr_b8) whose lane layout was pinned with probes.
//  * K/V tiles are filled one tile ahead by direct global->LDS loads into two
//    named buffers per operand (no register staging).
//  * After the kept tiles come summary tiles: the bf16 hi and lo parts of the
//    pooled keys of 64 consecutive blocks share one 128-row K tile, so two
//    MFMA passes give each pseudo-token logit about 16 mantissa bits; pooled
//    values are bf16; bias ln|block|. Kept, future and sink/diagonal pooled
//    columns are masked out.
//  * Units run heavy-row-first (sched), each row's slices on one XCD (unit
//    u goes to XCD u % 8) so they share that XCD's L2 copy of the K/V tiles.
// Every address is computed by the functions of attn_geom.h.
#include "attn_geom.h"

namespace fp {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(8))) int i32x8;
typedef __attribute__((ext_vector_type(2))) int i32x2;
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) uint8_t lds_u8;
typedef __attribute__((address_space(3))) bf16x8 lds_bf16x8;
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
typedef __attribute__((address_space(3))) i32x2 lds_i32x2;
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) u32x4 lds_u32x4;
typedef __attribute__((address_space(3))) int lds_int;
typedef __attribute__((address_space(3))) uint32_t lds_u32;

constexpr float LN2 = 0.6931471805599453f;

__device__ __forceinline__ uint32_t pk_bf16(float lo, float hi) {
    typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
    bf16x2 r;
    r[0] = (__bf16)lo;
    r[1] = (__bf16)hi;
    return __builtin_bit_cast(uint32_t, r);
}

__device__ __forceinline__ float bf16_round(float x) {
    return __uint_as_float(pk_bf16(x, 0.f) << 16);
}

// value of x held by lane l ^ 32 (permlane32 swap, no LDS traffic)
__device__ __forceinline__ float other_half(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(__lane_id() < 32 ? r[1] : r[0]);
}

// Online softmax, first part (no branch). One row group's tile held as S^T
// accumulators, log2 domain: element value s maps to logit s * f + bias,
// masked elements are -inf. Finds the lane's new reference maximum (lazy:
// it moves only when the tile maximum exceeds the old one by more than
// 2^LAZY; probabilities then reach at most 2^LAZY, harmless in fp32 sums and
// bf16 P; LAZY = 0 moves it whenever the maximum grows, and when it does not
// the rescale factor would be exactly 1), leaves the probabilities in sacc
// multiplied by 2^lw (the PV operand scale) and their sum in ts.
template <int NKB, int LAZY>
__device__ __forceinline__ void softmax_probs(f32x16 (&sacc)[NKB], float f, float bias, float lw, float m,
                                              float& mnew, float& ts, bool& need) {
    const float NEG_INF = -__builtin_inff();
    float mx = NEG_INF;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int v = 0; v < 16; ++v) mx = fmaxf(mx, sacc[kb][v]);
    mx = fmaxf(mx, other_half(mx));
    const float mcand = fmaxf(m, mx * f + bias);
    need = mcand > m + (float)LAZY;
    mnew = need ? mcand : m;
    const float nb = bias - (mnew == NEG_INF ? 0.f : mnew) + lw;
    float sum = 0.f;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            const float p = __builtin_amdgcn_exp2f(fmaf(sacc[kb][v], f, nb));
            sacc[kb][v] = p;
            sum += p;
        }
    ts = sum;
}

// Online softmax, second part: when any lane of the wavefront moved its
// reference, rescale the accumulators and running sums by 2^(m - mnew)
// (1 for lanes that did not); then add the tile's sum (without 2^lw).
template <int RG>
__device__ __forceinline__ void softmax_commit(const bool (&need)[RG], float (&m)[RG], const float (&mnew)[RG],
                                               float (&lsum)[RG], const float (&ts)[RG], float lw,
                                               f32x16 (&oacc)[RG][4]) {
    const float NEG_INF = -__builtin_inff();
    bool any = false;
#pragma unroll
    for (int rg = 0; rg < RG; ++rg) any |= need[rg];
    if (__builtin_amdgcn_ballot_w64(any) != 0ull) {
#pragma unroll
        for (int rg = 0; rg < RG; ++rg) {
            const float alpha = __builtin_amdgcn_exp2f(m[rg] - (mnew[rg] == NEG_INF ? 0.f : mnew[rg]));
            lsum[rg] *= alpha;
#pragma unroll
            for (int db = 0; db < 4; ++db)
#pragma unroll
                for (int v = 0; v < 16; ++v) oacc[rg][db][v] *= alpha;
        }
    }
#pragma unroll
    for (int rg = 0; rg < RG; ++rg) {
        m[rg] = mnew[rg];
        lsum[rg] += lw == 0.f ? ts[rg] : ts[rg] * __builtin_amdgcn_exp2f(-lw);
    }
}

// P -> E4M3 codes, 4 per dword (round to nearest even)
__device__ __forceinline__ uint32_t pk_fp8x4(float a, float b, float c, float d) {
    uint32_t w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0u, false);
    return __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
}

// OCP E4M3FN code -> float (exact)
__device__ __forceinline__ float e4m3_val(uint32_t c) {
    const uint32_t sgn = (c & 0x80u) << 24, e = (c >> 3) & 0xFu, mm = c & 0x7u;
    const float mag = e ? __uint_as_float(((e + 120u) << 23) | (mm << 20)) : (float)mm * 0.001953125f;
    return __uint_as_float(__float_as_uint(mag) | sgn);
}

// ---------------------------------------------------------------------------
// Direct global->LDS loads of one tile: each wavefront instruction fills
// 1 KiB of LDS (lane l -> bytes 16 l .. 16 l + 15). LDS row r holds key r
// (PERM: key vt_slot(r)); rows past the sequence repeat its last key.
// ---------------------------------------------------------------------------
// A 32-bit lane offset from a uniform base, passed through an empty asm so
// that the compiler cannot hoist a 64-bit widening of it out of the tile
// loop (two registers per offset): the load then takes the scalar-base form.
FP_HD uint32_t lane_off(uint32_t off) {
#if defined(__HIP_DEVICE_COMPILE__)
    asm volatile("" : "+v"(off));
#endif
    return off;
}

template <int STR, int BLK, int ESZ, bool PERM, int NW>
__device__ __forceinline__ void issue_full(const TileOffs<STR, BLK, ESZ, PERM, NW>& o, const uint8_t* tile_base,
                                           lds_u8* buf, int wave) {
#pragma unroll
    for (int k = 0; k < o.NP; ++k)
        if (o.has(k, wave))
            __builtin_amdgcn_global_load_lds((const void*)(tile_base + lane_off(o.off[k])),
                                             (lds_void*)(buf + (k * NW + wave) * PIECE), 16, 0, 0);
}

// Full paged tile, in two phases: every piece's page id is read first (pages
// = the tile's first slot in the staged list), then the loads are issued
// (base = the uniform part: head and the tile's in-page start). Reading LDS
// after some of the tile's loads are in flight would make the compiler drain
// them (it cannot tell the page list from the buffers being filled).
template <int STR, int BLK, int ESZ, bool PERM, int NW>
__device__ __forceinline__ void read_pages(const TileOffs<STR, BLK, ESZ, PERM, NW>& o, const lds_int* pages,
                                           int (&pg)[TileOffs<STR, BLK, ESZ, PERM, NW>::NP], int wave) {
#pragma unroll
    for (int k = 0; k < o.NP; ++k) pg[k] = o.has(k, wave) ? pages[o.page_slot(k)] : 0;
}
template <int STR, int BLK, int ESZ, bool PERM, int NW>
__device__ __forceinline__ void issue_paged(const TileOffs<STR, BLK, ESZ, PERM, NW>& o, const uint8_t* base,
                                            const int (&pg)[TileOffs<STR, BLK, ESZ, PERM, NW>::NP],
                                            unsigned long long page_bytes, lds_u8* buf, int wave) {
#pragma unroll
    for (int k = 0; k < o.NP; ++k)
        if (o.has(k, wave))
            __builtin_amdgcn_global_load_lds(
                (const void*)(base + (unsigned long long)pg[k] * page_bytes + o.in_page(k)),
                (lds_void*)(buf + (k * NW + wave) * PIECE), 16, 0, 0);
}

// Generic tile (ragged, or paged without the fast offsets): every piece's
// source is computed before any load is issued.
template <int STR, int BLK, int ESZ, bool PERM, bool PAGED, int NW>
__device__ __forceinline__ void issue_generic(const uint8_t* base, const KVAddr& ka, int b, int L, int g, int j,
                                              lds_u8* buf, int wave, int lane, const lds_int* pages) {
    using TO = TileOffs<STR, BLK, ESZ, PERM, NW>;
    asm volatile("" : "+v"(lane));   // recompute addresses per call, keep none live
    const uint8_t* src[TO::NP];
    auto pg = [&](int slot) { return pages[slot]; };
#pragma unroll
    for (int k = 0; k < TO::NP; ++k)
        src[k] = TO::has(k, wave) ? base + tile_src<STR, BLK, ESZ, PERM, PAGED>(ka, b, L, g, j, k * NW + wave, lane,
                                                                                 pg, pages != nullptr)
                                  : base;
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int k = 0; k < TO::NP; ++k)
        if (TO::has(k, wave))
            __builtin_amdgcn_global_load_lds((const void*)src[k], (lds_void*)(buf + (k * NW + wave) * PIECE), 16,
                                             0, 0);
}

template <int BLK, bool FP8, int NW>
struct KVOffs {
    static constexpr int ESZ = FP8 ? 1 : 2;
    TileOffs<FP8 ? KSTR8 : KSTR, BLK, ESZ, false, NW> k;
    TileOffs<FP8 ? VSTR8 : VSTR, BLK, ESZ, FP8, NW> v;
    static constexpr int NPK = decltype(k)::NP, NPV = decltype(v)::NP;
};

template <int BLK, bool FP8, bool PAGED, int NW>
__device__ __forceinline__ void issue_kv(const AttnArgs& a, int b, int L, int g, int j,
                                         lds_u8* kbuf, lds_u8* vbuf, int wave, int lane,
                                         const KVOffs<BLK, FP8, NW>& o, const lds_int* pages) {
    constexpr int ESZ = FP8 ? 1 : 2;
    if (PAGED && pages && a.paged_fast && (j + 1) * BLK <= L) {
        const int sh = a.ka.page_shift;
        const long long ub = (long long)((j * BLK) & ((1 << sh) - 1)) * a.ka.st + (long long)g * a.ka.sh;
        const lds_int* pt = pages + ((j * BLK) >> sh);
        int pgk[KVOffs<BLK, FP8, NW>::NPK], pgv[KVOffs<BLK, FP8, NW>::NPV];
        read_pages(o.k, pt, pgk, wave);
        read_pages(o.v, pt, pgv, wave);
        __builtin_amdgcn_sched_barrier(0);
        issue_paged(o.k, (const uint8_t*)a.k + ub * ESZ, pgk, (unsigned long long)a.ka.spage * ESZ, kbuf, wave);
        issue_paged(o.v, (const uint8_t*)a.v + ub * ESZ, pgv, (unsigned long long)a.va.spage * ESZ, vbuf, wave);
        return;
    }
    if (!PAGED && (j + 1) * BLK <= L) {
        const long long k0 = a.ka.template off<false>(b, j * BLK, g) * ESZ;
        const long long v0 = a.va.template off<false>(b, j * BLK, g) * ESZ;
        issue_full(o.k, (const uint8_t*)a.k + k0, kbuf, wave);
        issue_full(o.v, (const uint8_t*)a.v + v0, vbuf, wave);
        return;
    }
    issue_generic<FP8 ? KSTR8 : KSTR, BLK, ESZ, false, PAGED, NW>((const uint8_t*)a.k, a.ka, b, L, g, j, kbuf,
                                                                  wave, lane, pages);
    issue_generic<FP8 ? VSTR8 : VSTR, BLK, ESZ, FP8, PAGED, NW>((const uint8_t*)a.v, a.va, b, L, g, j, vbuf, wave,
                                                                lane, pages);
}

// Summary sub-tile m: the K tile holds the bf16 hi parts of its pooled keys
// in rows 0 .. SUMC-1 and the lo parts in rows SUMC .. BLK-1, so one tile load
// brings both and the two halves of QK^T accumulate into one logit.
// so (with fast): per-lane offsets for whole sub-tiles, kept in registers.
template <int BLK, int NW>
__device__ __forceinline__ void issue_summary(const AttnArgs& a, const SeqDesc& s, int g, int m,
                                              lds_u8* kbuf, lds_u8* vbuf, int wave, int lane,
                                              const SumOffs<BLK, NW>& so, bool fast) {
    using TG = TileGeom<BLK, false>;
    using SO = SumOffs<BLK, NW>;
    if (fast && SO::whole(m, s.nbk)) {
        const long long r0 = kbar_row(s, a.Hkv, g, TG::SUMC * m) * (D * 2);
        if (!a.scores) {
            const uint8_t* kb = (const uint8_t*)a.kbar_hi + r0;
#pragma unroll
            for (int k = 0; k < SO::NPK; ++k)
                if (SO::has_k(k, wave))
                    __builtin_amdgcn_global_load_lds((const void*)(kb + lane_off(so.k_off[k])),
                                                     (lds_void*)(kbuf + (k * NW + wave) * PIECE), 16, 0, 0);
        }
        const uint8_t* vb = (const uint8_t*)a.vbar_bf + r0;
#pragma unroll
        for (int k = 0; k < SO::NPV; ++k)
            if (SO::has_v(k, wave))
                __builtin_amdgcn_global_load_lds((const void*)(vb + (k * NW + wave) * PIECE + lane_off(so.v_off)),
                                                 (lds_void*)(vbuf + (k * NW + wave) * PIECE), 16, 0, 0);
        return;
    }
    // recompute the per-lane piece addresses here instead of keeping them
    // live across the tile loop (registers are the scarce resource)
    asm volatile("" : "+v"(lane));
#pragma unroll
    for (int w = 0; w < 2; ++w) {
        constexpr int KP = TG::SKPIECES, VP = TG::SVPIECES;
        if (w == 0 && a.scores) continue;           // block-score correction: no pooled keys needed
        lds_u8* buf = w == 0 ? kbuf : vbuf;
#pragma unroll
        for (int t0 = 0; t0 < (w == 0 ? KP : VP); t0 += NW) {
            const int t = t0 + wave;
            if (t < (w == 0 ? KP : VP)) {
                const SummarySrc src = summary_src<BLK>(s, a.Hkv, g, m, w, t, lane);
                const __bf16* arr = src.which == 0 ? a.kbar_hi : (src.which == 1 ? a.kbar_lo : a.vbar_bf);
                __builtin_amdgcn_global_load_lds((const void*)(arr + src.off), (lds_void*)(buf + t * PIECE), 16, 0,
                                                 0);
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Tile compute
// ---------------------------------------------------------------------------
// bf16 S^T for key blocks kb0 .. kb0 + NB - 1 (32 keys each) of the tile, all
// row groups: each K operand read feeds RG MFMAs.
template <int RG, int NB, int DORD, bool ACC>
__device__ __forceinline__ void qk_pad(const lds_u8* kt, const bf16x8 (&qf)[RG][8], int n, int lh, int kb0,
                                       f32x16 (&sacc)[RG][NB]) {
    if (!ACC) {
#pragma unroll
        for (int rg = 0; rg < RG; ++rg)
#pragma unroll
            for (int kb = 0; kb < NB; ++kb)
#pragma unroll
                for (int v = 0; v < 16; ++v) sacc[rg][kb][v] = 0.f;
    }
#pragma unroll
    for (int ks = 0; ks < 8; ++ks)
#pragma unroll
        for (int kb = 0; kb < NB; ++kb) {
            const bf16x8 aop = *(const lds_bf16x8*)(kt + k_read_off<DORD>(kb0 + kb, ks, n, lh));
#pragma unroll
            for (int rg = 0; rg < RG; ++rg)
                sacc[rg][kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aop, qf[rg][ks], sacc[rg][kb], 0, 0, 0);
        }
}

// bf16 O^T += V^T P^T: A operand = V^T fragment gathered by two transpose
// reads (16-lane group: lane 4e + r addresses V[k0 + e][d0 + 4r .. +4], lane
// i receives V[k0 + e][d0 + i] for e = 0..3); B operand = P from registers.
template <int RG, int NB>
__device__ __forceinline__ void pv_tr(const f32x16 (&sacc)[RG][NB], const lds_u8* vt, int lane, int kb0,
                                      f32x16 (&oacc)[RG][4]) {
#pragma unroll
    for (int kb = 0; kb < NB; ++kb)
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) {
            bf16x8 bop[RG];
#pragma unroll
            for (int rg = 0; rg < RG; ++rg)
#pragma unroll
                for (int e = 0; e < 8; ++e) bop[rg][e] = (__bf16)sacc[rg][kb][8 * s2 + e];
#pragma unroll
            for (int db = 0; db < 4; ++db) {
                s16x4 h[2];
#pragma unroll
                for (int aa = 0; aa < 2; ++aa)
                    h[aa] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                        (lds_s16x4*)(vt + v_read_off(kb0 + kb, s2, aa, db, lane)));
                const s16x4 h0 = h[0], h1 = h[1];
                typedef short s16x8 __attribute__((ext_vector_type(8)));
                const s16x8 cat = {h0[0], h0[1], h0[2], h0[3], h1[0], h1[1], h1[2], h1[3]};
                const bf16x8 aop = __builtin_bit_cast(bf16x8, cat);
#pragma unroll
                for (int rg = 0; rg < RG; ++rg)
                    oacc[rg][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aop, bop[rg], oacc[rg][db], 0, 0, 0);
            }
        }
}

// fp8 S^T for key blocks kb0, kb0 + 1: A = K rows (32 bytes per lane per
// 64-dim step, dims 64 ks + 32 lh ..), B = the query codes.
template <int RG>
__device__ __forceinline__ void qk_f8(const lds_u8* kt, const i32x8 (&qf8)[RG][2], int n, int lh, int kb0,
                                      f32x16 (&sacc)[RG][2]) {
#pragma unroll
    for (int rg = 0; rg < RG; ++rg)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int v = 0; v < 16; ++v) sacc[rg][kb][v] = 0.f;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            const lds_u8* ap = kt + k8_read_off(kb0 + kb, ks, n, lh);
            const u32x4 w0 = *(const lds_u32x4*)ap, w1 = *(const lds_u32x4*)(ap + 16);
            i32x8 aop;
            aop[0] = w0[0]; aop[1] = w0[1]; aop[2] = w0[2]; aop[3] = w0[3];
            aop[4] = w1[0]; aop[5] = w1[1]; aop[6] = w1[2]; aop[7] = w1[3];
#pragma unroll
            for (int rg = 0; rg < RG; ++rg)
                sacc[rg][kb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(aop, qf8[rg][ks], sacc[rg][kb], 0, 0,
                                                                              0, 127, 0, 127);
        }
}

// fp8 O^T += V^T P^T over the 64-key step s2 (accumulators sacc[rg][0..1]).
// B-lane (n, lh) byte e = 16 kbit + v holds P of key 32 kbit + 8 (v / 4) +
// 4 lh + v % 4. Transpose read c (16-lane group: lane i receives byte i % 8
// of the 8 bytes addressed by lane 2 e' + i / 8, e' = 0..7) gives A bytes
// 8c .. 8c + 7; with the keys stored at LDS row vt_slot(key), the 8 rows a
// lane half needs are the consecutive rows 16 c + 8 lh + e'.
template <int RG>
__device__ __forceinline__ void pv_f8(const f32x16 (&sacc)[RG][2], const lds_u8* vt, int lane, int s2,
                                      f32x16 (&oacc)[RG][4]) {
    i32x8 bop[RG];
#pragma unroll
    for (int rg = 0; rg < RG; ++rg)
#pragma unroll
        for (int kbit = 0; kbit < 2; ++kbit)
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4)
                bop[rg][4 * kbit + q4] =
                    (int)pk_fp8x4(sacc[rg][kbit][4 * q4], sacc[rg][kbit][4 * q4 + 1], sacc[rg][kbit][4 * q4 + 2],
                                  sacc[rg][kbit][4 * q4 + 3]);
#pragma unroll
    for (int db = 0; db < 4; ++db) {
        i32x8 aop;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const i32x2 r = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2*)(vt + v8_read_off(s2, c, db, lane)));
            aop[2 * c] = r[0];
            aop[2 * c + 1] = r[1];
        }
#pragma unroll
        for (int rg = 0; rg < RG; ++rg)
            oacc[rg][db] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(aop, bop[rg], oacc[rg][db], 0, 0, 0, 127,
                                                                          0, 127);
    }
}

// fp8 tile scales (one per 128 keys) as vector loads: the value is consumed a
// tile later, after the barrier's vector-memory wait, so it never stalls
__device__ __forceinline__ float load_scale(const float* p, long long idx) {
    int z = 0;
    asm volatile("" : "+v"(z));
    return p[idx + z];
}

template <int BLK, bool FP8, bool PAGED, typename Geo, int NW, bool SPLIT>
__global__ __launch_bounds__(NW * 64, 1) void attn_tile_kernel(Geo geo, AttnArgs a) {
    using TG = TileGeom<BLK, FP8>;
    constexpr int RG = 8 / NW;                      // 32-row groups per wavefront
    constexpr int NT = NW * 64;
    constexpr int NKB = TG::NKB;
    constexpr int SB = TG::SB;
    // two distinct buffers per operand (not one indexed array), so the
    // compiler can tell the tile being read from the tile being loaded
    __shared__ __align__(1024) uint8_t kA_[TG::KTILE];
    __shared__ __align__(1024) uint8_t kB_[TG::KTILE];
    __shared__ __align__(1024) uint8_t vA_[TG::VTILE];
    __shared__ __align__(1024) uint8_t vB_[TG::VTILE];
    __shared__ uint32_t kept[MAX_NB / 32];
    __shared__ int svmax_sh;
    // paged K/V: the sequence's page ids (K and V share the block table)
    constexpr int PAGE_CAP = 2048;
    __shared__ int pages_sh[PAGED ? PAGE_CAP : 1];
    lds_u8* const kA = (lds_u8*)kA_;
    lds_u8* const kB = (lds_u8*)kB_;
    lds_u8* const vA = (lds_u8*)vA_;
    lds_u8* const vB = (lds_u8*)vB_;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform: scalar LDS bases
    const int n = lane & 31, lh = lane >> 5;
    const float NEG_INF = -__builtin_inff();

    const UnitMap um = unit_map(blockIdx.x, a.slices, SPLIT ? a.nsplit : 1);
    if (um.pidx >= a.rows) return;
    // dense: rows in reverse order, so every (sequence, KV head) runs its
    // longest rows (latest query blocks) first
    const int r = a.dense ? a.rows - 1 - um.pidx : (a.sched ? a.sched[um.pidx] : um.pidx);
    const int b = geo.seq_of_row(r);
    const SeqDesc s = geo.seq(b);
    const int rl = r - s.row0;
    const int g = rl / s.nq, il = rl % s.nq;       // g: the row's group of query heads
    const int gk = g / a.kv_div;                     // its KV head
    const int i = s.i0 + il;
    const int t_lo = max(i * BLK, s.P), t_hi = min((i + 1) * BLK, s.L);
    const int G = a.G;
    const int npk = G * (t_hi - t_lo);
    if (um.slice * 256 >= npk) return;              // uniform over the workgroup

    // Two wavefronts per SIMD (w and w + 4) get different issue priorities, so
    // after each barrier one runs its MFMA phase ahead and the other's softmax
    // VALU work fills the MFMA pipe's shadow.
    if (NW == 8 && wave < 4) __builtin_amdgcn_s_setprio(1);

    int t[RG], h[RG];
    bool valid[RG];
#pragma unroll
    for (int rg = 0; rg < RG; ++rg) {
        const int prow = packed_row<NW>(um.slice, wave, rg, n);
        valid[rg] = prow < npk;
        const int tl = prow / G;
        t[rg] = t_lo + tl;
        h[rg] = g * G + (prow - tl * G);
    }

    // kept list of the row: from the CSR, or every block j <= i when dense
    const int rp0 = a.dense ? 0 : a.row_ptr[r];
    const int nnz = a.dense ? i + 1 : a.row_ptr[r + 1] - rp0;
    // kept codes are clamped to the row's blocks: a caller's list cannot move a tile load off the row
    const int j0 = a.dense ? 0 : min(max(a.col_idx[rp0], 0), i);
    // bf16: the kept blocks of the row, in their order (the CSR list), code t
    // in lane t mod 64 of kc, loaded 64 at a time, so the next kept code is one
    // lane read rather than a scan of the LDS bitmap (the fp8 kernel measured
    // no gain from it and scans). kt: the current tile's index in the list.
    constexpr bool LIST_CODES = !FP8;
    int kt = 0;
    int kc = (LIST_CODES && !a.dense && lane < nnz) ? a.col_idx[rp0 + lane] : 0;
    KVOffs<BLK, FP8, NW> kvo;
    if (!PAGED) {
        kvo.k.init(a.ka.st, wave, lane);
        kvo.v.init(a.va.st, wave, lane);
    } else if (a.paged_fast) {
        constexpr int LB = BLK == 128 ? 7 : 6;
        const int lshift = min(a.ka.page_shift, LB);
        kvo.k.init_paged(a.ka.st, lshift, wave, lane);
        kvo.v.init_paged(a.va.st, lshift, wave, lane);
    }
    // whole summary sub-tiles load through offsets computed once (not in split
    // parts, whose registers are full, nor in the paged fp8 kernel, which sits
    // at the register limit with them); the lo array must lie within 2 GiB
    // after the hi array for 32-bit offsets
    SumOffs<BLK, NW> so;
    constexpr bool SUM_OFFS = !SPLIT && !(PAGED && FP8);
    const unsigned long long lo_delta = (unsigned long long)((const char*)a.kbar_lo - (const char*)a.kbar_hi);
    const bool sum_fast = SUM_OFFS && !a.dense && lo_delta < (1ull << 31);
    if (sum_fast) so.init((uint32_t)lo_delta, wave, lane);
    // the first tile; a split row's part learns its first tile from the kept bitmap
    if (!SPLIT) issue_kv<BLK, FP8, PAGED, NW>(a, b, s.L, gk, j0, kA, vA, wave, lane, kvo, nullptr);
    // paged: stage the page ids for the later tiles (visible after the
    // barrier that follows the kept-bitmap build)
    const lds_int* pages = nullptr;
    if constexpr (PAGED) {
        const int npg = (s.L + (1 << a.ka.page_shift) - 1) >> a.ka.page_shift;
        if (npg <= PAGE_CAP) {
            const int* row = a.ka.table + (long long)b * a.ka.maxp;
            for (int p = tid; p < npg; p += NT) pages_sh[p] = row[p];
            pages = (const lds_int*)pages_sh;
        }
    }

    // Query fragments. bf16: lane (n, lh) holds q[t, h, 16 ks + 8 lh .. + 8];
    // fp8: the codes q[t, h, 64 ks + 32 lh .. + 32], widened to bf16 (exact)
    // in that order only when the summary tiles start.
    bf16x8 qf[RG][8];
    i32x8 qf8[RG][2];
    float f_row[RG];
#pragma unroll
    for (int rg = 0; rg < RG; ++rg) {
        f_row[rg] = a.scale_log2;
        if constexpr (FP8) {
            const uint8_t* qp = (const uint8_t*)a.q + (valid[rg] ? a.qa.off(b, s, t[rg], h[rg]) : 0);
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                const uint4 w0 =
                    valid[rg] ? *(const uint4*)(qp + ks * 64 + lh * 32) : make_uint4(0u, 0u, 0u, 0u);
                const uint4 w1 =
                    valid[rg] ? *(const uint4*)(qp + ks * 64 + lh * 32 + 16) : make_uint4(0u, 0u, 0u, 0u);
                qf8[rg][ks][0] = w0.x; qf8[rg][ks][1] = w0.y; qf8[rg][ks][2] = w0.z; qf8[rg][ks][3] = w0.w;
                qf8[rg][ks][4] = w1.x; qf8[rg][ks][5] = w1.y; qf8[rg][ks][6] = w1.z; qf8[rg][ks][7] = w1.w;
            }
            if (valid[rg]) f_row[rg] *= a.qs.at(b, h[rg], t[rg]);
        } else {
            const __bf16* qp = (const __bf16*)a.q + (valid[rg] ? a.qa.off(b, s, t[rg], h[rg]) : 0);
#pragma unroll
            for (int ks = 0; ks < 8; ++ks) {
                if (valid[rg]) qf[rg][ks] = *(const bf16x8*)(qp + ks * 16 + lh * 8);
                else
#pragma unroll
                    for (int e = 0; e < 8; ++e) qf[rg][ks][e] = (__bf16)0.f;
            }
        }
    }
    // fp8 tile scales of this row's (sequence, KV head): one per 128 keys
    const float* ksp = FP8 ? a.ks.p + (long long)b * a.ks.sb + (long long)gk * a.ks.sh : nullptr;
    const float* vsp = FP8 ? a.vs.p + (long long)b * a.vs.sb + (long long)gk * a.vs.sh : nullptr;
    float ksA = 1.f, vsA = 1.f, ksB = 1.f, vsB = 1.f;
    if constexpr (FP8 && !SPLIT) {
        ksA = load_scale(ksp, (j0 * BLK) >> 7);
        vsA = load_scale(vsp, (j0 * BLK) >> 7);
    }

    const int nw = (i >> 5) + 1;
    for (int w = tid; w < nw; w += NT) kept[w] = 0u;
    if (FP8 && tid == 0) svmax_sh = 0;
    __syncthreads();
    float svm = 0.f;
    for (int e = tid; e < nnz; e += NT) {
        const int j = a.dense ? e : a.col_idx[rp0 + e];
        if ((unsigned)j > (unsigned)i) continue;      // not a block of this row: ignored
        atomicOr(&kept[j >> 5], 1u << (j & 31));
        if (FP8) svm = fmaxf(svm, vsp[(j * BLK) >> 7]);
    }
    if constexpr (FP8) {
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) svm = fmaxf(svm, __shfl_xor(svm, off, 64));
        if (lane == 0) atomicMax(&svmax_sh, __float_as_int(svm));   // non-negative floats order as ints
    }

    float m[RG], lsum[RG];
    f32x16 oacc[RG][4];
#pragma unroll
    for (int rg = 0; rg < RG; ++rg) {
        m[rg] = NEG_INF;
        lsum[rg] = 0.f;
#pragma unroll
        for (int db = 0; db < 4; ++db)
#pragma unroll
            for (int v = 0; v < 16; ++v) oacc[rg][db][v] = 0.f;
    }
    const float lnb2 = (BLK == 128) ? 7.f : 6.f;    // log2 |block| of a pruned pseudo-token
    __syncthreads();                                  // tile 0 landed; kept bitmap complete
    // fp8: PV accumulates P 2^8 sv_j / svmax times the value codes (P <= 1:
    // no lazy rescale there), undone in the epilogue
    const float svmax = FP8 ? fmaxf(__int_as_float(svmax_sh), 1e-30f) : 1.f;
    const float lsvmax = FP8 ? __log2f(svmax) : 0.f;
    const uint32_t* kbits = kept;
    const bool no_corr = a.no_correction != 0;

    auto issue = [&](int code, lds_u8* kb, lds_u8* vb, float& ksn, float& vsn) __attribute__((always_inline)) {
        if (code >= 0) {
            issue_kv<BLK, FP8, PAGED, NW>(a, b, s.L, gk, code, kb, vb, wave, lane, kvo, pages);
            if constexpr (FP8) {
                ksn = load_scale(ksp, (code * BLK) >> 7);
                vsn = load_scale(vsp, (code * BLK) >> 7);
            }
        } else {
            issue_summary<BLK, NW>(a, s, gk, -1 - code, kb, vb, wave, lane, so, sum_fast);
        }
    };
    // causal mask inside the diagonal tile: keys after the row's token
    auto mask_diag = [&](f32x16 (&sh)[RG][2], int code, int hf) __attribute__((always_inline)) {
#pragma unroll
        for (int rg = 0; rg < RG; ++rg)
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    const int sk = code * BLK + (2 * hf + kb) * 32 + 8 * (v >> 2) + 4 * lh + (v & 3);
                    sh[rg][kb][v] = sk > t[rg] ? NEG_INF : sh[rg][kb][v];
                }
    };
    // softmax of one 64-key half of every row group, without the rescale
    auto probs = [&](f32x16 (&sh)[RG][2], const float (&f)[RG], float lw, float (&mn)[RG], float (&ts)[RG],
                     bool (&nd)[RG]) __attribute__((always_inline)) {
#pragma unroll
        for (int rg = 0; rg < RG; ++rg) {
            if constexpr (FP8) softmax_probs<2, 0>(sh[rg], f[rg], 0.f, lw, m[rg], mn[rg], ts[rg], nd[rg]);
            else softmax_probs<2, 8>(sh[rg], f[rg], 0.f, lw, m[rg], mn[rg], ts[rg], nd[rg]);
        }
    };
    auto qk_half = [&](const lds_u8* kc, int hf, f32x16 (&sh)[RG][2]) __attribute__((always_inline)) {
        if constexpr (FP8) qk_f8<RG>(kc, qf8, n, lh, 2 * hf, sh);
        else qk_pad<RG, 2, 0, false>(kc, qf, n, lh, 2 * hf, sh);
    };
    auto pv_half = [&](const f32x16 (&sh)[RG][2], const lds_u8* vc, int hf) __attribute__((always_inline)) {
        if constexpr (FP8) pv_f8<RG>(sh, vc, lane, hf, oacc);
        else pv_tr<RG, 2>(sh, vc, lane, 2 * hf, oacc);
    };
    // Exact tokens of kept block `code`, 64 keys at a time (32 S registers
    // live per row group).
    auto compute_kept = [&](int code, const lds_u8* kc, const lds_u8* vc, float ksj, float vsj)
                            __attribute__((always_inline)) {
        float f[RG];
#pragma unroll
        for (int rg = 0; rg < RG; ++rg) f[rg] = FP8 ? f_row[rg] * ksj : f_row[rg];
        const float lw = FP8 ? 8.f + __log2f(fmaxf(vsj, 1e-30f)) - lsvmax : 0.f;
        float mn[RG], ts[RG];
        bool nd[RG];
#pragma unroll
        for (int hf = 0; hf < NKB / 2; ++hf) {
            f32x16 sh[RG][2];
            qk_half(kc, hf, sh);
            if (code == i) mask_diag(sh, code, hf);
            probs(sh, f, lw, mn, ts, nd);
            softmax_commit<RG>(nd, m, mn, lsum, ts, lw, oacc);
            pv_half(sh, vc, hf);
        }
    };
    // fp8: the pseudo-token weights join the accumulator in its 2^8 / svmax units
    const float lw_sum = FP8 ? 8.f - lsvmax : 0.f;
    // Pooled pseudo-tokens of summary sub-tile -1 - code: hi and lo halves of
    // QK^T accumulate into one logit per pooled column; pseudo-tokens of kept
    // or non-causal columns are masked from the LDS bitmap.
    auto compute_summary = [&](int code, const lds_u8* kc, const lds_u8* vc) __attribute__((always_inline)) {
        const int mm = -1 - code;
        f32x16 sh[RG][SB];
        float fs[RG];
        // Pseudo-tokens of kept, future, sink and diagonal columns are masked by
        // an additive bias, 0 or -inf per column: accumulator element v of lane
        // half lh holds column 8 (v / 4) + 4 lh + v % 4 of the 32-column block,
        // so one sign-extended bit of the lane's shifted word gives the bias
        // bits (0 or those of -inf), and the bias starts the QK^T accumulation.
        auto set_bias = [&]() __attribute__((always_inline)) {
#pragma unroll
            for (int kb = 0; kb < SB; ++kb) {
                const int c0 = mm * TG::SUMC + kb * 32;
                const uint32_t pw = ~kept[min(c0 >> 5, MAX_NB / 32 - 1)] & range_bits(c0, 1, i - 1);
                const uint32_t masked = ~(lh ? pw >> 4 : pw);     // bit 8 q + r: column 8 q + 4 lh + r masked
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    // the empty asm keeps the extract and the and as two instructions
                    // (the compiler would otherwise rebuild a compare and a select)
                    int ext = __builtin_amdgcn_sbfe((int)masked, 8 * (v >> 2) + (v & 3), 1);
                    asm volatile("" : "+v"(ext));
                    const float bias = __int_as_float(ext & (int)0xFF800000);
#pragma unroll
                    for (int rg = 0; rg < RG; ++rg) sh[rg][kb][v] = bias;
                }
            }
        };
        if (a.scores) {
            // block-score correction: the pseudo-token logit of column j is the
            // block score S[h, i, j] (scale included), the same for every row
            // of the query block; masked columns are selected out
#pragma unroll
            for (int rg = 0; rg < RG; ++rg) {
                const float* srow = a.scores + score_off(s, h[rg], il, 0);
#pragma unroll
                for (int kb = 0; kb < SB; ++kb) {
                    const int c0 = mm * TG::SUMC + kb * 32;
                    const uint32_t pw = ~kept[min(c0 >> 5, MAX_NB / 32 - 1)] & range_bits(c0, 1, i - 1);
#pragma unroll
                    for (int v = 0; v < 16; ++v) {
                        const int bit = 8 * (v >> 2) + 4 * lh + (v & 3);
                        const float sc = srow[min(c0 + bit, s.nbk - 1)];
                        sh[rg][kb][v] = ((pw >> bit) & 1u) ? sc : NEG_INF;
                    }
                }
                fs[rg] = 1.4426950408889634f;                        // log2(e): S is in natural-log units
            }
        } else {
            set_bias();
            qk_pad<RG, SB, FP8 ? 1 : 0, true>(kc, qf, n, lh, 0, sh);     // hi rows
            qk_pad<RG, SB, FP8 ? 1 : 0, true>(kc, qf, n, lh, SB, sh);    // lo rows, same columns
#pragma unroll
            for (int rg = 0; rg < RG; ++rg) fs[rg] = f_row[rg];
        }
        float mn[RG], ts[RG];
        bool nd[RG];
#pragma unroll
        for (int rg = 0; rg < RG; ++rg) softmax_probs<SB, 8>(sh[rg], fs[rg], lnb2, lw_sum, m[rg], mn[rg], ts[rg], nd[rg]);
        softmax_commit<RG>(nd, m, mn, lsum, ts, lw_sum, oacc);
        pv_tr<RG, SB>(sh, vc, lane, 0, oacc);
    };

    // A split row's part runs tiles [first, first + count) of the row's
    // sequence (kept blocks, then summary sub-tiles): `remaining` counts them
    // down and ends the sequence after the last.
    int code0 = j0, remaining = 0x7fffffff;
    if constexpr (SPLIT) {
        const int T = __builtin_amdgcn_readfirstlane(nnz + (no_corr ? 0 : count_summary<TG::SUMC>(kbits, i, no_corr)));
        const SplitRange sr = split_range(T, um.split, a.nsplit);
        remaining = __builtin_amdgcn_readfirstlane(sr.count);
        if (remaining == 0) {
            // an empty part: nothing to add (m = -inf, l = 0, O = 0)
            const long long pu = split_part(um.pidx, a.slices, um.slice, a.nsplit, um.split);
#pragma unroll
            for (int rg = 0; rg < RG; ++rg) {
                if (!valid[rg]) continue;
                const int pl = packed_row<NW>(0, wave, rg, n);
                float* po = a.part_o + (pu * SLICE_ROWS + pl) * D;
#pragma unroll
                for (int db = 0; db < 4; ++db)
#pragma unroll
                    for (int q4 = 0; q4 < 4; ++q4)
                        *(float4*)(po + db * 32 + q4 * 8 + lh * 4) = make_float4(0.f, 0.f, 0.f, 0.f);
                if (lh == 0) *(float2*)(a.part_ml + (pu * SLICE_ROWS + pl) * 2) = make_float2(NEG_INF, 0.f);
            }
            return;
        }
        code0 = sr.first < nnz ? (a.dense ? sr.first : min(max(a.col_idx[rp0 + sr.first], 0), i))
                               : nth_summary<TG::SUMC>(kbits, i, sr.first - nnz, no_corr);
        code0 = __builtin_amdgcn_readfirstlane(code0);
        kt = __builtin_amdgcn_readfirstlane(sr.first);
        if (LIST_CODES && !a.dense && kt >= 64) kc = (kt - (kt & 63) + lane < nnz) ? a.col_idx[rp0 + kt - (kt & 63) + lane] : 0;
        issue(code0, kA, vA, ksA, vsA);
        __syncthreads();                              // the part's first tile landed
    }
    // the code after `code` in the sequence (kept block or summary sub-tile)
    auto next_tile = [&](int code) __attribute__((always_inline)) {
        if (SPLIT && --remaining <= 0) return TILE_NONE;
        if (LIST_CODES && code >= 0) {
            ++kt;
            if (kt >= nnz) return next_summary<TG::SUMC>(kbits, i, 0, no_corr);
            if (a.dense) return kt;                   // dense: every block j <= i, in order
            if ((kt & 63) == 0) kc = (kt + lane < nnz) ? a.col_idx[rp0 + kt + lane] : 0;
            return min(max(__builtin_amdgcn_readlane(kc, kt & 63), 0), i);
        }
        return next_code<TG::SUMC>(kbits, i, code, no_corr);
    };
    auto next_sum = [&](int code) __attribute__((always_inline)) {
        if (SPLIT && --remaining <= 0) return TILE_NONE;
        return next_summary<TG::SUMC>(kbits, i, -code, no_corr);
    };

    // Kept phase. Buffers alternate A, B; the loop ends once the code of the
    // following tile is a summary code (already issued) or NONE (both < 0).
    int nxt, ca = code0;
    bool in_b = false;
    if (!SPLIT || code0 >= 0) {
        while (true) {
            const int cb = next_tile(ca);
            if (cb != TILE_NONE) issue(cb, kB, vB, ksB, vsB);
            compute_kept(ca, kA, vA, ksA, vsA);
            __syncthreads();                          // next tile landed; A is free
            if (cb < 0) { nxt = cb; in_b = true; break; }
            const int cn = next_tile(cb);
            if (cn != TILE_NONE) issue(cn, kA, vA, ksA, vsA);
            compute_kept(cb, kB, vB, ksB, vsB);
            __syncthreads();
            if (cn < 0) { nxt = cn; in_b = false; break; }
            ca = cn;
        }
    } else {
        nxt = code0;                                  // the part starts among the summary sub-tiles (in A)
    }
    if constexpr (FP8) {
        // widen the query codes to bf16 (exact) in the fp8 fragment's dim order
        if (nxt != TILE_NONE) {
#pragma unroll
            for (int rg = 0; rg < RG; ++rg)
#pragma unroll
                for (int ks = 0; ks < 8; ++ks)
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        const int byte = (ks & 3) * 8 + e;              // within the 32-byte half
                        const uint32_t w = (uint32_t)qf8[rg][ks >> 2][byte >> 2];
                        qf[rg][ks][e] = (__bf16)e4m3_val((w >> ((byte & 3) * 8)) & 0xFFu);
                    }
        }
    }
    // Summary phase: realign so the loop below always starts on buffer A.
    if (in_b && nxt != TILE_NONE) {
        const int cn = next_sum(nxt);
        if (cn != TILE_NONE) issue_summary<BLK, NW>(a, s, gk, -1 - cn, kA, vA, wave, lane, so, sum_fast);
        compute_summary(nxt, kB, vB);
        __syncthreads();
        nxt = cn;
    }
    while (nxt != TILE_NONE) {
        const int cb = next_sum(nxt);
        if (cb != TILE_NONE) issue_summary<BLK, NW>(a, s, gk, -1 - cb, kB, vB, wave, lane, so, sum_fast);
        compute_summary(nxt, kA, vA);
        __syncthreads();
        if (cb == TILE_NONE) break;
        const int cn = next_sum(cb);
        if (cn != TILE_NONE) issue_summary<BLK, NW>(a, s, gk, -1 - cn, kA, vA, wave, lane, so, sum_fast);
        compute_summary(cb, kB, vB);
        __syncthreads();
        nxt = cn;
    }

    // ---------------- epilogue ----------------
    float ltot[RG];
#pragma unroll
    for (int rg = 0; rg < RG; ++rg) ltot[rg] = lsum[rg] + other_half(lsum[rg]);
    if constexpr (SPLIT) {
        // the part's unnormalised O (fp8: in value units) and (m, l), for the merge
        const long long pu = split_part(um.pidx, a.slices, um.slice, a.nsplit, um.split);
        const float sc = FP8 ? svmax * 0.00390625f : 1.f;
#pragma unroll
        for (int rg = 0; rg < RG; ++rg) {
            if (!valid[rg]) continue;
            const int pl = packed_row<NW>(0, wave, rg, n);
            float* po = a.part_o + (pu * SLICE_ROWS + pl) * D;
#pragma unroll
            for (int db = 0; db < 4; ++db)
#pragma unroll
                for (int q4 = 0; q4 < 4; ++q4)
                    *(float4*)(po + db * 32 + q4 * 8 + lh * 4) =
                        make_float4(oacc[rg][db][4 * q4] * sc, oacc[rg][db][4 * q4 + 1] * sc,
                                    oacc[rg][db][4 * q4 + 2] * sc, oacc[rg][db][4 * q4 + 3] * sc);
            if (lh == 0) *(float2*)(a.part_ml + (pu * SLICE_ROWS + pl) * 2) = make_float2(m[rg], ltot[rg]);
        }
        return;
    }
#pragma unroll
    for (int rg = 0; rg < RG; ++rg) {
        if (!valid[rg]) continue;
        const float inv = (FP8 ? svmax * 0.00390625f : 1.f) / ltot[rg];
        if (a.o_f32) {
            float* op = (float*)a.o + a.oa.off(b, s, t[rg], h[rg]);
#pragma unroll
            for (int db = 0; db < 4; ++db)
#pragma unroll
                for (int q4 = 0; q4 < 4; ++q4)
                    *(float4*)(op + db * 32 + q4 * 8 + lh * 4) =
                        make_float4(oacc[rg][db][4 * q4] * inv, oacc[rg][db][4 * q4 + 1] * inv,
                                    oacc[rg][db][4 * q4 + 2] * inv, oacc[rg][db][4 * q4 + 3] * inv);
        } else {
            __bf16* op = (__bf16*)a.o + a.oa.off(b, s, t[rg], h[rg]);
#pragma unroll
            for (int db = 0; db < 4; ++db)
#pragma unroll
                for (int q4 = 0; q4 < 4; ++q4) {
                    uint2 w;
                    w.x = pk_bf16(oacc[rg][db][4 * q4] * inv, oacc[rg][db][4 * q4 + 1] * inv);
                    w.y = pk_bf16(oacc[rg][db][4 * q4 + 2] * inv, oacc[rg][db][4 * q4 + 3] * inv);
                    *(uint2*)(op + db * 32 + q4 * 8 + lh * 4) = w;
                }
        }
        if (a.lse && lh == 0) a.lse[a.la.off(b, s, t[rg], h[rg])] = (m[rg] + __log2f(ltot[rg])) * LN2;
    }
}

// bf16 operands of the summary tiles: Kbar = hi + lo (two bf16 terms), Vbar
// (only Vbar when kbar is null).
__global__ __launch_bounds__(256) void summary_prep_kernel(const float* kbar, const float* vbar, __bf16* hi,
                                                           __bf16* lo, __bf16* vb, long long n4) {
    const long long e = (long long)blockIdx.x * 256 + threadIdx.x;
    if (e >= n4) return;
    const float4 v = ((const float4*)vbar)[e];
    uint2 w;
    w.x = pk_bf16(v.x, v.y);
    w.y = pk_bf16(v.z, v.w);
    ((uint2*)vb)[e] = w;
    if (!kbar) return;                  // pooled values only
    const float4 k = ((const float4*)kbar)[e];
    uint2 h, l;
    h.x = pk_bf16(k.x, k.y);
    h.y = pk_bf16(k.z, k.w);
    l.x = pk_bf16(k.x - bf16_round(k.x), k.y - bf16_round(k.y));
    l.y = pk_bf16(k.z - bf16_round(k.z), k.w - bf16_round(k.w));
    ((uint2*)hi)[e] = h;
    ((uint2*)lo)[e] = l;
}

hipError_t launch_summary_prep(const float* kbar, const float* vbar, __bf16* hi, __bf16* lo, __bf16* vb,
                               long long nfloats, hipStream_t st) {
    const long long n4 = nfloats / 4;
    if (n4 == 0) return hipSuccess;
    summary_prep_kernel<<<(unsigned)((n4 + 255) / 256), 256, 0, st>>>(kbar, vbar, hi, lo, vb, n4);
    return hipGetLastError();
}

// Merge of a split row's parts: one workgroup per 8 packed rows of a (row,
// slice), 32 threads per packed row (4 dims each). With M = max m_s and
// w_s = 2^(m_s - M): o = sum w_s O_s / sum w_s l_s, lse = (M + log2 sum w_s l_s)
// ln 2; the parts are added in their order, so the result does not depend on
// timing. Every part's (m, l), then every part's O, is loaded before use.
constexpr int MERGE_ROWS = 8;
template <typename Geo>
__global__ __launch_bounds__(256) void split_merge_kernel(Geo geo, AttnArgs a, int blk) {
    constexpr int GROUPS = SLICE_ROWS / MERGE_ROWS;
    const int grp = blockIdx.x % GROUPS, unit = blockIdx.x / GROUPS;
    const int slice = unit % a.slices, pidx = unit / a.slices;
    if (pidx >= a.rows) return;
    const int r = a.sched ? a.sched[pidx] : pidx;
    const int b = geo.seq_of_row(r);
    const SeqDesc s = geo.seq(b);
    const int rl = r - s.row0;
    const int g = rl / s.nq, il = rl % s.nq;
    const int i = s.i0 + il;
    const int t_lo = max(i * blk, s.P), t_hi = min((i + 1) * blk, s.L);
    const int npk = a.G * (t_hi - t_lo);
    const int c = threadIdx.x & 31;
    const int pl = grp * MERGE_ROWS + (threadIdx.x >> 5);
    const int prow = slice * SLICE_ROWS + pl;
    if (prow >= npk) return;
    const int tl = prow / a.G;
    const int t = t_lo + tl, h = g * a.G + (prow - tl * a.G);
    const float NEG_INF = -__builtin_inff();
    float2 ml[SPLIT_MAX];
    float4 po[SPLIT_MAX];
#pragma unroll
    for (int sp = 0; sp < SPLIT_MAX; ++sp) {
        const long long pu = split_part(pidx, a.slices, slice, a.nsplit, sp < a.nsplit ? sp : 0);
        ml[sp] = sp < a.nsplit ? *(const float2*)(a.part_ml + (pu * SLICE_ROWS + pl) * 2) : make_float2(NEG_INF, 0.f);
        po[sp] = *(const float4*)(a.part_o + (pu * SLICE_ROWS + pl) * D + 4 * c);
    }
    float M = NEG_INF;
#pragma unroll
    for (int sp = 0; sp < SPLIT_MAX; ++sp) M = fmaxf(M, ml[sp].x);
    float L = 0.f;
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int sp = 0; sp < SPLIT_MAX; ++sp) {
        // an empty part, or no key of this row in it, weighs nothing
        const float w = ml[sp].x == NEG_INF ? 0.f : __builtin_amdgcn_exp2f(ml[sp].x - M);
        L += w * ml[sp].y;
        acc.x += w * po[sp].x; acc.y += w * po[sp].y; acc.z += w * po[sp].z; acc.w += w * po[sp].w;
    }
    const float inv = 1.f / L;
    if (a.o_f32) {
        float* op = (float*)a.o + a.oa.off(b, s, t, h) + 4 * c;
        *(float4*)op = make_float4(acc.x * inv, acc.y * inv, acc.z * inv, acc.w * inv);
    } else {
        __bf16* op = (__bf16*)a.o + a.oa.off(b, s, t, h) + 4 * c;
        uint2 w2;
        w2.x = pk_bf16(acc.x * inv, acc.y * inv);
        w2.y = pk_bf16(acc.z * inv, acc.w * inv);
        *(uint2*)op = w2;
    }
    if (a.lse && c == 0) a.lse[a.la.off(b, s, t, h)] = (M + __log2f(L)) * LN2;
}

template <int BLK, int NW, typename Geo>
static void attn_launch(const Geo& geo, const AttnArgs& a, int fp8, hipStream_t st) {
    AttnArgs b2 = a;
    b2.slices = attn_slices(a.G, BLK);
    const int units = cdiv(a.rows, 8) * 8 * b2.slices;
    // contiguous K/V come with the fixed geometry, the paged cache with the
    // sequence table (the entry points pair them so)
    constexpr bool PG = Geo::PAGED_KV;
    if constexpr (!PG) {
        if (a.nsplit > 1 && !a.dense) {
            // a grid too small for the chip: each row's tiles in nsplit parts, then the merge
            if (fp8) attn_tile_kernel<BLK, true, PG, Geo, NW, true><<<units * a.nsplit, NW * 64, 0, st>>>(geo, b2);
            else attn_tile_kernel<BLK, false, PG, Geo, NW, true><<<units * a.nsplit, NW * 64, 0, st>>>(geo, b2);
            split_merge_kernel<Geo><<<a.rows * b2.slices * (SLICE_ROWS / MERGE_ROWS), 256, 0, st>>>(geo, b2, BLK);
            return;
        }
    }
    if (fp8) attn_tile_kernel<BLK, true, PG, Geo, NW, false><<<units, NW * 64, 0, st>>>(geo, b2);
    else attn_tile_kernel<BLK, false, PG, Geo, NW, false><<<units, NW * 64, 0, st>>>(geo, b2);
}

// The launched shape is NW = 8 (two wavefronts per SIMD, 32 rows each). The
// template also builds NW = 4 (one wavefront per SIMD, 64 rows), but ROCm
// 7.2 allocates that shape's MFMA accumulators in VGPRs and spills 55-210
// VGPRs (plus hundreds of SGPRs) at 512 registers, so it is not launched.
constexpr int ATTN_WAVES = 8;

template <typename Geo>
static hipError_t attn_dispatch(const Geo& geo, const AttnArgs& a, int blk, int fp8, hipStream_t st) {
    if (blk == 128) attn_launch<128, ATTN_WAVES>(geo, a, fp8, st);
    else attn_launch<64, ATTN_WAVES>(geo, a, fp8, st);
    return hipGetLastError();
}

hipError_t launch_attn(const GeoFixed* gf, const GeoTable* gt, const AttnArgs& a, int blk,
                       int fp8, int paged, hipStream_t st) {
    if (a.rows == 0) return hipSuccess;
    if (paged != (gf ? 0 : 1)) return hipErrorInvalidValue;
    return gf ? attn_dispatch(*gf, a, blk, fp8, st) : attn_dispatch(*gt, a, blk, fp8, st);
}

}  // namespace fp
