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
//  * 8 wavefronts x 32 packed query rows. S^T = K Q^T and O^T = V^T P^T on
//    MFMA (bf16: 32x32x16; fp8: the scaled 32x32x64 f8f6f4 form with unit
//    scales), so each lane owns one query row: row max and row sum are
//    lane-local plus one exchange with lane ^ 32, and the accumulator
//    rescale is a per-lane scalar.
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
#include "fp_internal.h"

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

constexpr float LN2 = 0.6931471805599453f;

// swap bits 2 and 3 of a key index
__device__ __forceinline__ int vt_slot(int key) {
    return (key & ~0xC) | ((key >> 1) & 4) | ((key << 1) & 8);
}

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

// Online-softmax update for one tile held as S^T accumulators (log2 domain).
// Element value s maps to logit s * f + bias; masked elements are -inf. The
// probabilities are left in sacc multiplied by 2^lw (the PV operand scale);
// lsum accumulates them without it.
template <int NKB, int LAZY = 0>
__device__ __forceinline__ void online_update(f32x16 (&sacc)[NKB], float f, float bias, float lw,
                                              float& m, float& lsum, f32x16 (&oacc)[4]) {
    const float NEG_INF = -__builtin_inff();
    float mx = NEG_INF;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int v = 0; v < 16; ++v) mx = fmaxf(mx, sacc[kb][v]);
    mx = fmaxf(mx, other_half(mx));
    const float mcand = fmaxf(m, mx * f + bias);
    // Lazy rescale: keep the running reference m while the tile maximum stays
    // within 2^LAZY of it (probabilities then reach at most 2^LAZY, harmless
    // in fp32 sums and bf16 P); rescale only when some lane of the wave needs to.
    // LAZY = 0 rescales whenever the maximum grows; when it does not, the
    // factor would be exactly 1, so skipping it changes no bit.
    const bool need = mcand > m + (float)LAZY;
    if (__builtin_amdgcn_ballot_w64(need) != 0ull) {
        const float mnew = need ? mcand : m;
        const float alpha = __builtin_amdgcn_exp2f(m - (mnew == NEG_INF ? 0.f : mnew));
        lsum *= alpha;
#pragma unroll
        for (int db = 0; db < 4; ++db)
#pragma unroll
            for (int v = 0; v < 16; ++v) oacc[db][v] *= alpha;
        m = mnew;
    }
    const float muse = m == NEG_INF ? 0.f : m;
    const float nb = bias - muse + lw;
    float ts = 0.f;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            const float p = __builtin_amdgcn_exp2f(fmaf(sacc[kb][v], f, nb));
            sacc[kb][v] = p;
            ts += p;
        }
    lsum += lw == 0.f ? ts : ts * __builtin_amdgcn_exp2f(-lw);
}

// Bits b of a 32-column word starting at column c0 with lo <= c0 + b <= hi.
__device__ __forceinline__ uint32_t range_bits(int c0, int lo, int hi) {
    const int a = max(lo - c0, 0), z = min(hi - c0, 31);
    if (a > z) return 0u;
    return (0xFFFFFFFFu >> (31 - z)) & (0xFFFFFFFFu << a);
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
// Tile layouts in LDS (128 dims per row; rows padded, not XOR-swizzled, so
// every operand address is lane_base + immediate and no per-lane address
// table has to stay live in registers):
//   bf16 K rows every 272 bytes: the QK^T operand read (16 lanes = 16 rows
//     at one 16-byte chunk) lands on 16 distinct 4-bank groups;
//   bf16 V rows every 320 bytes: a transpose read covers 8 rows x 64 bytes,
//     served 32 lanes (4 rows) at a time; a stride of 64 bytes mod 256 puts
//     those rows on disjoint banks (measured: no conflicts, half the LDS
//     cycles of a 288-byte stride);
//   fp8 K rows every 144 bytes (16 mod 256, same argument as bf16 K);
//   fp8 V rows every 160 bytes, keys permuted inside each 64-key step (bits 2
//     and 3 swapped) so that each 32-lane half of a transpose read covers 8
//     consecutive rows x 32 bytes, which a stride of 40 dwords puts on 8
//     disjoint 8-bank groups.
// The summary tiles always use the bf16 layouts.
// ---------------------------------------------------------------------------
constexpr int KSTR = 272;
constexpr int VSTR = 320;
constexpr int KSTR8 = 144;
constexpr int VSTR8 = 160;

// Direct global->LDS loads of one tile: each wavefront instruction fills
// 1 KiB of LDS (lane l -> bytes 16 l .. 16 l + 15), so a lane works out which
// (row, chunk) its 16 bytes belong to; lanes that land on row padding stay
// inactive. LDS row r holds key r (PERM: key vt_slot(r)); rows past the
// sequence repeat its last key. ESZ = bytes per element.

// Lane byte offsets (relative to the tile's first key row) of the pieces
// this lane loads, for contiguous K/V; computed once per workgroup. Unsigned
// 32-bit offsets from a uniform base let each load use the scalar-base
// addressing form, so only one register per piece stays live.
template <int STR, int BLK, int ESZ, bool PERM>
struct TileOffs {
    static constexpr int PIECES = BLK * STR / 1024;
    static constexpr int NP = (PIECES + 7) / 8;
    static constexpr uint32_t PAD = 0xFFFFFFFFu;     // lane lands on row padding
    uint32_t off[NP];
    __device__ __forceinline__ void init(long long tok_stride, int wave, int lane) {
#pragma unroll
        for (int k = 0; k < NP; ++k) {
            const int pb = (k * 8 + wave) * 1024 + lane * 16;
            const int row = pb / STR;
            const int ch = (pb - row * STR) >> 4;
            const int key = PERM ? vt_slot(row) : row;
            off[k] = ch < 8 * ESZ ? (uint32_t)(key * tok_stride * ESZ + ch * 16) : PAD;
        }
    }
    // full tile (every row inside the sequence): one uniform base per tile
    __device__ __forceinline__ void issue(const uint8_t* tile_base, lds_u8* buf, int wave) const {
#pragma unroll
        for (int k = 0; k < NP; ++k) {
            const int t = k * 8 + wave;
            if (t < PIECES && off[k] != PAD)
                __builtin_amdgcn_global_load_lds((const void*)(tile_base + off[k]),
                                                 (lds_void*)(buf + t * 1024), 16, 0, 0);
        }
    }
    // Paged K/V: a tile's key `key` lies in page slot key >> lshift of the
    // tile (lshift = log2 min(page, BLK)) at in-page row key & (2^lshift - 1).
    // off packs that in-page byte offset (low 24 bits) with the slot.
    __device__ __forceinline__ void init_paged(long long tok_stride, int lshift, int wave, int lane) {
#pragma unroll
        for (int k = 0; k < NP; ++k) {
            const int pb = (k * 8 + wave) * 1024 + lane * 16;
            const int row = pb / STR;
            const int ch = (pb - row * STR) >> 4;
            const int key = PERM ? vt_slot(row) : row;
            const uint32_t inpage = (uint32_t)((key & ((1 << lshift) - 1)) * tok_stride * ESZ + ch * 16);
            off[k] = ch < 8 * ESZ ? (inpage | ((uint32_t)(key >> lshift) << 24)) : PAD;
        }
    }
    // Full paged tile, in two phases: read_pages looks up every piece's page
    // id first (pages = the tile's first slot in the staged list), then
    // issue_paged issues the loads (base = the uniform part: head and the
    // tile's in-page start). Reading LDS after some of the tile's loads are
    // in flight would make the compiler drain them (it cannot tell the page
    // list from the buffers being filled), so no LDS read may follow a load.
    __device__ __forceinline__ void read_pages(const lds_int* pages, int wave, int (&pg)[NP]) const {
#pragma unroll
        for (int k = 0; k < NP; ++k) {
            const int t = k * 8 + wave;
            pg[k] = (t < PIECES && off[k] != PAD) ? pages[off[k] >> 24] : 0;
        }
    }
    __device__ __forceinline__ void issue_paged(const uint8_t* base, const int (&pg)[NP],
                                                unsigned long long page_bytes, lds_u8* buf, int wave) const {
#pragma unroll
        for (int k = 0; k < NP; ++k) {
            const int t = k * 8 + wave;
            if (t < PIECES && off[k] != PAD)
                __builtin_amdgcn_global_load_lds(
                    (const void*)(base + (unsigned long long)pg[k] * page_bytes + (off[k] & 0xFFFFFFu)),
                    (lds_void*)(buf + t * 1024), 16, 0, 0);
        }
    }
};

// Generic tile addresses (ragged tiles, or paged tiles whose page list is not
// staged): every piece's source is computed before any load is issued, for
// the same reason as above (a paged lookup is a memory read).
template <int STR, int BLK, int ESZ, bool PERM, bool PAGED>
struct TileSrcs {
    static constexpr int PIECES = BLK * STR / 1024;
    static constexpr int NP = (PIECES + 7) / 8;
    const uint8_t* src[NP];
    __device__ __forceinline__ void compute(const uint8_t* base, const KVAddr& ka, int b, int L, int g, int j,
                                            int wave, int lane, const lds_int* pages) {
        asm volatile("" : "+v"(lane));   // recompute addresses per call, keep none live
        const int rmax = L - 1 - j * BLK;
#pragma unroll
        for (int k = 0; k < NP; ++k) {
            const int t = k * 8 + wave;
            const int pb = t * 1024 + lane * 16;
            const int row = pb / STR;
            const int ch = (pb - row * STR) >> 4;
            const int key = PERM ? vt_slot(row) : row;
            const int sk = j * BLK + min(key, rmax);
            src[k] = nullptr;
            if (t < PIECES && ch < 8 * ESZ) {
                // paged: the sequence's page ids staged in LDS when they fit, else the block table
                const long long off = PAGED && pages ? ka.off_page(pages[sk >> ka.page_shift], sk, g)
                                                     : ka.template off<PAGED>(b, sk, g);
                src[k] = base + off * ESZ + ch * 16;
            }
        }
    }
    __device__ __forceinline__ void issue(lds_u8* buf, int wave) const {
#pragma unroll
        for (int k = 0; k < NP; ++k) {
            const int t = k * 8 + wave;
            if (t < PIECES && src[k] != nullptr)
                __builtin_amdgcn_global_load_lds((const void*)src[k], (lds_void*)(buf + t * 1024), 16, 0, 0);
        }
    }
};

template <int BLK, bool FP8>
struct KVOffs {
    static constexpr int ESZ = FP8 ? 1 : 2;
    TileOffs<FP8 ? KSTR8 : KSTR, BLK, ESZ, false> k;
    TileOffs<FP8 ? VSTR8 : VSTR, BLK, ESZ, FP8> v;
    static constexpr int NPK = decltype(k)::NP, NPV = decltype(v)::NP;
};

template <int BLK, bool FP8, bool PAGED>
__device__ __forceinline__ void issue_kv(const AttnArgs& a, int b, int L, int g, int j,
                                         lds_u8* kbuf, lds_u8* vbuf, int wave, int lane,
                                         const KVOffs<BLK, FP8>& o, const lds_int* pages) {
    constexpr int ESZ = FP8 ? 1 : 2;
    if (PAGED && pages && a.paged_fast && (j + 1) * BLK <= L) {
        const int sh = a.ka.page_shift;
        const long long ub = (long long)((j * BLK) & ((1 << sh) - 1)) * a.ka.st + (long long)g * a.ka.sh;
        const lds_int* pt = pages + ((j * BLK) >> sh);
        int pgk[KVOffs<BLK, FP8>::NPK], pgv[KVOffs<BLK, FP8>::NPV];
        o.k.read_pages(pt, wave, pgk);
        o.v.read_pages(pt, wave, pgv);
        __builtin_amdgcn_sched_barrier(0);
        o.k.issue_paged((const uint8_t*)a.k + ub * ESZ, pgk, (unsigned long long)a.ka.spage * ESZ, kbuf, wave);
        o.v.issue_paged((const uint8_t*)a.v + ub * ESZ, pgv, (unsigned long long)a.va.spage * ESZ, vbuf, wave);
        return;
    }
    if (!PAGED && (j + 1) * BLK <= L) {
        const long long k0 = a.ka.template off<false>(b, j * BLK, g) * ESZ;
        const long long v0 = a.va.template off<false>(b, j * BLK, g) * ESZ;
        o.k.issue((const uint8_t*)a.k + k0, kbuf, wave);
        o.v.issue((const uint8_t*)a.v + v0, vbuf, wave);
        return;
    }
    TileSrcs<FP8 ? KSTR8 : KSTR, BLK, ESZ, false, PAGED> ks;
    TileSrcs<FP8 ? VSTR8 : VSTR, BLK, ESZ, FP8, PAGED> vs;
    ks.compute((const uint8_t*)a.k, a.ka, b, L, g, j, wave, lane, pages);
    vs.compute((const uint8_t*)a.v, a.va, b, L, g, j, wave, lane, pages);
    __builtin_amdgcn_sched_barrier(0);
    ks.issue(kbuf, wave);
    vs.issue(vbuf, wave);
}

// bf16 S^T for key blocks kb0 .. kb0 + NB - 1 (32 keys each) of the tile.
// DORD 0: step ks covers dims 16 ks + 8 lh .. +8; DORD 1: dims 64 (ks / 4) +
// 32 lh + 8 (ks % 4) .. +8 (the fp8 query fragment's order).
template <int NB, int DORD>
__device__ __forceinline__ void qk_pad(const lds_u8* kt, const bf16x8 (&qf)[8], int n, int lh, int kb0,
                                       f32x16 (&sacc)[NB], bool accumulate) {
    if (!accumulate) {
#pragma unroll
        for (int kb = 0; kb < NB; ++kb)
#pragma unroll
            for (int v = 0; v < 16; ++v) sacc[kb][v] = 0.f;
    }
#pragma unroll
    for (int ks = 0; ks < 8; ++ks)
#pragma unroll
        for (int kb = 0; kb < NB; ++kb) {
            const int d0 = DORD ? 64 * (ks >> 2) + 32 * lh + 8 * (ks & 3) : 16 * ks + 8 * lh;
            const bf16x8 aop = *(const lds_bf16x8*)(kt + ((kb0 + kb) * 32 + n) * KSTR + d0 * 2);
            sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aop, qf[ks], sacc[kb], 0, 0, 0);
        }
}

// bf16 O^T += V^T P^T: A operand = V^T fragment gathered by two transpose
// reads (16-lane group: lane 4e + r addresses V[k0 + e][d0 + 4r .. +4], lane
// i receives V[k0 + e][d0 + i] for e = 0..3); B operand = P from registers.
template <int NB>
__device__ __forceinline__ void pv_tr(const f32x16 (&sacc)[NB], const lds_u8* vt, int lane, int kb0,
                                      f32x16 (&oacc)[4]) {
    const int jj = lane & 15, q = lane >> 4;
    const int rsub = 4 * (q >> 1) + (jj >> 2);
    const int dsub = 16 * (q & 1) + 4 * (jj & 3);
#pragma unroll
    for (int kb = 0; kb < NB; ++kb)
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) {
            bf16x8 bop;
#pragma unroll
            for (int e = 0; e < 8; ++e) bop[e] = (__bf16)sacc[kb][8 * s2 + e];
#pragma unroll
            for (int db = 0; db < 4; ++db) {
                s16x4 h[2];
#pragma unroll
                for (int aa = 0; aa < 2; ++aa) {
                    const int row = (kb0 + kb) * 32 + 16 * s2 + 8 * aa + rsub;
                    const int d = 32 * db + dsub;
                    h[aa] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(vt + row * VSTR + d * 2));
                }
                const s16x4 h0 = h[0], h1 = h[1];
                typedef short s16x8 __attribute__((ext_vector_type(8)));
                const s16x8 cat = {h0[0], h0[1], h0[2], h0[3], h1[0], h1[1], h1[2], h1[3]};
                const bf16x8 aop = __builtin_bit_cast(bf16x8, cat);
                oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aop, bop, oacc[db], 0, 0, 0);
            }
        }
}

// fp8 S^T for key blocks kb0 .. kb0 + NB - 1: A = K rows (32 bytes per lane
// per 64-dim step, dims 64 ks + 32 lh ..), B = the query codes.
template <int NB>
__device__ __forceinline__ void qk_f8(const lds_u8* kt, const i32x8 (&qf8)[2], int n, int lh, int kb0,
                                      f32x16 (&sacc)[NB]) {
#pragma unroll
    for (int kb = 0; kb < NB; ++kb)
#pragma unroll
        for (int v = 0; v < 16; ++v) sacc[kb][v] = 0.f;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int kb = 0; kb < NB; ++kb) {
            const lds_u8* ap = kt + ((kb0 + kb) * 32 + n) * KSTR8 + ks * 64 + lh * 32;
            const u32x4 w0 = *(const lds_u32x4*)ap, w1 = *(const lds_u32x4*)(ap + 16);
            i32x8 aop;
            aop[0] = w0[0]; aop[1] = w0[1]; aop[2] = w0[2]; aop[3] = w0[3];
            aop[4] = w1[0]; aop[5] = w1[1]; aop[6] = w1[2]; aop[7] = w1[3];
            sacc[kb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(aop, qf8[ks], sacc[kb], 0, 0, 0, 127, 0,
                                                                      127);
        }
}

// fp8 O^T += V^T P^T over the 64-key step s2 (accumulators sacc[0], sacc[1]).
// B-lane (n, lh) byte e = 16 kbit + v holds P of key 32 kbit + 8 (v / 4) +
// 4 lh + v % 4. Transpose read c (16-lane group: lane i receives byte i % 8
// of the 8 bytes addressed by lane 2 e' + i / 8, e' = 0..7) gives A bytes
// 8c .. 8c + 7; with the keys stored at LDS row vt_slot(key), the 8 rows a
// lane half needs are the consecutive rows 16 c + 8 lh + e'.
__device__ __forceinline__ void pv_f8(const f32x16 (&sacc)[2], const lds_u8* vt, int lane, int s2,
                                      f32x16 (&oacc)[4]) {
    i32x8 bop;
#pragma unroll
    for (int kbit = 0; kbit < 2; ++kbit)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4)
            bop[4 * kbit + q4] = (int)pk_fp8x4(sacc[kbit][4 * q4], sacc[kbit][4 * q4 + 1], sacc[kbit][4 * q4 + 2],
                                               sacc[kbit][4 * q4 + 3]);
    const int a = lane & 15, half = (lane >> 4) & 1, lh = lane >> 5;
    const lds_u8* base = vt + (s2 * 64 + 8 * lh + (a >> 1)) * VSTR8 + 16 * half + 8 * (a & 1);
#pragma unroll
    for (int db = 0; db < 4; ++db) {
        i32x8 aop;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const i32x2 r = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2*)(base + 16 * c * VSTR8 + db * 32));
            aop[2 * c] = r[0];
            aop[2 * c + 1] = r[1];
        }
        oacc[db] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(aop, bop, oacc[db], 0, 0, 0, 127, 0, 127);
    }
}

// Summary sub-tile m covers pooled columns [SUMC m, SUMC m + SUMC) (SUMC =
// BLK / 2): its K tile holds the bf16 hi parts of those pooled keys in rows
// 0 .. SUMC-1 and the lo parts in rows SUMC .. BLK-1, so one ordinary tile
// load brings both, and the two halves of QK^T accumulate into one logit.
template <int BLK>
__device__ __forceinline__ void issue_summary(const AttnArgs& a, const SeqDesc& s, int g, int m,
                                              lds_u8* kbuf, lds_u8* vbuf, int wave, int lane) {
    constexpr int SUMC = BLK / 2;
    // recompute the per-lane piece addresses here instead of keeping them
    // live across the tile loop (registers are the scarce resource)
    asm volatile("" : "+v"(lane));
#pragma unroll
    for (int w = 0; w < 2; ++w) {
        constexpr int KP = BLK * KSTR / 1024, VP = SUMC * VSTR / 1024;
        const int STR = w == 0 ? KSTR : VSTR;
        const int PIECES = w == 0 ? KP : VP;
        lds_u8* buf = w == 0 ? kbuf : vbuf;
#pragma unroll
        for (int t0 = 0; t0 < (w == 0 ? KP : VP); t0 += 8) {
            const int t = t0 + wave;
            if (t < PIECES) {
                const int pb = t * 1024 + lane * 16;
                const int row = pb / STR;
                const int ch = (pb - row * STR) >> 4;
                const int part = row >= SUMC;                       // 0 hi / 1 lo (K rows)
                if (ch >= 16) continue;
                const int jp = min(SUMC * m + row - part * SUMC, s.nbk - 1);
                const long long pr = kbar_row(s, a.Hkv, g, jp) * D + ch * 8;
                const __bf16* src = w == 0 ? (part ? a.kbar_lo : a.kbar_hi) + pr : a.vbar_bf + pr;
                __builtin_amdgcn_global_load_lds((const void*)src, (lds_void*)(buf + t * 1024), 16, 0, 0);
            }
        }
    }
}

// fp8 tile scales (one per 128 keys) as vector loads: the value is consumed a
// tile later, after the barrier's vector-memory wait, so it never stalls
__device__ __forceinline__ float load_scale(const float* p, long long idx) {
    int z = 0;
    asm volatile("" : "+v"(z));
    return p[idx + z];
}

template <int BLK, bool FP8, bool PAGED, typename Geo>
__global__ __launch_bounds__(512, 1) void attn_tile_kernel(Geo geo, AttnArgs a) {
    constexpr int NKB = BLK / 32;
    constexpr int SB = NKB / 2;                     // 32-column blocks per summary sub-tile
    constexpr int SUMC = BLK / 2;
    constexpr int KTILE = BLK * KSTR;               // fits an fp8 K tile and a summary K tile
    constexpr int VTILE = FP8 ? (BLK * VSTR8 > SUMC * VSTR ? BLK * VSTR8 : SUMC * VSTR) : BLK * VSTR;
    constexpr int NONE = -0x7fffffff;
    // two distinct buffers per operand (not one indexed array), so the
    // compiler can tell the tile being read from the tile being loaded
    __shared__ __align__(1024) uint8_t kA_[KTILE];
    __shared__ __align__(1024) uint8_t kB_[KTILE];
    __shared__ __align__(1024) uint8_t vA_[VTILE];
    __shared__ __align__(1024) uint8_t vB_[VTILE];
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

    const int u = blockIdx.x;
    const int xcd = u & 7, k8 = u >> 3;
    const int pidx = 8 * (k8 / a.slices) + xcd;
    const int slice = k8 % a.slices;
    if (pidx >= a.rows) return;
    const int r = a.sched ? a.sched[pidx] : pidx;
    const int b = geo.seq_of_row(r);
    const SeqDesc s = geo.seq(b);
    const int rl = r - s.row0;
    const int g = rl / s.nq, il = rl % s.nq;
    const int i = s.i0 + il;
    const int t_lo = max(i * BLK, s.P), t_hi = min((i + 1) * BLK, s.L);
    const int G = a.G;
    const int npk = G * (t_hi - t_lo);
    if (slice * 256 >= npk) return;                  // uniform over the workgroup

    // The two wavefronts sharing a SIMD (w and w + 4) get different issue
    // priorities, so after each barrier one runs its MFMA phase ahead and the
    // other's softmax VALU work fills the MFMA pipe's shadow.
    if (wave < 4) __builtin_amdgcn_s_setprio(1);

    const int prow = slice * 256 + wave * 32 + n;
    const bool valid = prow < npk;
    const int tl = prow / G, hl = prow - tl * G;
    const int t = t_lo + tl;
    const int h = g * G + hl;

    const int rp0 = a.row_ptr[r], nnz = a.row_ptr[r + 1] - rp0;
    const int j0 = a.col_idx[rp0];
    KVOffs<BLK, FP8> kvo;
    if (!PAGED) {
        kvo.k.init(a.ka.st, wave, lane);
        kvo.v.init(a.va.st, wave, lane);
    } else if (a.paged_fast) {
        constexpr int LB = BLK == 128 ? 7 : 6;
        const int lshift = min(a.ka.page_shift, LB);
        kvo.k.init_paged(a.ka.st, lshift, wave, lane);
        kvo.v.init_paged(a.va.st, lshift, wave, lane);
    }
    issue_kv<BLK, FP8, PAGED>(a, b, s.L, g, j0, kA, vA, wave, lane, kvo, nullptr);
    // paged: stage the page ids for the later tiles (visible after the
    // barrier that follows the kept-bitmap build)
    const lds_int* pages = nullptr;
    if constexpr (PAGED) {
        const int npg = (s.L + (1 << a.ka.page_shift) - 1) >> a.ka.page_shift;
        if (npg <= PAGE_CAP) {
            const int* row = a.ka.table + (long long)b * a.ka.maxp;
            for (int p = tid; p < npg; p += 512) pages_sh[p] = row[p];
            pages = (const lds_int*)pages_sh;
        }
    }

    // Query fragment. bf16: lane (n, lh) holds q[t, h, 16 ks + 8 lh .. + 8];
    // fp8: the codes q[t, h, 64 ks + 32 lh .. + 32], widened to bf16 (exact)
    // in that order only when the summary tiles start.
    bf16x8 qf[8];
    i32x8 qf8[2];
    float f_row = a.scale_log2;
    if constexpr (FP8) {
        const uint8_t* qp = (const uint8_t*)a.q + (valid ? a.qa.off(b, s, t, h) : 0);
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            const uint4 w0 = valid ? *(const uint4*)(qp + ks * 64 + lh * 32) : make_uint4(0u, 0u, 0u, 0u);
            const uint4 w1 = valid ? *(const uint4*)(qp + ks * 64 + lh * 32 + 16) : make_uint4(0u, 0u, 0u, 0u);
            qf8[ks][0] = w0.x; qf8[ks][1] = w0.y; qf8[ks][2] = w0.z; qf8[ks][3] = w0.w;
            qf8[ks][4] = w1.x; qf8[ks][5] = w1.y; qf8[ks][6] = w1.z; qf8[ks][7] = w1.w;
        }
        if (valid) f_row *= a.qs.at(b, h, t);
    } else {
        const __bf16* qp = (const __bf16*)a.q + (valid ? a.qa.off(b, s, t, h) : 0);
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) {
            if (valid) qf[ks] = *(const bf16x8*)(qp + ks * 16 + lh * 8);
            else
#pragma unroll
                for (int e = 0; e < 8; ++e) qf[ks][e] = (__bf16)0.f;
        }
    }
    // fp8 tile scales of this row's (sequence, KV head): one per 128 keys
    const float* ksp = FP8 ? a.ks.p + (long long)b * a.ks.sb + (long long)g * a.ks.sh : nullptr;
    const float* vsp = FP8 ? a.vs.p + (long long)b * a.vs.sb + (long long)g * a.vs.sh : nullptr;
    float ksA = 1.f, vsA = 1.f, ksB = 1.f, vsB = 1.f;
    if constexpr (FP8) {
        ksA = load_scale(ksp, (j0 * BLK) >> 7);
        vsA = load_scale(vsp, (j0 * BLK) >> 7);
    }

    const int nw = (i >> 5) + 1;
    for (int w = tid; w < nw; w += 512) kept[w] = 0u;
    if (FP8 && tid == 0) svmax_sh = 0;
    __syncthreads();
    float svm = 0.f;
    for (int e = tid; e < nnz; e += 512) {
        const int j = a.col_idx[rp0 + e];
        atomicOr(&kept[j >> 5], 1u << (j & 31));
        if (FP8) svm = fmaxf(svm, vsp[(j * BLK) >> 7]);
    }
    if constexpr (FP8) {
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) svm = fmaxf(svm, __shfl_xor(svm, off, 64));
        if (lane == 0) atomicMax(&svmax_sh, __float_as_int(svm));   // non-negative floats order as ints
    }

    float m = NEG_INF, lsum = 0.f;
    f32x16 oacc[4];
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int v = 0; v < 16; ++v) oacc[db][v] = 0.f;
    const float lnb2 = (BLK == 128) ? 7.f : 6.f;    // log2 |block| of a pruned pseudo-token
    __syncthreads();                                  // tile 0 landed; kept bitmap complete
    // fp8: PV accumulates P 2^8 sv_j / svmax times the value codes (P <= 1:
    // no lazy rescale there), undone in the epilogue
    const float svmax = FP8 ? fmaxf(__int_as_float(svmax_sh), 1e-30f) : 1.f;
    const float lsvmax = FP8 ? __log2f(svmax) : 0.f;

    // Tile sequence: the kept blocks in column order (codes >= 0 are block
    // indices), then the summary sub-tiles that hold at least one pruned
    // column (code -1 - m for sub-tile m). The code of the next tile is known
    // before its loads are issued, so no vector-memory wait inside a tile's
    // compute drains the prefetch.
    auto next_summary = [&](int m0) -> int {
        if (a.no_correction) return NONE;             // ablation: no pseudo-tokens
        for (int mm = m0; mm * SUMC <= i - 1; ++mm) {
            const int c_lo = max(1, mm * SUMC), c_hi = min(i - 1, mm * SUMC + SUMC - 1);
            uint32_t anyw = 0u;
            for (int wd = c_lo >> 5; wd <= (c_hi >> 5); ++wd)
                anyw |= ~kept[wd] & range_bits(wd * 32, c_lo, c_hi);
            if (anyw) return -1 - mm;
        }
        return NONE;
    };
    // The next kept column comes from the LDS bitmap (no global-memory
    // round trip between tiles).
    auto next_code = [&](int code) -> int {
        if (code >= 0) {
            int wd = (code + 1) >> 5;
            uint32_t w = code + 1 <= i ? kept[wd] & (~0u << ((code + 1) & 31)) : 0u;
            while (w == 0u && wd < (i >> 5)) w = kept[++wd];
            w = __builtin_amdgcn_readfirstlane(w);
            wd = __builtin_amdgcn_readfirstlane(wd);
            if (w != 0u) return wd * 32 + __builtin_ctz(w);
            return next_summary(0);
        }
        return next_summary(-code);
    };
    auto issue = [&](int code, lds_u8* kb, lds_u8* vb, float& ksn, float& vsn) __attribute__((always_inline)) {
        if (code >= 0) {
            issue_kv<BLK, FP8, PAGED>(a, b, s.L, g, code, kb, vb, wave, lane, kvo, pages);
            if constexpr (FP8) {
                ksn = load_scale(ksp, (code * BLK) >> 7);
                vsn = load_scale(vsp, (code * BLK) >> 7);
            }
        } else {
            issue_summary<BLK>(a, s, g, -1 - code, kb, vb, wave, lane);
        }
    };
    auto mask_diag = [&](f32x16 (&sh)[2], int code, int hf) __attribute__((always_inline)) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int sk = code * BLK + (2 * hf + kb) * 32 + 8 * (v >> 2) + 4 * lh + (v & 3);
                sh[kb][v] = sk > t ? NEG_INF : sh[kb][v];
            }
    };
    // Exact tokens of kept block `code`, 64 keys at a time (32 S registers live).
    auto compute_kept = [&](int code, const lds_u8* kc, const lds_u8* vc, float ksj, float vsj)
                            __attribute__((always_inline)) {
        if constexpr (FP8) {
            const float f = f_row * ksj;
            const float lw = 8.f + __log2f(fmaxf(vsj, 1e-30f)) - lsvmax;
#pragma unroll
            for (int hf = 0; hf < NKB / 2; ++hf) {
                f32x16 sh[2];
                qk_f8<2>(kc, qf8, n, lh, 2 * hf, sh);
                if (code == i) mask_diag(sh, code, hf);
                online_update<2, 0>(sh, f, 0.f, lw, m, lsum, oacc);
                pv_f8(sh, vc, lane, hf, oacc);
            }
        } else {
#pragma unroll
            for (int hf = 0; hf < NKB / 2; ++hf) {
                f32x16 sh[2];
                qk_pad<2, 0>(kc, qf, n, lh, 2 * hf, sh, false);
                if (code == i) mask_diag(sh, code, hf);
                online_update<2, 8>(sh, f_row, 0.f, 0.f, m, lsum, oacc);
                pv_tr<2>(sh, vc, lane, 2 * hf, oacc);
            }
        }
    };
    // fp8: the pseudo-token weights join the accumulator in its 2^8 / svmax units
    const float lw_sum = FP8 ? 8.f - lsvmax : 0.f;
    // Pooled pseudo-tokens of summary sub-tile -1 - code: hi and lo halves of
    // QK^T accumulate into one logit per pooled column; pseudo-tokens of kept
    // or non-causal columns are masked from the LDS bitmap.
    auto compute_summary = [&](int code, const lds_u8* kc, const lds_u8* vc) __attribute__((always_inline)) {
        const int mm = -1 - code;
        f32x16 sh[SB];
        qk_pad<SB, FP8 ? 1 : 0>(kc, qf, n, lh, 0, sh, false);    // hi rows
        qk_pad<SB, FP8 ? 1 : 0>(kc, qf, n, lh, SB, sh, true);    // lo rows, same columns
#pragma unroll
        for (int kb = 0; kb < SB; ++kb) {
            const int c0 = mm * SUMC + kb * 32;
            const uint32_t pw = ~kept[min(c0 >> 5, MAX_NB / 32 - 1)] & range_bits(c0, 1, i - 1);
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int bit = 8 * (v >> 2) + 4 * lh + (v & 3);
                sh[kb][v] = ((pw >> bit) & 1u) ? sh[kb][v] : NEG_INF;
            }
        }
        online_update<SB, 8>(sh, f_row, lnb2, lw_sum, m, lsum, oacc);
        pv_tr<SB>(sh, vc, lane, 0, oacc);
    };

    // Kept phase. Buffers alternate A, B; the loop ends once the code of the
    // following tile is a summary code (already issued) or NONE (both < 0).
    int nxt, ca = j0;
    bool in_b;
    while (true) {
        const int cb = next_code(ca);
        if (cb != NONE) issue(cb, kB, vB, ksB, vsB);
        compute_kept(ca, kA, vA, ksA, vsA);
        __syncthreads();                              // next tile landed; A is free
        if (cb < 0) { nxt = cb; in_b = true; break; }
        const int cn = next_code(cb);
        if (cn != NONE) issue(cn, kA, vA, ksA, vsA);
        compute_kept(cb, kB, vB, ksB, vsB);
        __syncthreads();
        if (cn < 0) { nxt = cn; in_b = false; break; }
        ca = cn;
    }
    if constexpr (FP8) {
        // widen the query codes to bf16 (exact) in the fp8 fragment's dim order
        if (nxt != NONE) {
#pragma unroll
            for (int ks = 0; ks < 8; ++ks)
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const int byte = (ks & 3) * 8 + e;              // within the 32-byte half
                    const uint32_t w = (uint32_t)qf8[ks >> 2][byte >> 2];
                    qf[ks][e] = (__bf16)e4m3_val((w >> ((byte & 3) * 8)) & 0xFFu);
                }
        }
    }
    // Summary phase: realign so the loop below always starts on buffer A.
    if (in_b && nxt != NONE) {
        const int cn = next_summary(-nxt);
        if (cn != NONE) issue_summary<BLK>(a, s, g, -1 - cn, kA, vA, wave, lane);
        compute_summary(nxt, kB, vB);
        __syncthreads();
        nxt = cn;
    }
    while (nxt != NONE) {
        const int cb = next_summary(-nxt);
        if (cb != NONE) issue_summary<BLK>(a, s, g, -1 - cb, kB, vB, wave, lane);
        compute_summary(nxt, kA, vA);
        __syncthreads();
        if (cb == NONE) break;
        const int cn = next_summary(-cb);
        if (cn != NONE) issue_summary<BLK>(a, s, g, -1 - cn, kA, vA, wave, lane);
        compute_summary(cb, kB, vB);
        __syncthreads();
        nxt = cn;
    }

    // ---------------- epilogue ----------------
    const float ltot = lsum + other_half(lsum);
    if (!valid) return;
    const float inv = (FP8 ? svmax * 0.00390625f : 1.f) / ltot;
    if (a.o_f32) {
        float* op = (float*)a.o + a.oa.off(b, s, t, h);
#pragma unroll
        for (int db = 0; db < 4; ++db)
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4)
                *(float4*)(op + db * 32 + q4 * 8 + lh * 4) =
                    make_float4(oacc[db][4 * q4] * inv, oacc[db][4 * q4 + 1] * inv, oacc[db][4 * q4 + 2] * inv,
                                oacc[db][4 * q4 + 3] * inv);
    } else {
        __bf16* op = (__bf16*)a.o + a.oa.off(b, s, t, h);
#pragma unroll
        for (int db = 0; db < 4; ++db)
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
                uint2 w;
                w.x = pk_bf16(oacc[db][4 * q4] * inv, oacc[db][4 * q4 + 1] * inv);
                w.y = pk_bf16(oacc[db][4 * q4 + 2] * inv, oacc[db][4 * q4 + 3] * inv);
                *(uint2*)(op + db * 32 + q4 * 8 + lh * 4) = w;
            }
    }
    if (a.lse && lh == 0) a.lse[a.la.off(b, s, t, h)] = (m + __log2f(ltot)) * LN2;
}

// bf16 operands of the summary tiles: Kbar = hi + lo (two bf16 terms), Vbar.
__global__ __launch_bounds__(256) void summary_prep_kernel(const float* kbar, const float* vbar, __bf16* hi,
                                                           __bf16* lo, __bf16* vb, long long n4) {
    const long long e = (long long)blockIdx.x * 256 + threadIdx.x;
    if (e >= n4) return;
    const float4 k = ((const float4*)kbar)[e];
    const float4 v = ((const float4*)vbar)[e];
    uint2 h, l, w;
    h.x = pk_bf16(k.x, k.y);
    h.y = pk_bf16(k.z, k.w);
    l.x = pk_bf16(k.x - bf16_round(k.x), k.y - bf16_round(k.y));
    l.y = pk_bf16(k.z - bf16_round(k.z), k.w - bf16_round(k.w));
    w.x = pk_bf16(v.x, v.y);
    w.y = pk_bf16(v.z, v.w);
    ((uint2*)hi)[e] = h;
    ((uint2*)lo)[e] = l;
    ((uint2*)vb)[e] = w;
}

hipError_t launch_summary_prep(const float* kbar, const float* vbar, __bf16* hi, __bf16* lo, __bf16* vb,
                               long long nfloats, hipStream_t st) {
    const long long n4 = nfloats / 4;
    if (n4 == 0) return hipSuccess;
    summary_prep_kernel<<<(unsigned)((n4 + 255) / 256), 256, 0, st>>>(kbar, vbar, hi, lo, vb, n4);
    return hipGetLastError();
}

template <int BLK, typename Geo>
static void attn_launch(const Geo& geo, const AttnArgs& a, int fp8, int paged, hipStream_t st) {
    AttnArgs b2 = a;
    b2.slices = cdiv(a.G * BLK, 256);
    const int units = cdiv(a.rows, 8) * 8 * b2.slices;
    // contiguous K/V come with the fixed geometry, the paged cache with the
    // sequence table (the entry points pair them so)
    if constexpr (Geo::PAGED_KV) {
        if (fp8) attn_tile_kernel<BLK, true, true, Geo><<<units, 512, 0, st>>>(geo, b2);
        else attn_tile_kernel<BLK, false, true, Geo><<<units, 512, 0, st>>>(geo, b2);
    } else {
        if (fp8) attn_tile_kernel<BLK, true, false, Geo><<<units, 512, 0, st>>>(geo, b2);
        else attn_tile_kernel<BLK, false, false, Geo><<<units, 512, 0, st>>>(geo, b2);
    }
}

template <typename Geo>
static hipError_t attn_dispatch(const Geo& geo, const AttnArgs& a, int blk, int fp8, int paged,
                                hipStream_t st) {
    if (blk == 128) attn_launch<128>(geo, a, fp8, paged, st);
    else attn_launch<64>(geo, a, fp8, paged, st);
    return hipGetLastError();
}

hipError_t launch_attn(const GeoFixed* gf, const GeoTable* gt, const AttnArgs& a, int blk,
                       int fp8, int paged, hipStream_t st) {
    if (a.rows == 0) return hipSuccess;
    return gf ? attn_dispatch(*gf, a, blk, fp8, paged, st) : attn_dispatch(*gt, a, blk, fp8, paged, st);
}

}  // namespace fp
