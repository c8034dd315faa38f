// Max-based dynamic threshold (E3-E5) and compaction of the kept blocks into
// CSR lists plus a heavy-row-first schedule.
//
// The threshold keeps a key block when its estimate lies within tau of the
// query block's row maximum (lode.cx page, "How It Works"; aimodeling.com
// page, "From Prototype to Production"); with grouped-query attention the G
// query heads of a KV head share one list (the union over the heads), which
// is what lets the attention pass pack those heads into one tile (lode.cx
// page, PackGQA bullet). Sink and diagonal blocks are always kept.
//
// select_rows: one wavefront per row (b, g, i). Pass 1 reduces the G row
//   maxima, pass 2 forms R = max_h (S - M_h) per key block, tests it and
//   compacts the decisions with a 64-lane ballot into a bit row + count.
// scan_rows:   single workgroup exclusive scan of the counts -> row_ptr.
// expand_rows: one wavefront per row, ballot + lane-prefix popcount writes the
//   ascending column list at row_ptr.
// sort_*:      stable counting sort of the rows -> sched, over chunks of rows
//   (histograms, offsets, scatter; the bins span the counts up to the largest
//   one, which scan_rows records). The order is heavy-row-first inside
//   groups of consecutive (sequence, KV head) pairs whose K/V together stay
//   within a budget sized for the memory-side cache, groups in row order:
//   key = (group ascending, count descending), ties by row id.
#include "fp_internal.h"

namespace fp {

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
    return v;
}

template <typename Geo>
__global__ __launch_bounds__(256) void select_rows_kernel(Geo geo, SelectArgs a) {
    const int lane = threadIdx.x & 63;
    const int r = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (r >= a.rows) return;
    const int b = geo.seq_of_row(r);
    const SeqDesc s = geo.seq(b);
    const int rl = r - s.row0;
    const int g = rl / s.nq, il = rl % s.nq;
    const int i = s.i0 + il;
    const int G = a.Hq / a.Hkv;
    const float NEG_INF = -__builtin_inff();

    float M[MAX_G];
#pragma unroll
    for (int hh = 0; hh < MAX_G; ++hh) {
        M[hh] = NEG_INF;
        if (hh < G) {
            const float* row = a.scores + score_off(s, g * G + hh, il, 0);
            float m = NEG_INF;
            for (int j = lane; j <= i; j += 64) m = fmaxf(m, row[j]);
            M[hh] = wave_max(m);
        }
    }
    int count = 0;
    uint32_t* bits = a.bits + (long long)r * a.nbw;
    for (int jc = 0; jc <= i; jc += 64) {
        const int j = jc + lane;
        bool keep = false;
        if (j <= i) {
            float R = NEG_INF;
#pragma unroll
            for (int hh = 0; hh < MAX_G; ++hh)
                if (hh < G) R = fmaxf(R, a.scores[score_off(s, g * G + hh, il, j)] - M[hh]);
            keep = (R >= a.neg_tau) || j == 0 || j == i;
        }
        const unsigned long long bal = __ballot(keep);
        count += __popcll(bal);
        if (lane == 0) bits[jc >> 5] = (uint32_t)bal;
        if (lane == 1 && (jc >> 5) + 1 < a.nbw) bits[(jc >> 5) + 1] = (uint32_t)(bal >> 32);
    }
    if (lane == 0) {
        a.counts[r] = count;
        a.keys[r] = row_group(s, g, a.Hkv, a.grp_units, a.ngrp);
    }
}

// ---------------------------------------------------------------------------
// Fused E2-E5 (fixed shape): the scores of a row are computed from the pooled
// rows where they are needed and never written to HBM. One workgroup per
// (sequence, KV head, QB = 32 / G query blocks): its S columns are the QB x G
// (query block, query head) pairs, the rows are all key blocks, kept in LDS
// (32 x (nbk + 1) floats). Each of the 8 wavefronts takes every 8th 32-key
// tile and computes S^T = Kbar Qbar^T on v_mfma_f32_32x32x2_f32 with the
// query side in registers and the next tile's pooled keys loaded while the
// current one is multiplied; the dims are summed in the same order, pairing and scale as
// scores_kernel, so every S value -- and every decision -- is the one the
// unfused path makes. Then the row maxima (E3) per column, the group union
// (E4) and the threshold (E5) per query block, ballot-compacted into the
// same bit rows and counts select_rows_kernel writes.
// ---------------------------------------------------------------------------
constexpr int FUSED_WAVES = 8;

__global__ __launch_bounds__(FUSED_WAVES * 64) void select_fused_kernel(GeoFixed geo, SelectArgs a) {
    extern __shared__ __align__(16) float S_sh[];   // [FUSED_COLS][nbk + 1]
    __shared__ float M_sh[FUSED_COLS];
    typedef __attribute__((ext_vector_type(16))) float f32x16;
    const float NEG_INF = -__builtin_inff();
    const int G = a.Hq / a.Hkv;
    const int QB = FUSED_COLS / G;
    const int nb = geo.nb;
    const int ntq = cdiv(nb, QB);
    const int u = blockIdx.x;
    const int bg = u / ntq, qt = u % ntq;
    const int b = bg / a.Hkv, g = bg % a.Hkv;
    const SeqDesc s = geo.seq(b);
    const int il0 = qt * QB;
    const int nql = min(QB, s.nq - il0);
    const int cols = nql * G;
    const int imax = s.i0 + il0 + nql - 1;
    const int sst = nb + 1;                          // padded row stride of S_sh
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, n = lane & 31, lh = lane >> 5;

    // query side of the MFMA: column n = (query block n / G, head n % G);
    // step (pass p, t, component c) takes dim 32 p + 4 t + c from lanes 0-31
    // and dim 32 p + 16 + 4 t + c from lanes 32-63, as scores_kernel does
    float4 qv[4][4];
    {
        const bool ok = n < cols;
        const int ql = ok ? n / G : 0, hh = ok ? n % G : 0;
        const float* qr = a.qbar + qbar_row(s, a.Hq, g * G + hh, il0 + ql) * D;
#pragma unroll
        for (int p = 0; p < 4; ++p)
#pragma unroll
            for (int t = 0; t < 4; ++t)
                qv[p][t] = ok ? *(const float4*)(qr + 32 * p + 16 * lh + 4 * t) : make_float4(0.f, 0.f, 0.f, 0.f);
    }
    const int nkt = imax / 32 + 1;
    // pooled keys of key tile kt for this lane: row kt * 32 + n, the dims of qv
    auto load_tile = [&](int kt, float4 (&kv)[4][4]) {
        const int jrow = min(kt * 32 + n, s.nbk - 1);
        const float* kr = a.kbar + kbar_row(s, a.Hkv_pool, g / a.kv_div, jrow) * D;
#pragma unroll
        for (int p = 0; p < 4; ++p)
#pragma unroll
            for (int t = 0; t < 4; ++t) kv[p][t] = *(const float4*)(kr + 32 * p + 16 * lh + 4 * t);
    };
    float4 kn[4][4];
    if (wave < nkt) load_tile(wave, kn);
    for (int kt = wave; kt < nkt; kt += FUSED_WAVES) {
        float4 kv[4][4];
#pragma unroll
        for (int p = 0; p < 4; ++p)
#pragma unroll
            for (int t = 0; t < 4; ++t) kv[p][t] = kn[p][t];
        if (kt + FUSED_WAVES < nkt) load_tile(kt + FUSED_WAVES, kn);
        f32x16 acc;
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[v] = 0.f;
#pragma unroll
        for (int p = 0; p < 4; ++p)
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                acc = __builtin_amdgcn_mfma_f32_32x32x2f32(kv[p][t].x, qv[p][t].x, acc, 0, 0, 0);
                acc = __builtin_amdgcn_mfma_f32_32x32x2f32(kv[p][t].y, qv[p][t].y, acc, 0, 0, 0);
                acc = __builtin_amdgcn_mfma_f32_32x32x2f32(kv[p][t].z, qv[p][t].z, acc, 0, 0, 0);
                acc = __builtin_amdgcn_mfma_f32_32x32x2f32(kv[p][t].w, qv[p][t].w, acc, 0, 0, 0);
            }
        // accumulator: lane holds column n, key rows 8 (v / 4) + 4 lh + v % 4
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            const int j = kt * 32 + 8 * (v >> 2) + 4 * lh + (v & 3);
            if (j < nb) S_sh[n * sst + j] = acc[v] * a.scale;
        }
    }
    __syncthreads();
    // E3: row maximum of each column over its visible key blocks j <= i
    for (int c = wave; c < cols; c += FUSED_WAVES) {
        const int i = s.i0 + il0 + c / G;
        float m = NEG_INF;
        for (int j = lane; j <= i; j += 64) m = fmaxf(m, S_sh[c * sst + j]);
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
        if (lane == 0) M_sh[c] = m;
    }
    __syncthreads();
    // E4-E5 per query block: union over the group's heads, threshold, ballot
    for (int ql = wave; ql < nql; ql += FUSED_WAVES) {
        const int i = s.i0 + il0 + ql;
        const int r = s.row0 + g * s.nq + il0 + ql;
        uint32_t* bits = a.bits + (long long)r * a.nbw;
        int count = 0;
        for (int jc = 0; jc <= i; jc += 64) {
            const int j = jc + lane;
            bool keep = false;
            if (j <= i) {
                float R = NEG_INF;
                for (int hh = 0; hh < G; ++hh) R = fmaxf(R, S_sh[(ql * G + hh) * sst + j] - M_sh[ql * G + hh]);
                keep = (R >= a.neg_tau) || j == 0 || j == i;
            }
            const unsigned long long bal = __ballot(keep);
            count += __popcll(bal);
            if (lane == 0) bits[jc >> 5] = (uint32_t)bal;
            if (lane == 1 && (jc >> 5) + 1 < a.nbw) bits[(jc >> 5) + 1] = (uint32_t)(bal >> 32);
        }
        if (lane == 0) {
            a.counts[r] = count;
            a.keys[r] = row_group(s, g, a.Hkv, a.grp_units, a.ngrp);
        }
    }
}

// Exclusive scan of counts into row_ptr[0..rows]; one workgroup of 1024.
__global__ __launch_bounds__(1024) void scan_rows_kernel(SelectArgs a) {
    __shared__ int part[1024];
    const int tid = threadIdx.x;
    const int per = cdiv(a.rows, 1024);
    const int lo = min(tid * per, a.rows), hi = min(lo + per, a.rows);
    __shared__ int cmax;
    if (tid == 0) cmax = 0;
    int sum = 0, mx = 0;
    for (int r = lo; r < hi; ++r) {
        sum += a.counts[r];
        mx = max(mx, a.counts[r]);
    }
    part[tid] = sum;
    __syncthreads();
    atomicMax(&cmax, mx);
    for (int o = 1; o < 1024; o <<= 1) {           // Hillis-Steele inclusive scan
        const int v = tid >= o ? part[tid - o] : 0;
        __syncthreads();
        part[tid] += v;
        __syncthreads();
    }
    int run = part[tid] - sum;                      // exclusive prefix of this chunk
    if (tid == 0) {
        a.row_ptr[0] = 0;
        *a.maxc = cmax;                             // read by the schedule sort
    }
    for (int r = lo; r < hi; ++r) {
        run += a.counts[r];
        a.row_ptr[r + 1] = run;
    }
}

template <typename Geo>
__global__ __launch_bounds__(256) void expand_rows_kernel(Geo geo, SelectArgs a) {
    const int lane = threadIdx.x & 63;
    const int r = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (r >= a.rows) return;
    const int b = geo.seq_of_row(r);
    const SeqDesc s = geo.seq(b);
    const int il = (r - s.row0) % s.nq;
    const int i = s.i0 + il;
    const uint32_t* bits = a.bits + (long long)r * a.nbw;
    int pos = a.row_ptr[r];
    for (int jc = 0; jc <= i; jc += 64) {
        const uint32_t lo = bits[jc >> 5];
        const uint32_t hi = (jc + 32 <= i) ? bits[(jc >> 5) + 1] : 0u;
        const unsigned long long m = ((unsigned long long)hi << 32) | lo;
        const unsigned long long below = lane ? (m & ((~0ull) >> (64 - lane))) : 0ull;
        if ((m >> lane) & 1ull) a.col_idx[pos + __popcll(below)] = jc + lane;
        pos += __popcll(m);
    }
}

// Stable counting sort of the rows by key (group-major, then kept count),
// descending, ties by row id ascending, in three passes over chunks of
// SORT_CHUNK consecutive rows:
//   sort_hist:    per chunk, a histogram of the keys (LDS atomics) -> hist[c][k];
//   sort_offsets: per key k (descending) and chunk c (ascending), the first
//                 position of chunk c's rows with key k, written over hist;
//   sort_scatter: per chunk, each row's rank among the equal keys before it
//                 in the chunk, added to that position -> sched.
// Sort key of row r: group-major (group 0 largest), then the kept count; the
// histograms hold ngrp * (largest count + 1) bins.
__device__ __forceinline__ int sort_key(const SelectArgs& a, int r, int nc) {
    return (a.ngrp - 1 - a.keys[r]) * nc + a.counts[r];
}

__global__ __launch_bounds__(SORT_CHUNK) void sort_hist_kernel(SelectArgs a) {
    extern __shared__ __align__(16) int hsh[];   // [nbin]
    const int nc = *a.maxc + 1, nbin = a.ngrp * nc, c = blockIdx.x, tid = threadIdx.x;
    for (int k = tid; k < nbin; k += SORT_CHUNK) hsh[k] = 0;
    __syncthreads();
    const int r = c * SORT_CHUNK + tid;
    if (r < a.rows) atomicAdd(&hsh[sort_key(a, r, nc)], 1);
    __syncthreads();
    int* out = a.hist + (long long)c * nbin;
    for (int k = tid; k < nbin; k += SORT_CHUNK) out[k] = hsh[k];
}

__global__ __launch_bounds__(1024) void sort_offsets_kernel(SelectArgs a) {
    __shared__ int part[1024];
    const int nbin = a.ngrp * (*a.maxc + 1), nch = cdiv(a.rows, SORT_CHUNK), tid = threadIdx.x;
    const int per = cdiv(nbin, 1024);
    const int lo = min(tid * per, nbin), hi = min(lo + per, nbin);
    int sum = 0;                                   // rows with a key in [lo, hi)
    for (int k = lo; k < hi; ++k)
        for (int c = 0; c < nch; ++c) sum += a.hist[(long long)c * nbin + k];
    part[tid] = sum;
    __syncthreads();
    for (int o = 1; o < 1024; o <<= 1) {           // inclusive suffix scan over threads
        const int v = tid + o < 1024 ? part[tid + o] : 0;
        __syncthreads();
        part[tid] += v;
        __syncthreads();
    }
    int run = part[tid] - sum;                     // rows with a larger key than hi - 1
    for (int k = hi - 1; k >= lo; --k)
        for (int c = 0; c < nch; ++c) {
            int* h = a.hist + (long long)c * nbin + k;
            const int n = *h;
            *h = run;
            run += n;
        }
}

__global__ __launch_bounds__(SORT_CHUNK) void sort_scatter_kernel(SelectArgs a) {
    __shared__ __align__(16) int keys[SORT_CHUNK];
    const int nc = *a.maxc + 1, nbin = a.ngrp * nc, c = blockIdx.x, tid = threadIdx.x;
    const int r = c * SORT_CHUNK + tid;
    const int key = r < a.rows ? sort_key(a, r, nc) : -1;
    keys[tid] = key;
    __syncthreads();
    if (key < 0) return;
    int rank = 0;                                  // equal keys earlier in the chunk
    const int4* k4 = (const int4*)keys;
    const int n4 = tid >> 2;
#pragma unroll 8
    for (int t4 = 0; t4 < n4; ++t4) {
        const int4 w = k4[t4];
        rank += (w.x == key) + (w.y == key) + (w.z == key) + (w.w == key);
    }
    for (int t = n4 * 4; t < tid; ++t) rank += keys[t] == key;
    a.sched[a.hist[(long long)c * nbin + key] + rank] = r;
}

template <typename Geo>
static hipError_t select_dispatch(const Geo& geo, const SelectArgs& a, hipStream_t st, bool fused = false) {
    const int wg = cdiv(a.rows, 4);
    if (!fused) select_rows_kernel<Geo><<<wg, 256, 0, st>>>(geo, a);
    scan_rows_kernel<<<1, 1024, 0, st>>>(a);
    expand_rows_kernel<Geo><<<wg, 256, 0, st>>>(geo, a);
    if (a.sched) {
        const int nch = cdiv(a.rows, SORT_CHUNK);
        const size_t shm = (size_t)a.ngrp * (a.max_nbk + 1) * sizeof(int);
        if (shm > 65536) {
            hipError_t e = hipFuncSetAttribute((const void*)sort_hist_kernel,
                                               hipFuncAttributeMaxDynamicSharedMemorySize, (int)shm);
            if (e != hipSuccess) return e;
        }
        sort_hist_kernel<<<nch, SORT_CHUNK, shm, st>>>(a);
        sort_offsets_kernel<<<1, 1024, 0, st>>>(a);
        sort_scatter_kernel<<<nch, SORT_CHUNK, 0, st>>>(a);
    }
    return hipGetLastError();
}

hipError_t launch_select(const GeoFixed* gf, const GeoTable* gt, const SelectArgs& a, hipStream_t st) {
    if (a.rows == 0) return hipSuccess;
    return gf ? select_dispatch(*gf, a, st) : select_dispatch(*gt, a, st);
}

hipError_t launch_select_fused(const GeoFixed& gf, const SelectArgs& a, hipStream_t st) {
    if (a.rows == 0) return hipSuccess;
    if (gf.nb > FUSED_MAX_NBK) return hipErrorInvalidValue;
    const int G = a.Hq / a.Hkv;
    const int ntq = cdiv(gf.nb, FUSED_COLS / G);
    const size_t shm = (size_t)FUSED_COLS * (gf.nb + 1) * sizeof(float);
    if (shm > 65536) {
        hipError_t e = hipFuncSetAttribute((const void*)select_fused_kernel,
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)shm);
        if (e != hipSuccess) return e;
    }
    select_fused_kernel<<<gf.nseq * a.Hkv * ntq, FUSED_WAVES * 64, shm, st>>>(gf, a);
    return select_dispatch(gf, a, st, true);
}

}  // namespace fp
