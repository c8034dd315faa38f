"""Shared helpers of the GPU parity tests: kept-list decoding and the
comparison rules (kept lists exact except inside the 1e-3 threshold band;
outputs within the stated tolerances, evaluated under the GPU's validated
kept lists)."""
from __future__ import annotations

import numpy as np

import os
from concurrent.futures import ThreadPoolExecutor

import oracle

BAND = 1e-3
TOL = {"bf16": (2e-2, 2e-3), "fp8": (6e-2, 6e-3)}   # (max-abs, mean-abs)


def workers() -> int:
    """Oracle threads: the host's cores, at most 16 (numpy's BLAS calls
    release the GIL)."""
    return max(1, min(16, os.cpu_count() or 1))


def _row_chunks(todo, n):
    return [todo[w::n] for w in range(n)] if todo else []


def attend_threaded(q, k, v, keep, kbar, vbar, c, B, P, rows=None, correction=True):
    """oracle.attend over every (g, il) row (or `rows`), split over threads
    that fill one shared (o, lse) pair: the rows are independent, so the
    result is the same as one call. BLAS runs single-threaded per call."""
    from threadpoolctl import threadpool_limits
    L, Hkv, d = k.shape
    Hq = q.shape[1]
    i0, nq = oracle.query_blocks(P, L, B)
    o = np.full((L - P, Hq, d), np.nan)
    lse = np.full((Hq, L - P), np.nan)
    todo = list(rows) if rows is not None else [(g, il) for il in range(nq) for g in range(Hkv)]
    # heavy rows (late query blocks) first, dealt round-robin
    todo.sort(key=lambda r: -r[1])
    with threadpool_limits(limits=1), ThreadPoolExecutor(workers()) as ex:
        list(ex.map(lambda ch: oracle.attend(q, k, v, keep, kbar, vbar, c, B, P, rows=ch,
                                             correction=correction, out=(o, lse)),
                    _row_chunks(todo, workers())))
    return o, lse


# Worst relative error of one 128-dim logit c<q,k> computed on the MFMA units,
# as a fraction of c * sum_d |q_d| |k_d|: bf16 (32x32x16, fp32 accumulation)
# is held to the fp32 summation bound of 128 terms, 2^-17 (a probe of random,
# wide-range and cancelling bf16 operands against exact sums measured at most
# 2^-21.2); the fp8 form (32x32x64 f8f6f4) adds its 64 products with far
# fewer bits -- the same probe on random E4M3 codes measured up to 2^-12.4 --
# so fp8 logits are held to 2^-11.
KEPT_REL = {"bf16": 2.0 ** -17, "fp8": 2.0 ** -11}


def lse_bound(q, k, keep, kbar, lse_ref, c, B, P, rows=None, correction=True, kind="bf16", pruned=None):
    """Per-element bound on |lse_gpu - lse_oracle| [Hq, L-P], from the data.

    lse is 1-Lipschitz in every logit (max norm), so the bound is the largest
    error of any one logit of the row plus the rounding of lse itself:
      kept token s:   c<q,k_s> from exact products summed on the MFMA over
                      128 dims: at most KEPT_REL[kind] * c * sum_d |q_d| |k_sd|;
      pseudo-token j: c<q,Kbar_j> with Kbar_j split into bf16 hi + lo
                      (residual at most 2^-16 |Kbar_j| per element) and 256
                      products summed in fp32 (2^-16 again): 2^-15 * c *
                      sum_d |q_d| |Kbar_jd|;
      lse itself:     m + log2(l), scaled by ln 2, in fp32, with exp2/log2
                      approximations: 2^-19 * (1 + |lse|).
    sum_d |q_d| |k_sd| is bounded by sum_d |q_d| max_s |k_sd| over the row's
    kept tokens (pruned blocks: exact per block). Rows not evaluated are NaN.
    correction=False: the ablation without pseudo-tokens. pruned: a separate
    mask of the pseudo-token blocks (default: every block keep leaves out),
    e.g. the blocks any head of a group prunes when lists are per head."""
    L, Hkv, d = k.shape
    Hq = q.shape[1]
    G = Hq // Hkv
    i0, nq = oracle.query_blocks(P, L, B)
    bound = np.full((Hq, L - P), np.nan)
    todo = list(rows) if rows is not None else [(g, il) for il in range(nq) for g in range(Hkv)]
    with ThreadPoolExecutor(workers()) as ex:
        list(ex.map(lambda ch: _lse_bound_rows(q, k, keep, kbar, lse_ref, c, B, P, G, i0, ch, bound, correction,
                                               KEPT_REL[kind], ~keep if pruned is None else pruned),
                    _row_chunks(todo, workers())))
    return bound


def _lse_bound_rows(q, k, keep, kbar, lse_ref, c, B, P, G, i0, todo, bound, correction, kept_rel, pruned):
    L = k.shape[0]
    for g, il in todo:
        i = i0 + il
        lo, hi = max(i * B, P), min((i + 1) * B, L)
        kj = np.nonzero(keep[g, il, :i + 1])[0]
        pj = np.nonzero(pruned[g, il, :i + 1])[0] if correction else []
        kmax = np.max([np.abs(k[j * B:min((j + 1) * B, L), g]).max(axis=0) for j in kj], axis=0)
        qa = np.abs(q[lo - P:hi - P, g * G:(g + 1) * G])          # [rows, G, d]
        a_kept = c * (qa @ kmax)                                   # [rows, G]
        a_pr = (c * (qa @ np.abs(kbar[g, pj]).T)).max(axis=2) if len(pj) else 0.0
        lr = lse_ref[g * G:(g + 1) * G, lo - P:hi - P].T
        bound[g * G:(g + 1) * G, lo - P:hi - P] = (kept_rel * a_kept + 2.0 ** -15 * a_pr
                                                   + 2.0 ** -19 * (1 + np.abs(lr))).T


def check_lse(lse_gpu, lse_ref, bound):
    """Every evaluated element within its per-row bound; returns (max error,
    largest error / bound)."""
    ok = ~np.isnan(lse_ref)
    err = np.abs(lse_gpu[ok] - lse_ref[ok])
    b = bound[ok]
    worst = float((err / b).max())
    assert (err <= b).all(), f"lse error {float(err[err > b].max()):.3e} beyond its bound ({worst:.2f}x)"
    return float(err.max()), worst


def csr_to_keep(row_ptr: np.ndarray, col_idx: np.ndarray, row0: int, Hkv: int, nq: int, nb: int) -> np.ndarray:
    keep = np.zeros((Hkv, nq, nb), dtype=bool)
    for g in range(Hkv):
        for il in range(nq):
            r = row0 + g * nq + il
            cols = col_idx[row_ptr[r]:row_ptr[r + 1]]
            keep[g, il, cols] = True
    return keep


def check_csr_wellformed(row_ptr: np.ndarray, col_idx: np.ndarray, i_of_row) -> None:
    assert row_ptr[0] == 0
    assert np.all(np.diff(row_ptr) >= 1)
    for r in range(len(row_ptr) - 1):
        cols = col_idx[row_ptr[r]:row_ptr[r + 1]]
        i = i_of_row(r)
        assert np.all(np.diff(cols) > 0), f"row {r}: columns not strictly ascending"
        assert cols[0] == 0 and cols[-1] == i, f"row {r}: sink/diagonal missing"


def compare_masks(gpu_keep: np.ndarray, ref_keep: np.ndarray, R: np.ndarray, tau: float):
    diff = gpu_keep != ref_keep
    with np.errstate(invalid="ignore"):         # R = -inf (future) with tau = +inf: NaN, not in the band
        band = np.abs(R + tau) <= BAND
    out_band = int((diff & ~band).sum())
    assert out_band == 0, f"{out_band} kept-block mismatches outside the threshold band"
    return int(diff.sum()), int(band.sum())


def compare_outputs(o_gpu: np.ndarray, o_ref: np.ndarray, kind: str):
    mask = ~np.isnan(o_ref)
    err = np.abs(o_gpu[mask] - o_ref[mask])
    mx, mean = float(err.max()), float(err.mean())
    tmax, tmean = TOL[kind]
    assert mx <= tmax and mean <= tmean, f"{kind}: max|err| {mx:.3e} (<= {tmax}), mean|err| {mean:.3e} (<= {tmean})"
    return mx, mean


# Schedule groups (the library's documented rule): the (sequence, KV head)
# pairs, in row order, are cut by where each pair's K/V starts, in units of
# 128 MiB of K and V; the groups are widened when ngroups * (max_nbk + 1)
# would pass 32768 histogram bins.
SCHED_GROUP_BYTES = 128 << 20
SORT_MAX_BINS = 32768


def sched_groups(seg_nbk, seg_rows, block, esz, max_nbk):
    """Group id of every row; seg_nbk / seg_rows: key blocks and rows of each
    (sequence, KV head) pair in row order."""
    units = max(SCHED_GROUP_BYTES // (block * 128 * esz * 2), 1)
    total = int(sum(seg_nbk))
    ng = max(-(-total // units), 1)
    nmax = max(SORT_MAX_BINS // (max_nbk + 1), 1)
    if ng > nmax:
        units = -(-total // nmax)
        ng = max(-(-total // units), 1)
    groups, start = [], 0
    for nbk, nr in zip(seg_nbk, seg_rows):
        groups += [min(start // units, ng - 1)] * nr
        start += nbk
    return np.array(groups, dtype=np.int64)


def fixed_sched_groups(batch, Hkv, nb, block, esz):
    return sched_groups([nb] * (batch * Hkv), [nb] * (batch * Hkv), block, esz, nb)


def check_sched(sched: np.ndarray, counts: np.ndarray, groups: np.ndarray) -> None:
    """Heavy-row-first within each group, groups in order, ties by row id."""
    assert sorted(sched.tolist()) == list(range(len(counts)))
    order = sorted(range(len(counts)), key=lambda r: (groups[r], -counts[r], r))
    assert sched.tolist() == order
