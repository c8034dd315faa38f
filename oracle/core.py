"""E1-E6 for one sequence, float64, numpy. Test infrastructure only.

Each function cites the passage it follows. The pages (FlashPrefill V2 news
summaries) describe the method in prose only; equation numbers E1-E6 refer to
the reading written out in this package's docstring.
"""
from __future__ import annotations

import math
from typing import Dict, Optional, Sequence, Tuple

import numpy as np

NEG_INF = -np.inf


def nblocks(L: int, B: int) -> int:
    """Key blocks of a sequence of L keys (blocks partition tokens into fixed-size
    groups: stuffinsider.com page, "Technical Details")."""
    return (L + B - 1) // B


def query_blocks(P: int, L: int, B: int) -> Tuple[int, int]:
    """(first, count) of the query blocks holding present rows [P, L); none
    when there are no present rows (P = L: the whole sequence is cached)."""
    i0 = P // B
    if P >= L:
        return i0, 0
    i1 = (L - 1) // B
    return i0, i1 - i0 + 1


def pool_queries(q: np.ndarray, B: int, P: int, L: int) -> np.ndarray:
    """E1 for queries: q [L-P, Hq, d] holds rows P..L-1.  Returns Qbar [Hq, nq, d],
    the mean over the present rows of each query block (block-level estimate,
    aipulsen.com article body)."""
    i0, nq = query_blocks(P, L, B)
    Hq, d = q.shape[1], q.shape[2]
    out = np.empty((Hq, nq, d))
    for il in range(nq):
        i = i0 + il
        lo, hi = max(i * B, P), min((i + 1) * B, L)
        out[:, il, :] = q[lo - P:hi - P].mean(axis=0)
    return out


def pool_keys(k: np.ndarray, B: int) -> np.ndarray:
    """E1 for keys or values: k [L, H, d] -> [H, nb, d], mean over each key block."""
    L, H, d = k.shape
    nb = nblocks(L, B)
    out = np.empty((H, nb, d))
    for j in range(nb):
        out[:, j, :] = k[j * B:min((j + 1) * B, L)].mean(axis=0)
    return out


def pool_update(sums: np.ndarray, counts: np.ndarray, x_new: np.ndarray, start: int,
                B: int) -> Tuple[np.ndarray, np.ndarray]:
    """E1 kept incrementally across chunks (the pages' chunked prefill over a
    paged KV cache: lode.cx page, "How It Works", implementation paragraph;
    aimodeling.com page, "Framework integration" bullet). sums [H, nb, d] and
    counts [nb] are the running per-block sums and token counts of the keys
    (or values) seen so far; x_new [n, H, d] holds the keys at positions
    start .. start+n-1. Each new token is added to the sum of its block. The
    block means are sums / counts (pool_means). Returns new arrays, grown as
    far as the new tokens reach."""
    n, H, d = x_new.shape
    nb = nblocks(start + n, B)
    S = np.zeros((H, max(nb, sums.shape[1]), d))
    C = np.zeros(S.shape[1], dtype=np.int64)
    S[:, :sums.shape[1]] = sums
    C[:counts.shape[0]] = counts
    for t in range(n):
        j = (start + t) // B
        S[:, j] += x_new[t]
        C[j] += 1
    return S, C


def pool_means(sums: np.ndarray, counts: np.ndarray, L: int, B: int) -> np.ndarray:
    """The pooled keys of blocks 0 .. nblocks(L)-1 from running sums: the mean
    over each block's present tokens (E1)."""
    nb = nblocks(L, B)
    assert counts.shape[0] >= nb and counts[:nb].min() > 0
    return sums[:, :nb] / counts[:nb, None]


def block_scores(qbar: np.ndarray, kbar: np.ndarray, c: float, i0: int) -> np.ndarray:
    """E2: S[h, il, j] = c <Qbar[h, il], Kbar[g(h), j]> for j <= i0 + il, -inf above.

    One estimate per (query block, key block) pair (aipulsen.com article body;
    the "small sample of attention scores" of the lode.cx page, "How It Works")."""
    Hq, nq, d = qbar.shape
    Hkv, nb, _ = kbar.shape
    G = Hq // Hkv
    S = np.full((Hq, nq, nb), NEG_INF)
    for h in range(Hq):
        g = h // G
        full = c * (qbar[h] @ kbar[g].T)            # [nq, nb]
        for il in range(nq):
            i = i0 + il
            S[h, il, :i + 1] = full[il, :i + 1]
    return S


def select(S: np.ndarray, G: int, tau: float, i0: int, per_head: bool = False) -> Tuple[np.ndarray, np.ndarray]:
    """E3-E5: max-based dynamic threshold (lode.cx page, "How It Works";
    aimodeling.com page, "From Prototype to Production").

    Returns (keep bool [Hkv, nq, nb], R float [Hkv, nq, nb]) with R = -inf and
    keep = False for j > i.  Sink j = 0 and diagonal j = i are always kept.
    per_head: the variant without the GQA union (E4 over one head): each
    query head keeps its own list, keep and R are [Hq, nq, nb]."""
    if isinstance(tau, float) and math.isnan(tau):
        raise ValueError("tau is NaN")
    if per_head:
        return select(S, 1, tau, i0)
    Hq, nq, nb = S.shape
    Hkv = Hq // G
    M = S.max(axis=2)                                # E3, over visible j only (rest -inf)
    R = np.full((Hkv, nq, nb), NEG_INF)
    keep = np.zeros((Hkv, nq, nb), dtype=bool)
    for g in range(Hkv):
        for il in range(nq):
            i = i0 + il
            diff = S[g * G:(g + 1) * G, il, :i + 1] - M[g * G:(g + 1) * G, il, None]
            R[g, il, :i + 1] = diff.max(axis=0)      # E4: union over the group's heads
            keep[g, il, :i + 1] = R[g, il, :i + 1] >= -tau   # E5, inclusive
            keep[g, il, 0] = True
            keep[g, il, i] = True
    return keep, R


def attend(q: np.ndarray, k: np.ndarray, v: np.ndarray, keep: np.ndarray,
           kbar: np.ndarray, vbar: np.ndarray, c: float, B: int, P: int,
           rows: Optional[Sequence[Tuple[int, int]]] = None,
           correction: bool = True,
           out: Optional[Tuple[np.ndarray, np.ndarray]] = None,
           block_scores: Optional[np.ndarray] = None) -> Tuple[np.ndarray, np.ndarray]:
    """E6: sparse attention over kept blocks plus the mean-correction pseudo-tokens.

    Sparse operator over kept blocks: lode.cx page, "How It Works" and the
    operator bullet list; correction term for pruning bias: lode.cx page, "How
    It Works", and aimodeling.com page, "Error correction" bullet.

    q [L-P, Hq, d] (rows P..L-1), k/v [L, Hkv, d], keep [Hkv, nq, nb].
    rows: optional list of (g, il) to evaluate; other outputs stay NaN.
    correction=False is the ablation without the correction: the pruned blocks
    are dropped (no pseudo-tokens).
    out: optional preallocated (o, lse) to fill instead (only the rows
    evaluated are written; callers may split the rows over threads).
    Per-head lists (keep [Hq, nq, nb], the variant without the GQA union):
    each query head h attends its own list; rows are then (h, il) pairs.
    block_scores (S [Hq, nq, nb] of E2): the variant whose pruned block j
    stands in with the logit S[h, i, j] + ln|J_j| for every row of query
    block i, instead of c<q_t, Kbar_j> + ln|J_j|.
    Returns o [L-P, Hq, d] and lse [Hq, L-P]."""
    L, Hkv, d = k.shape
    Hq = q.shape[1]
    if keep.shape[0] == Hq and Hq != Hkv:
        # per-head lists: each head is its own group of one, reading KV head h // G
        G = Hq // Hkv
        todo = rows if rows is not None else [(h, il) for h in range(Hq)
                                              for il in range(query_blocks(P, L, B)[1])]
        if out is None:
            out = (np.full((L - P, Hq, d), np.nan), np.full((Hq, L - P), np.nan))
        for h, il in todo:
            sub = attend(q[:, h:h + 1], k[:, h // G:h // G + 1], v[:, h // G:h // G + 1], keep[h:h + 1],
                         kbar[h // G:h // G + 1], vbar[h // G:h // G + 1], c, B, P, rows=[(0, il)],
                         correction=correction,
                         block_scores=None if block_scores is None else block_scores[h:h + 1])
            i0, _ = query_blocks(P, L, B)
            lo, hi = max((i0 + il) * B, P), min((i0 + il + 1) * B, L)
            out[0][lo - P:hi - P, h] = sub[0][lo - P:hi - P, 0]
            out[1][h, lo - P:hi - P] = sub[1][0, lo - P:hi - P]
        return out
    G = Hq // Hkv
    i0, nq = query_blocks(P, L, B)
    if out is None:
        o = np.full((L - P, Hq, d), np.nan)
        lse = np.full((Hq, L - P), np.nan)
    else:
        o, lse = out
    todo = rows if rows is not None else [(g, il) for g in range(Hkv) for il in range(nq)]
    for (g, il) in todo:
        i = i0 + il
        lo, hi = max(i * B, P), min((i + 1) * B, L)
        kept_j = [j for j in range(i + 1) if keep[g, il, j]]
        pruned_j = [j for j in range(i + 1) if not keep[g, il, j]] if correction else []
        tok = np.concatenate([np.arange(j * B, min((j + 1) * B, L)) for j in kept_j])
        Kx = k[tok, g, :]
        Vx = v[tok, g, :]
        Kp = kbar[g, pruned_j, :]
        Vp = vbar[g, pruned_j, :]
        bias = np.array([math.log(min((j + 1) * B, L) - j * B) for j in pruned_j])
        t = np.arange(lo, hi)
        future = tok[None, :] > t[:, None]           # causal inside kept blocks
        for h in range(g * G, (g + 1) * G):
            Q = q[lo - P:hi - P, h, :]               # [rows, d]
            z = c * (Q @ Kx.T)
            z[future] = NEG_INF
            if block_scores is None:
                zp = c * (Q @ Kp.T) + bias[None, :]
            else:                                    # one logit per block pair, the same for every row
                zp = np.repeat(block_scores[h, il, pruned_j][None, :] + bias[None, :], hi - lo, axis=0)
            m = np.maximum(z.max(axis=1), zp.max(axis=1) if len(pruned_j) else NEG_INF)
            w = np.exp(z - m[:, None])
            wp = np.exp(zp - m[:, None])
            l = w.sum(axis=1) + wp.sum(axis=1)
            o[lo - P:hi - P, h, :] = (w @ Vx + wp @ Vp) / l[:, None]
            lse[h, lo - P:hi - P] = m + np.log(l)
    return o, lse


VARIANTS = ("mean", "none", "per_head", "block_score")


def prefill(q: np.ndarray, k: np.ndarray, v: np.ndarray, B: int, tau: float,
            c: Optional[float] = None, P: int = 0,
            keep: Optional[np.ndarray] = None,
            rows: Optional[Sequence[Tuple[int, int]]] = None,
            with_output: bool = True, correction: bool = True,
            variant: str = "mean",
            pooled_kv: Optional[Tuple[np.ndarray, np.ndarray]] = None) -> Dict[str, np.ndarray]:
    """E1-E6 for one sequence.  keep overrides the oracle's own mask (used to
    evaluate E6 under another, validated mask); correction=False evaluates the
    ablation without the mean correction. variant: "mean" (E1-E6 as stated),
    "none" (no correction), "per_head" (one kept list per query head, no GQA
    union; keep and R are [Hq, nq, nb]) or "block_score" (the pruned blocks'
    pseudo-tokens take the block score S[h, i, j] + ln|J_j| as logit).
    pooled_kv: (Kbar, Vbar) [Hkv, nblocks(L), d] kept from earlier chunks
    (prefill_chunked), used in place of pooling k and v here."""
    if variant not in VARIANTS:
        raise ValueError(f"unknown variant {variant}")
    if variant == "none":
        correction = False
    L, Hkv, d = k.shape
    Hq = q.shape[1]
    assert q.shape[0] == L - P and Hq % Hkv == 0 and v.shape == k.shape
    G = Hq // Hkv
    if c is None:
        c = 1.0 / math.sqrt(d)
    i0, nq = query_blocks(P, L, B)
    qbar = pool_queries(q, B, P, L)
    if pooled_kv is None:
        kbar, vbar = pool_keys(k, B), pool_keys(v, B)
    else:
        kbar, vbar = pooled_kv
        assert kbar.shape == (Hkv, nblocks(L, B), d) and vbar.shape == kbar.shape
    S = block_scores(qbar, kbar, c, i0)
    own_keep, R = select(S, G, tau, i0, per_head=variant == "per_head")
    out = dict(qbar=qbar, kbar=kbar, vbar=vbar, S=S, R=R, keep=own_keep, i0=i0, nq=nq)
    if with_output:
        use = own_keep if keep is None else keep
        out["o"], out["lse"] = attend(q, k, v, use, kbar, vbar, c, B, P, rows=rows, correction=correction,
                                      block_scores=S if variant == "block_score" else None)
    return out


def prefill_chunked(q: np.ndarray, k: np.ndarray, v: np.ndarray, B: int, tau: float,
                    ends: Sequence[int], c: Optional[float] = None,
                    variant: str = "mean", with_output: bool = True) -> list:
    """Chunked prefill of one sequence with a pooled-KV cache: chunk n holds
    the query rows [ends[n-1], ends[n]) (ends[-1] = L) and sees the keys
    [0, ends[n]). The per-block sums of K and V are carried from chunk to
    chunk and each chunk adds only its own keys (pool_update); E2-E6 then run
    on the cached means (prefill with pooled_kv). q, k, v hold the whole
    sequence. Returns one prefill result per chunk."""
    L, Hkv, d = k.shape
    sk = np.zeros((Hkv, 0, d)); sv = np.zeros((Hkv, 0, d)); cnt = np.zeros(0, dtype=np.int64)
    out, P = [], 0
    for end in ends:
        assert P < end <= L
        sk, cnt_k = pool_update(sk, cnt, k[P:end], P, B)
        sv, cnt = pool_update(sv, cnt, v[P:end], P, B)
        assert np.array_equal(cnt_k, cnt)
        pooled = (pool_means(sk, cnt, end, B), pool_means(sv, cnt, end, B))
        out.append(prefill(q[P:end], k[:end], v[:end], B, tau, c=c, P=P, variant=variant,
                           pooled_kv=pooled, with_output=with_output))
        P = end
    return out


# ---------------------------------------------------------------------------
# bookkeeping used by reports (counts of blocks and FLOPs)
# ---------------------------------------------------------------------------

def threshold_margin(R: np.ndarray, tau: float) -> np.ndarray:
    """|R + tau|: distance of each block's estimate to the threshold."""
    return np.abs(R + tau)


def causal_block_pairs(P: int, L: int, B: int) -> int:
    i0, nq = query_blocks(P, L, B)
    return sum(i0 + il + 1 for il in range(nq))


def kept_fraction(keep: np.ndarray, P: int, L: int, B: int) -> float:
    """Kept (g, i, j) block pairs over all causal block pairs of all KV heads."""
    return float(keep.sum()) / (keep.shape[0] * causal_block_pairs(P, L, B))


def _pairs(i: int, j: int, P: int, L: int, B: int) -> int:
    lo, hi = max(i * B, P), min((i + 1) * B, L)
    klo, khi = j * B, min((j + 1) * B, L)
    if j < i:
        return (hi - lo) * (khi - klo)
    # diagonal: count s <= t
    return sum(min(t, khi - 1) - klo + 1 for t in range(lo, hi))


def dense_flops(P: int, L: int, d: int, Hq: int) -> float:
    """4 d Hq sum_{present t} (t + 1): dense causal QK^T plus PV."""
    n = L - P
    return 4.0 * d * Hq * (n * (P + 1) + n * (n - 1) / 2.0)


def kept_flops(keep: np.ndarray, P: int, L: int, B: int, d: int, G: int) -> float:
    """4 d G sum over kept (g, i, j) of the causal (t, s) pairs in the block pair."""
    i0, nq = query_blocks(P, L, B)
    tot = 0
    for g in range(keep.shape[0]):
        for il in range(nq):
            i = i0 + il
            for j in np.nonzero(keep[g, il])[0]:
                tot += _pairs(i, int(j), P, L, B)
    return 4.0 * d * G * tot


def correction_flops(keep: np.ndarray, P: int, L: int, B: int, d: int, G: int) -> float:
    """4 d G sum over (g, i) of |I_i| * |pruned_i|."""
    i0, nq = query_blocks(P, L, B)
    tot = 0
    for il in range(nq):
        i = i0 + il
        rows = min((i + 1) * B, L) - max(i * B, P)
        npr = (i + 1) - keep[:, il, :i + 1].sum(axis=1)
        tot += rows * int(npr.sum())
    return 4.0 * d * G * tot
