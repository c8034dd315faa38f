"""Loop-by-loop routines for tiny inputs, written independently of core.py so
that the two can pin each other. Test infrastructure only.

Everything is pure Python over float64 scalars: no matrix products, no numpy
reductions, one token pair at a time.
"""
from __future__ import annotations

import math
from typing import List, Tuple

import numpy as np


def _dot(a, b) -> float:
    return sum(float(x) * float(y) for x, y in zip(a, b))


def block_mean_logit(q, k, c, P, L, B, h, g, i, j) -> float:
    """Mean over the block pair of the token logits c<q_t, k_s> (present rows only)."""
    acc = 0.0
    n = 0
    for t in range(max(i * B, P), min((i + 1) * B, L)):
        for s in range(j * B, min((j + 1) * B, L)):
            acc += c * _dot(q[t - P, h], k[s, g])
            n += 1
    return acc / n


def select_enum(q, k, c, P, L, B, G, tau, per_head=False) -> np.ndarray:
    """Kept-block mask [Hkv, nq, nb] by enumeration: for every (g, i, j) test
    whether some head of the group has a block score within tau of its own row
    maximum, or j is the sink or the diagonal. per_head: one list per query
    head ([Hq, nq, nb]), each head judged on its own scores."""
    Hq = q.shape[1]
    if per_head:
        Hkv_real = k.shape[1]
        out = []
        for h in range(Hq):
            kk = k[:, [h // (Hq // Hkv_real)]]
            out.append(select_enum(q[:, [h]], kk, c, P, L, B, 1, tau)[0])
        return np.array(out)
    Hkv = Hq // G
    i0 = P // B
    i1 = (L - 1) // B
    nb = (L + B - 1) // B
    keep = np.zeros((Hkv, i1 - i0 + 1, nb), dtype=bool)
    for g in range(Hkv):
        for i in range(i0, i1 + 1):
            sc = {}
            for h in range(g * G, (g + 1) * G):
                for j in range(i + 1):
                    sc[h, j] = block_mean_logit(q, k, c, P, L, B, h, h // G, i, j)
            for j in range(i + 1):
                ok = j == 0 or j == i
                for h in range(g * G, (g + 1) * G):
                    best = max(sc[h, jj] for jj in range(i + 1))
                    if sc[h, j] - best >= -tau:
                        ok = True
                keep[g, i - i0, j] = ok
    return keep


def attend_augmented(q, k, v, keep, c, P, L, B, G, block_score=False) -> Tuple[np.ndarray, np.ndarray]:
    """Softmax attention of every present row over an explicitly built list of
    (logit, value) entries: each causal token of a kept block, and one entry
    per pruned block whose key and value are the block's token means and whose
    logit carries + ln(block size). keep is [Hkv, ...] (one list per KV head)
    or [Hq, ...] (one per query head). block_score: the pruned block's logit
    is the block pair's mean token logit (the block score) + ln(block size),
    the same for every row of the query block."""
    Hq, d = q.shape[1], q.shape[2]
    Hkv = Hq // G
    o = np.zeros((L - P, Hq, d))
    lse = np.zeros((Hq, L - P))
    for t in range(P, L):
        i = t // B
        for h in range(Hq):
            g = h // G
            lst = h if keep.shape[0] == Hq else g
            entries: List[Tuple[float, List[float]]] = []
            for j in range(i + 1):
                toks = list(range(j * B, min((j + 1) * B, L)))
                if keep[lst, i - P // B, j]:
                    for s in toks:
                        if s <= t:
                            entries.append((c * _dot(q[t - P, h], k[s, g]), list(v[s, g])))
                else:
                    kb = [sum(float(k[s, g, e]) for s in toks) / len(toks) for e in range(d)]
                    vb = [sum(float(v[s, g, e]) for s in toks) / len(toks) for e in range(d)]
                    z = (block_mean_logit(q, k, c, P, L, B, h, g, i, j) if block_score
                         else c * _dot(q[t - P, h], kb))
                    entries.append((z + math.log(len(toks)), vb))
            m = max(z for z, _ in entries)
            den = sum(math.exp(z - m) for z, _ in entries)
            for e in range(d):
                o[t - P, h, e] = sum(math.exp(z - m) * val[e] for z, val in entries) / den
            lse[h, t - P] = m + math.log(den)
    return o, lse


def dense_causal_loops(q, k, v, c, P, L, G) -> np.ndarray:
    """Textbook causal softmax attention, one pair at a time."""
    Hq, d = q.shape[1], q.shape[2]
    o = np.zeros((L - P, Hq, d))
    for t in range(P, L):
        for h in range(Hq):
            g = h // G
            z = [c * _dot(q[t - P, h], k[s, g]) for s in range(t + 1)]
            m = max(z)
            w = [math.exp(x - m) for x in z]
            den = sum(w)
            for e in range(d):
                o[t - P, h, e] = sum(w[s] * float(v[s, g, e]) for s in range(t + 1)) / den
    return o
