"""Batch front-ends of the oracle: a fixed-shape batch [batch, S, H, d] and a
paged varlen batch (paged KV cache plus continuous batching: lode.cx page,
operator paragraph; aimodeling.com page, "Framework integration" bullet).
Test infrastructure only.
"""
from __future__ import annotations

import math
from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np
import torch

from .core import prefill
from .fp8 import widen_fp8


def widen_bf16(t: torch.Tensor) -> np.ndarray:
    """Exact widening of a bfloat16 CPU tensor to float64."""
    assert t.dtype == torch.bfloat16
    return t.to(torch.float64).numpy()


def _widen(t: torch.Tensor, scale: Optional[torch.Tensor]) -> np.ndarray:
    if t.dtype == torch.bfloat16:
        return widen_bf16(t)
    assert t.dtype == torch.uint8 and scale is not None
    return widen_fp8(t.numpy(), scale.numpy())


def prefill_fixed(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, B: int, tau: float,
                  c: Optional[float] = None,
                  q_scale=None, k_scale=None, v_scale=None,
                  keep: Optional[Sequence[np.ndarray]] = None,
                  rows: Optional[Sequence[Sequence[Tuple[int, int]]]] = None,
                  with_output: bool = True) -> List[Dict[str, np.ndarray]]:
    """E1-E6 for every sequence of a fixed-shape batch (q [batch, S, Hq, d])."""
    out = []
    for b in range(q.shape[0]):
        qs = None if q_scale is None else q_scale[b]
        ks = None if k_scale is None else k_scale[b]
        vs = None if v_scale is None else v_scale[b]
        out.append(prefill(_widen(q[b], qs), _widen(k[b], ks), _widen(v[b], vs), B, tau, c,
                           P=0, keep=None if keep is None else keep[b],
                           rows=None if rows is None else rows[b], with_output=with_output))
    return out


def gather_pages(cache: torch.Tensor, table_row: np.ndarray, L: int) -> torch.Tensor:
    """Token s of a sequence lives in slot s % page of physical page table_row[s // page]."""
    page = cache.shape[1]
    toks = []
    for s in range(0, L, page):
        pg = int(table_row[s // page])
        n = min(page, L - s)
        toks.append(cache[pg, :n])
    return torch.cat(toks, dim=0)


def varlen_sequence(q: torch.Tensor, cu_seqlens_q: np.ndarray, seqlens_k: np.ndarray,
                    k_cache: torch.Tensor, v_cache: torch.Tensor, block_table: np.ndarray, b: int,
                    q_scale=None, k_scale=None, v_scale=None) -> Tuple[np.ndarray, np.ndarray, np.ndarray, int]:
    """(q, k, v) of sequence b widened to float64 -- present query rows
    [P, L), keys and values [0, L) gathered from the pages -- and P. fp8 codes
    take the sequence's scales, one per 128 positions ([H, nsb] per sequence)."""
    L = int(seqlens_k[b])
    lo, hi = int(cu_seqlens_q[b]), int(cu_seqlens_q[b + 1])
    P = L - (hi - lo)
    row = np.asarray(block_table)[b]
    kb, vb, qb = gather_pages(k_cache, row, L), gather_pages(v_cache, row, L), q[lo:hi]
    if q.dtype == torch.bfloat16:
        return widen_bf16(qb), widen_bf16(kb), widen_bf16(vb), P
    return (widen_fp8(qb.numpy(), q_scale[b].numpy(), pos0=P), widen_fp8(kb.numpy(), k_scale[b].numpy()),
            widen_fp8(vb.numpy(), v_scale[b].numpy()), P)


def prefill_varlen(q: torch.Tensor, cu_seqlens_q: np.ndarray, seqlens_k: np.ndarray,
                   k_cache: torch.Tensor, v_cache: torch.Tensor, block_table: np.ndarray,
                   B: int, tau: float, c: Optional[float] = None,
                   keep: Optional[Sequence[np.ndarray]] = None,
                   rows: Optional[Sequence[Sequence[Tuple[int, int]]]] = None,
                   with_output: bool = True,
                   q_scale=None, k_scale=None, v_scale=None) -> List[Dict[str, np.ndarray]]:
    """E1-E6 per sequence of a paged varlen batch.  Sequence b has L_b =
    seqlens_k[b] keys (cache, new chunk included) and q_len_b = cu[b+1] - cu[b]
    present rows [L_b - q_len_b, L_b) packed in q (bf16, or fp8 codes with
    per-sequence scales)."""
    out = []
    for b in range(len(seqlens_k)):
        qw, kw, vw, P = varlen_sequence(q, cu_seqlens_q, seqlens_k, k_cache, v_cache, block_table, b,
                                        q_scale, k_scale, v_scale)
        out.append(prefill(qw, kw, vw, B, tau, c, P=P,
                           keep=None if keep is None else keep[b],
                           rows=None if rows is None else rows[b], with_output=with_output))
    return out
