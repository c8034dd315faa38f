"""Plain, slow, obviously-correct CPU oracle for block-sparse prefill attention.

TEST INFRASTRUCTURE ONLY. Nothing on the product path imports this package:
only the tests, the smoke check and the benchmark's CPU-baseline leg do. It
shares no code with the GPU library (no kernels, headers, helpers or
constants) and imports nothing from it.

What it computes (FlashPrefill V2, as described on the lode.cx page, "How It
Works", the aipulsen.com article body, and the aimodeling.com page, "From
Prototype to Production"): a block-level score estimate per (query block, key
block) pair, a max-based dynamic threshold relative to the row maximum, sparse
attention over the kept blocks, and a mean-correction term standing in for the
pruned blocks. The pages state no formulas; the equations below are the
plainest reading and are this library's contract.

Notation: sequence of L keys, of which rows t in [P, L) are present queries
(P = cached prefix, 0 for a one-shot prefill). Square blocks of B tokens on
the absolute-position grid. Query block i covers I_i = [max(iB, P),
min((i+1)B, L)); key block j covers J_j = [jB, min((j+1)B, L)). G = Hq / Hkv
query heads share KV head g(h) = floor(h / G). c = softmax scale.

  E1  Qbar[h,i] = mean_{t in I_i} q[t,h]     Kbar[g,j] = mean_{s in J_j} k[s,g]
      Vbar[g,j] = mean_{s in J_j} v[s,g]
  E2  S[h,i,j] = c * <Qbar[h,i], Kbar[g(h),j]>          (0 <= j <= i)
  E3  M[h,i] = max_{0<=j<=i} S[h,i,j]
  E4  R[g,i,j] = max_{h in group g} (S[h,i,j] - M[h,i])
  E5  keep[g,i] = {0, i} U { j <= i : R[g,i,j] >= -tau };  pruned = [0, i] \\ keep
  E6  for t in I_i and head h of group g:
        exact tokens A = { s in J_j, j in keep[g,i] : s <= t }, logit z_s = c<q_t, k_s>
        one pseudo-token per pruned block j: key Kbar[g,j], value Vbar[g,j],
        logit c<q_t, Kbar[g,j]> + ln|J_j|
        o[t,h] = softmax-weighted sum of the values over A and the pseudo-tokens
        lse[h,t] = log of the softmax denominator (with the max added back)

Everything is float64. Inputs are the stored tensors widened exactly.

Parity pins (tests/test_oracle_*.py): E1-E2 against the block-averaged full
logit matrix; E3-E5 against a loop-by-loop enumeration, monotonicity in tau
and its limits; E6 against textbook dense causal attention (torch SDPA in
float64) at tau = inf, exactness for block size 1 and for block-constant K/V
at every tau, a closed form for zero queries (cumulative mean of v at every
tau), a loop-by-loop augmented-softmax routine, causality and key-offset
invariance; the fp8 decode against torch's own float8_e4m3fn cast. The
paper's actual estimator and correction formulas are not printed on the pages,
so E1-E6 themselves are "parity unpinned" against the paper: they are the
stated reading.
"""
from .core import (
    nblocks, query_blocks, pool_queries, pool_keys, pool_update, pool_means, prefill_chunked,
    block_scores, select,
    attend, prefill, kept_fraction, threshold_margin, causal_block_pairs,
    dense_flops, kept_flops, correction_flops,
)
from .fp8 import decode_e4m3, widen_fp8
from .batch import prefill_fixed, prefill_varlen, varlen_sequence, widen_bf16

__all__ = [
    "nblocks", "query_blocks", "pool_queries", "pool_keys", "pool_update", "pool_means", "prefill_chunked",
    "block_scores", "select",
    "attend", "prefill", "kept_fraction", "threshold_margin", "causal_block_pairs",
    "dense_flops", "kept_flops", "correction_flops", "decode_e4m3", "widen_fp8",
    "prefill_fixed", "prefill_varlen", "varlen_sequence", "widen_bf16",
]
