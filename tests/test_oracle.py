"""Pins of the CPU oracle against facts that do not come from the oracle itself:
closed forms, textbook/library special cases, brute-force enumeration,
invariants and a hand-derived worked example."""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from oracle import brute
from oracle.core import prefill, pool_queries, pool_keys, block_scores, select, attend

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def rnd(shape, seed, scale=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * scale


def dense_sdpa(q, k, v, c, P=0):
    """Dense causal attention through torch's scaled_dot_product_attention in
    float64 (bottom-right aligned when P > 0 by an explicit mask)."""
    Lq, Hq, d = q.shape
    L, Hkv, _ = k.shape
    G = Hq // Hkv
    qt = torch.from_numpy(q).permute(1, 0, 2)[None]
    kt = torch.from_numpy(k).repeat_interleave(G, dim=1).permute(1, 0, 2)[None]
    vt = torch.from_numpy(v).repeat_interleave(G, dim=1).permute(1, 0, 2)[None]
    t = torch.arange(P, L)[:, None]
    s = torch.arange(L)[None, :]
    mask = s <= t
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask, scale=c)
    return o[0].permute(1, 0, 2).numpy()


def dense_numpy(q, k, v, c, P=0):
    Lq, Hq, d = q.shape
    L, Hkv, _ = k.shape
    G = Hq // Hkv
    o = np.empty_like(q)
    lse = np.empty((Hq, Lq))
    t = np.arange(P, L)[:, None]
    s = np.arange(L)[None, :]
    for h in range(Hq):
        z = c * q[:, h] @ k[:, h // G].T
        z[s > t] = -np.inf
        m = z.max(1, keepdims=True)
        w = np.exp(z - m)
        o[:, h] = (w @ v[:, h // G]) / w.sum(1, keepdims=True)
        lse[h] = (m[:, 0] + np.log(w.sum(1)))
    return o, lse


# --------------------------------------------------------------------------
# P1: E1-E2 closed form -- block score = mean token logit of the block pair
# --------------------------------------------------------------------------
@pytest.mark.parametrize("L,P,B", [(100, 0, 16), (100, 37, 16), (64, 0, 8), (70, 64, 8)])
def test_scores_equal_block_averaged_logits(L, P, B):
    Hq, Hkv, d = 4, 2, 16
    q = rnd((L - P, Hq, d), 1)
    k = rnd((L, Hkv, d), 2)
    c = 0.3
    i0, nq = oracle.query_blocks(P, L, B)
    S = block_scores(pool_queries(q, B, P, L), pool_keys(k, B), c, i0)
    G = Hq // Hkv
    for h in range(Hq):
        full = c * q[:, h] @ k[:, h // G].T          # [rows P.., L]
        for il in range(nq):
            i = i0 + il
            rows = slice(max(i * B, P) - P, min((i + 1) * B, L) - P)
            for j in range(nb := oracle.nblocks(L, B)):
                if j > i:
                    assert S[h, il, j] == -np.inf
                    continue
                ref = full[rows, j * B:min((j + 1) * B, L)].mean()
                assert abs(S[h, il, j] - ref) <= 1e-12 * max(1.0, abs(ref))


# --------------------------------------------------------------------------
# P2: E3-E5 by enumeration, monotone in tau, and its limits
# --------------------------------------------------------------------------
@pytest.mark.parametrize("P", [0, 5, 16])
@pytest.mark.parametrize("tau", [0.05, 0.2, 0.6])
def test_select_matches_enumeration(P, tau):
    L, B, Hq, Hkv, d = 44, 8, 4, 2, 8
    q = rnd((L - P, Hq, d), 3) + 1.0
    k = rnd((L, Hkv, d), 4) + np.linspace(0, 2, L)[:, None, None]
    c = 0.5
    out = prefill(q, k, k, B, tau, c, P=P, with_output=False)
    ref = brute.select_enum(q, k, c, P, L, B, Hq // Hkv, tau)
    # no estimate sits within 1e-9 of the threshold, so the sets must agree exactly
    fin = np.isfinite(out["R"])
    assert np.all(np.abs(out["R"][fin] + tau) > 1e-9)
    assert np.array_equal(out["keep"], ref)


def test_select_monotone_and_limits():
    L, B, Hq, Hkv, d = 256, 16, 8, 2, 16
    q = rnd((L, Hq, d), 5) + 0.5
    k = rnd((L, Hkv, d), 6) + np.cumsum(rnd((L, Hkv, d), 7, 0.3), axis=0)
    i0, nq = oracle.query_blocks(0, L, B)
    S = block_scores(pool_queries(q, B, 0, L), pool_keys(k, B), 0.25, i0)
    prev = None
    for tau in [-1.0, 0.0, 0.5, 1.0, 2.0, 4.0, np.inf]:
        keep, R = select(S, Hq // Hkv, tau, i0)
        if prev is not None:
            assert np.all(keep[prev])                         # K(tau1) subset of K(tau2)
        prev = keep
        if tau == np.inf:
            tri = np.tril(np.ones((nq, oracle.nblocks(L, B)), dtype=bool))
            assert np.array_equal(keep, np.broadcast_to(tri, keep.shape))
        if tau < 0:
            exp = np.zeros_like(keep)
            exp[:, :, 0] = True
            for il in range(nq):
                exp[:, il, il] = True
            assert np.array_equal(keep, exp)
    assert np.nanmax(np.where(np.isfinite(R), R, np.nan)) == 0.0   # R <= 0, argmax at 0


def test_select_identical_heads_equals_single_head():
    L, B, d = 128, 16, 16
    q1 = rnd((L, 1, d), 8) + 0.7
    k = rnd((L, 1, d), 9) + np.cumsum(rnd((L, 1, d), 10, 0.5), axis=0)
    qG = np.repeat(q1, 4, axis=1)
    a = prefill(q1, k, k, B, 1.0, 0.2, with_output=False)["keep"]
    b = prefill(qG, k, k, B, 1.0, 0.2, with_output=False)["keep"]
    assert np.array_equal(a, b)


def test_group_union_and_head_mapping():
    # group 1's heads see keys of KV head 1 only: make KV head 0 flat (all blocks
    # tie) and KV head 1 strongly structured; group 0 must keep everything.
    L, B, d = 96, 16, 8
    q = rnd((L, 4, d), 11) + 1.0
    k = np.zeros((L, 2, d))
    k[:, 1] = np.linspace(-3, 3, L)[:, None] * np.ones(d)
    out = prefill(q, k, k, B, 0.5, 1.0, with_output=False)
    nq = out["nq"]
    tri = np.tril(np.ones((nq, nq), dtype=bool))
    assert np.array_equal(out["keep"][0], tri)
    assert not np.array_equal(out["keep"][1], tri)


# --------------------------------------------------------------------------
# P3: tau = inf equals textbook dense causal attention
# --------------------------------------------------------------------------
@pytest.mark.parametrize("L,B,P", [(128, 16, 0), (100, 32, 0), (90, 16, 41)])
def test_tau_inf_is_dense(L, B, P):
    Hq, Hkv, d = 4, 2, 32
    q = rnd((L - P, Hq, d), 12)
    k = rnd((L, Hkv, d), 13)
    v = rnd((L, Hkv, d), 14)
    c = 1 / math.sqrt(d)
    out = prefill(q, k, v, B, np.inf, c, P=P)
    ref = dense_sdpa(q, k, v, c, P)
    ref2, lse2 = dense_numpy(q, k, v, c, P)
    assert np.abs(out["o"] - ref).max() < 1e-12
    assert np.abs(out["o"] - ref2).max() < 1e-12
    assert np.abs(out["lse"] - lse2).max() < 1e-12


def test_dense_loops_tiny():
    L, Hq, Hkv, d = 12, 2, 1, 4
    q = rnd((L, Hq, d), 15)
    k = rnd((L, Hkv, d), 16)
    v = rnd((L, Hkv, d), 17)
    out = prefill(q, k, v, 4, np.inf, 0.5)
    assert np.abs(out["o"] - brute.dense_causal_loops(q, k, v, 0.5, 0, L, 2)).max() < 1e-12


# --------------------------------------------------------------------------
# P4 / P5: the correction is exact for block size 1 and for block-constant K, V
# --------------------------------------------------------------------------
@pytest.mark.parametrize("tau", [-1.0, 0.0, 0.3, 2.0])
def test_block_size_one_is_exact(tau):
    L, Hq, Hkv, d = 40, 4, 2, 16
    q = rnd((L, Hq, d), 18) * 2
    k = rnd((L, Hkv, d), 19) * 2
    v = rnd((L, Hkv, d), 20)
    out = prefill(q, k, v, 1, tau, 0.4)
    ref, lse = dense_numpy(q, k, v, 0.4)
    assert out["keep"].sum() < out["keep"].shape[0] * L * (L + 1) / 2 or tau > 1
    assert np.abs(out["o"] - ref).max() < 1e-12
    assert np.abs(out["lse"] - lse).max() < 1e-12


@pytest.mark.parametrize("tau", [-1.0, 0.5, 3.0])
def test_block_constant_kv_is_exact(tau):
    L, B, Hq, Hkv, d = 96, 8, 4, 1, 16
    nb = L // B
    q = rnd((L, Hq, d), 21)
    kb = rnd((nb, Hkv, d), 22) * 2
    vb = rnd((nb, Hkv, d), 23)
    k = np.repeat(kb, B, axis=0)
    v = np.repeat(vb, B, axis=0)
    out = prefill(q, k, v, B, tau, 0.3)
    ref, lse = dense_numpy(q, k, v, 0.3)
    # rows whose diagonal block is partially visible still see exact tokens there
    assert np.abs(out["o"] - ref).max() < 1e-12
    assert np.abs(out["lse"] - lse).max() < 1e-12


@pytest.mark.parametrize("tau", [-1.0, 1.0, np.inf])
@pytest.mark.parametrize("P", [0, 13])
def test_zero_queries_give_cumulative_mean(tau, P):
    # all logits are 0, so every visible token has equal weight whether it is
    # kept exactly or stands inside a pruned block's pseudo-token (weight |J|)
    L, B, Hq, Hkv, d = 77, 8, 2, 1, 8
    q = np.zeros((L - P, Hq, d))
    k = rnd((L, Hkv, d), 24)
    v = rnd((L, Hkv, d), 25)
    keep_override = None
    out = prefill(q, k, v, B, tau, 1.0, P=P)
    if tau == -1.0:
        # force pruning even though every estimate ties at the row maximum
        keep = np.zeros_like(out["keep"])
        i0, nq = oracle.query_blocks(P, L, B)
        for il in range(nq):
            keep[:, il, 0] = True
            keep[:, il, i0 + il] = True
        out = prefill(q, k, v, B, tau, 1.0, P=P, keep=keep)
    cm = np.cumsum(v[:, 0], axis=0) / np.arange(1, L + 1)[:, None]
    for h in range(Hq):
        assert np.abs(out["o"][:, h] - cm[P:]).max() < 1e-12
        assert np.abs(out["lse"][h] - np.log(np.arange(P + 1, L + 1))).max() < 1e-12


# --------------------------------------------------------------------------
# P6: expanded form, computed pair by pair by an independent routine
# --------------------------------------------------------------------------
@pytest.mark.parametrize("P,tau", [(0, 0.3), (0, 1.0), (7, 0.3), (0, -1.0)])
def test_attend_matches_augmented_loops(P, tau):
    L, B, Hq, Hkv, d = 34, 4, 4, 2, 4
    q = rnd((L - P, Hq, d), 26) + 0.8
    k = rnd((L, Hkv, d), 27) + np.cumsum(rnd((L, Hkv, d), 28, 0.6), axis=0)
    v = rnd((L, Hkv, d), 29)
    out = prefill(q, k, v, B, tau, 0.5, P=P)
    assert (~out["keep"]).any()
    o, lse = brute.attend_augmented(q, k, v, out["keep"], 0.5, P, L, B, Hq // Hkv)
    assert np.abs(out["o"] - o).max() < 1e-12
    assert np.abs(out["lse"] - lse).max() < 1e-12


@pytest.mark.parametrize("P,tau", [(0, 0.3), (7, 1.0), (0, -1.0)])
def test_no_correction_is_masked_dense(P, tau):
    """The ablation without the mean correction is causal softmax attention over
    the tokens of the kept blocks alone, written out here token by token."""
    L, B, Hq, Hkv, d = 34, 4, 4, 2, 4
    q = rnd((L - P, Hq, d), 26) + 0.8
    k = rnd((L, Hkv, d), 27) + np.cumsum(rnd((L, Hkv, d), 28, 0.6), axis=0)
    v = rnd((L, Hkv, d), 29)
    out = prefill(q, k, v, B, tau, 0.5, P=P, correction=False)
    keep, i0 = out["keep"], out["i0"]
    assert (~keep).any()
    G = Hq // Hkv
    for h in range(Hq):
        g = h // G
        for t in range(P, L):
            il = t // B - i0
            s_ok = [s for s in range(t + 1) if keep[g, il, s // B]]
            z = np.array([0.5 * float(q[t - P, h] @ k[s, g]) for s in s_ok])
            w = np.exp(z - z.max())
            o = sum(wi * v[s, g] for wi, s in zip(w, s_ok)) / w.sum()
            assert np.abs(out["o"][t - P, h] - o).max() < 1e-12
            assert abs(out["lse"][h, t - P] - (z.max() + math.log(w.sum()))) < 1e-12
    # with every block kept the two variants coincide
    both = [prefill(q, k, v, B, np.inf, 0.5, P=P, correction=cr)["o"] for cr in (True, False)]
    assert np.abs(both[0] - both[1]).max() == 0.0


# --------------------------------------------------------------------------
# P7: causality with the mask held fixed;  P8: key-offset invariance
# --------------------------------------------------------------------------
def test_causal_mask_with_fixed_mask():
    L, B, Hq, Hkv, d = 64, 16, 2, 1, 8
    q = rnd((L, Hq, d), 30)
    k = rnd((L, Hkv, d), 31)
    v = rnd((L, Hkv, d), 32)
    base = prefill(q, k, v, B, 0.2, 0.5)
    for t in [0, 5, 17, 40, 63]:
        k2, v2 = k.copy(), v.copy()
        k2[t + 1:] += rnd(k2[t + 1:].shape, 33 + t) * 5
        v2[t + 1:] += rnd(v2[t + 1:].shape, 34 + t) * 5
        # keep the mask and pooled values; future-token edits must not reach row t
        o, lse = attend(q, k2, v2, base["keep"], base["kbar"], base["vbar"], 0.5, B, 0)
        assert np.abs(o[t] - base["o"][t]).max() < 1e-12
        assert np.abs(lse[:, t] - base["lse"][:, t]).max() < 1e-12


def test_key_offset_invariance():
    L, B, Hq, Hkv, d = 96, 16, 4, 2, 16
    q = rnd((L, Hq, d), 35) + 0.5
    k = rnd((L, Hkv, d), 36) + np.cumsum(rnd((L, Hkv, d), 37, 0.4), axis=0)
    v = rnd((L, Hkv, d), 38)
    a = prefill(q, k, v, B, 0.7, 0.4)
    shift = rnd((1, Hkv, d), 39) * 3
    b = prefill(q, k + shift, v, B, 0.7, 0.4)
    assert np.array_equal(a["keep"], b["keep"])
    assert np.abs(a["o"] - b["o"]).max() < 1e-9


# --------------------------------------------------------------------------
# P9: chunked prefill, varlen batch, paged storage
# --------------------------------------------------------------------------
def test_chunk_rows_equal_one_shot_rows():
    L, B, Hq, Hkv, d = 120, 16, 4, 2, 8
    q = rnd((L, Hq, d), 40) + 0.5
    k = rnd((L, Hkv, d), 41) + np.cumsum(rnd((L, Hkv, d), 42, 0.5), axis=0)
    v = rnd((L, Hkv, d), 43)
    full = prefill(q, k, v, B, 0.5, 0.4)
    for P in [16, 37, 100]:
        part = prefill(q[P:], k, v, B, 0.5, 0.4, P=P)
        first_full = -(-P // B) * B                 # rows of full query blocks of the chunk
        assert np.abs(part["o"][first_full - P:] - full["o"][first_full:]).max() < 1e-12
        il0 = first_full // B - P // B
        assert np.array_equal(part["keep"][:, il0:], full["keep"][:, first_full // B:])


@pytest.mark.parametrize("ends", [(37,), (16, 40, 75), (5, 6, 64, 65, 100), (48, 96, 113)])
def test_pool_update_chunks_equal_one_shot_pooling(ends):
    """Running per-block sums fed chunk by chunk give exactly the one-shot
    block means (E1) once every token is in: dyadic inputs make every sum
    exact, so the comparison is bit for bit; the counts are the block sizes."""
    L, B, H, d = ends[-1], 16, 3, 5
    x = np.random.default_rng(44).integers(-64, 64, (L, H, d)) / 8.0
    sums, counts, P = np.zeros((H, 0, d)), np.zeros(0, dtype=np.int64), 0
    for end in ends:
        sums, counts = oracle.pool_update(sums, counts, x[P:end], P, B)
        # after each chunk the means cover exactly the keys seen so far
        assert np.array_equal(oracle.pool_means(sums, counts, end, B), pool_keys(x[:end], B))
        sizes = [min((j + 1) * B, end) - j * B for j in range(-(-end // B))]
        assert counts.tolist() == sizes
        P = end


def test_prefill_chunked_equals_uncached_chunks_and_one_shot_rows():
    """A chunked prefill that carries the pooled K/V from chunk to chunk
    equals, chunk by chunk, a prefill that pools all of the chunk's keys
    afresh, and its rows in full query blocks equal the one-shot prefill's."""
    L, B, Hq, Hkv, d = 150, 16, 4, 2, 8
    q = rnd((L, Hq, d), 45) + 0.5
    k = rnd((L, Hkv, d), 46) + np.cumsum(rnd((L, Hkv, d), 47, 0.5), axis=0)
    v = rnd((L, Hkv, d), 48)
    full = prefill(q, k, v, B, 0.5, 0.4)
    ends = (40, 41, 100, 150)
    chunks = oracle.prefill_chunked(q, k, v, B, 0.5, ends, c=0.4)
    P = 0
    for end, ch in zip(ends, chunks):
        fresh = prefill(q[P:end], k[:end], v[:end], B, 0.5, 0.4, P=P)
        assert np.abs(ch["kbar"] - pool_keys(k[:end], B)).max() < 1e-12
        assert np.array_equal(ch["keep"], fresh["keep"])
        assert np.abs(ch["o"] - fresh["o"]).max() < 1e-12
        first_full = -(-P // B) * B
        last_full = end // B * B                    # rows of blocks complete within the chunk
        if last_full > first_full:
            assert np.abs(ch["o"][first_full - P:last_full - P] - full["o"][first_full:last_full]).max() < 1e-12
        P = end


def test_varlen_paged_batch_equals_per_sequence():
    import synth
    cfg = synth.config(5, Hq=4, Hkv=2, len_range=(150, 400), n_seqs=3, block=64, page_size=16)
    inp = synth.gen_paged(cfg)
    outs = oracle.prefill_varlen(inp.q, inp.cu_seqlens_q, inp.seqlens_k, inp.k_cache,
                                 inp.v_cache, inp.block_table.numpy(), 64, 4.0)
    for b in range(3):
        kb, vb = synth.unpage(inp, b)
        qb = inp.q[inp.cu_seqlens_q[b]:inp.cu_seqlens_q[b + 1]]
        L = int(inp.seqlens_k[b])
        ref = prefill(oracle.widen_bf16(qb), oracle.widen_bf16(kb), oracle.widen_bf16(vb),
                      64, 4.0, P=L - qb.shape[0])
        assert np.array_equal(outs[b]["keep"], ref["keep"])
        assert np.abs(outs[b]["o"] - ref["o"]).max() == 0.0


# --------------------------------------------------------------------------
# worked example derived by hand (tests/golden/tiny_hand.json)
# --------------------------------------------------------------------------
def test_hand_worked_example():
    with open(os.path.join(GOLDEN, "tiny_hand.json")) as f:
        g = json.load(f)
    w = [Fraction(x) for x in g["k_as_log"]]
    k = np.array([math.log(x) for x in w]).reshape(6, 1, 1)
    q = np.array(g["q"], dtype=np.float64).reshape(6, 1, 1)
    v = np.array(g["v"], dtype=np.float64).reshape(6, 1, 1)
    for case in g["cases"]:
        out = prefill(q, k, v, 2, case["tau"], 1.0)
        assert list(out["keep"][0, 2]) == case["keep_row2"]
        for t in range(6):
            assert abs(out["o"][t, 0, 0] - float(Fraction(case["o"][t]))) < 1e-13
            assert abs(out["lse"][0, t] - math.log(Fraction(case["lse_exp"][t]))) < 1e-13


# --------------------------------------------------------------------------
# P10: fp8 codec against torch's float8_e4m3fn
# --------------------------------------------------------------------------
def test_fp8_decode_all_codes_match_torch():
    codes = np.arange(256, dtype=np.uint8)
    ours = oracle.decode_e4m3(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan) and nan.sum() == 2
    assert np.array_equal(ours[~nan], ref[~nan])
    assert ours[~nan].max() == 448.0


def test_fp8_quantiser_rounds_to_nearest_code():
    import synth
    x = rnd((300, 16), 44) * np.array([1e-3, 1, 30, 1e3] * 4)[None, :]
    x[128:256] = 0.0                                   # an all-zero scale block
    codes, sc = synth.quantize_fp8(x)
    assert sc[1] == 1.0
    table = oracle.decode_e4m3(np.arange(256, dtype=np.uint8))
    finite = table[~np.isnan(table)]
    dec = oracle.decode_e4m3(codes.numpy())
    for t in range(0, 300, 7):
        s = float(sc[t // 128])
        for e in range(16):
            y = np.float32(x[t, e] / s)
            best = np.abs(finite - y).min()
            assert abs(dec[t, e] - y) == best


# --------------------------------------------------------------------------
# FLOP bookkeeping: dense count against a direct sum
# --------------------------------------------------------------------------
@pytest.mark.parametrize("P,L,B", [(0, 100, 16), (30, 100, 16)])
def test_flop_counts(P, L, B):
    d, Hq, Hkv = 8, 4, 2
    dense = oracle.dense_flops(P, L, d, Hq)
    assert dense == 4 * d * Hq * sum(t + 1 for t in range(P, L))
    i0, nq = oracle.query_blocks(P, L, B)
    keep = np.zeros((Hkv, nq, oracle.nblocks(L, B)), dtype=bool)
    for il in range(nq):
        keep[:, il, :i0 + il + 1] = True
    assert oracle.kept_flops(keep, P, L, B, d, Hq // Hkv) == dense
    assert oracle.correction_flops(keep, P, L, B, d, Hq // Hkv) == 0


def test_widen_fp8_position_offset():
    """Rows that start at position pos0 take the scales of their own
    128-position blocks: widening rows [P, T) with pos0 = P equals rows
    [P, T) of the widening from position 0, and each value is code * scale."""
    rng = np.random.default_rng(5)
    T, H, d, P = 300, 2, 4, 77
    codes = rng.integers(0, 256, size=(T, H, d), dtype=np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0                      # no NaN codes
    scales = rng.uniform(0.5, 2.0, size=(H, 3)).astype(np.float32)
    full = oracle.widen_fp8(codes, scales)
    part = oracle.widen_fp8(codes[P:], scales, pos0=P)
    assert np.array_equal(part, full[P:])
    t, h, e = 200, 1, 3                                    # position 200 lies in block 1
    assert full[t, h, e] == oracle.decode_e4m3(codes[t:t + 1, h:h + 1, e:e + 1])[0, 0, 0] * np.float64(scales[h, 1])


def test_query_blocks_without_present_rows():
    """Query blocks are the blocks holding present rows: a prefix that ends
    mid-block starts in that block, and a fully cached sequence has none (its
    prefill has no rows, no kept lists and no outputs)."""
    assert oracle.query_blocks(300, 1000, 128) == (2, 6)
    assert oracle.query_blocks(256, 257, 128) == (2, 1)
    assert oracle.query_blocks(700, 700, 128)[1] == 0
    rng = np.random.default_rng(1)
    k = rng.standard_normal((700, 1, 8))
    ref = prefill(np.zeros((0, 2, 8)), k, k, 128, 1.0, P=700)
    assert ref["keep"].shape == (1, 0, 6) and ref["o"].shape[0] == 0


# --------------------------------------------------------------------------
# Variants: per-query-head lists (no GQA union) and the block-score correction
# --------------------------------------------------------------------------
def walk_inputs(L, Hq, Hkv, d, seed, P=0):
    q = rnd((L - P, Hq, d), seed) + 0.8
    k = rnd((L, Hkv, d), seed + 1) + np.cumsum(rnd((L, Hkv, d), seed + 2, 0.6), axis=0)
    v = rnd((L, Hkv, d), seed + 3)
    return q, k, v


@pytest.mark.parametrize("P,tau", [(0, 0.3), (0, 1.0), (9, 0.5)])
def test_per_head_lists_union_is_the_group_list(P, tau):
    """The group's list (E4 with the union) is exactly the OR of its heads'
    own lists, each head's list is a subset of it, and per-head lists come
    out of an independent enumeration."""
    L, B, Hq, Hkv, d = 80, 8, 4, 2, 8
    q, k, v = walk_inputs(L, Hq, Hkv, d, 40, P)
    union = prefill(q, k, v, B, tau, 0.5, P=P, with_output=False)
    ph = prefill(q, k, v, B, tau, 0.5, P=P, with_output=False, variant="per_head")
    G = Hq // Hkv
    assert ph["keep"].shape[0] == Hq
    for g in range(Hkv):
        assert np.array_equal(union["keep"][g], ph["keep"][g * G:(g + 1) * G].any(axis=0))
    assert (union["keep"].sum() < ph["keep"].reshape(Hkv, G, *ph["keep"].shape[1:]).sum())  # heads differ
    enum = brute.select_enum(q, k, 0.5, P, L, B, G, tau, per_head=True)
    assert np.array_equal(ph["keep"], enum)


def test_per_head_lists_of_identical_heads_equal_the_union():
    L, B, d = 64, 8, 8
    q1 = rnd((L, 1, d), 44) + 0.7
    k = rnd((L, 1, d), 45) + np.cumsum(rnd((L, 1, d), 46, 0.5), axis=0)
    v = rnd((L, 1, d), 47)
    qG = np.repeat(q1, 4, axis=1)
    a = prefill(qG, k, v, B, 0.5, 0.3)
    b = prefill(qG, k, v, B, 0.5, 0.3, variant="per_head")
    for h in range(4):
        assert np.array_equal(b["keep"][h], a["keep"][0])
    assert np.abs(a["o"] - b["o"]).max() < 1e-12 and np.abs(a["lse"] - b["lse"]).max() < 1e-12


@pytest.mark.parametrize("P,tau", [(0, 0.3), (7, 1.0)])
def test_per_head_attend_matches_augmented_loops(P, tau):
    L, B, Hq, Hkv, d = 34, 4, 4, 2, 4
    q, k, v = walk_inputs(L, Hq, Hkv, d, 48, P)
    out = prefill(q, k, v, B, tau, 0.5, P=P, variant="per_head")
    o, lse = brute.attend_augmented(q, k, v, out["keep"], 0.5, P, L, B, Hq // Hkv)
    assert np.abs(out["o"] - o).max() < 1e-12 and np.abs(out["lse"] - lse).max() < 1e-12


@pytest.mark.parametrize("variant", ["per_head", "block_score"])
@pytest.mark.parametrize("tau", [-1.0, 0.3, 2.0])
def test_variants_exact_for_block_size_one(variant, tau):
    """With 1-token blocks a pruned block's pseudo-token is its token (and the
    block score is that token's logit), so every variant equals dense attention."""
    L, Hq, Hkv, d = 30, 4, 2, 8
    q, k, v = walk_inputs(L, Hq, Hkv, d, 52)
    out = prefill(q, k, v, 1, tau, 0.4, variant=variant)
    ref, lse = dense_numpy(q, k, v, 0.4)
    assert np.abs(out["o"] - ref).max() < 1e-12 and np.abs(out["lse"] - lse).max() < 1e-12


@pytest.mark.parametrize("tau", [-1.0, 0.5, 3.0])
def test_block_score_equals_mean_correction_for_block_constant_queries(tau):
    """When q is constant inside every query block, the block score of (i, j)
    is every row's own pseudo-token logit: the two corrections coincide (any
    K, V); with block-constant K and V too, both equal dense attention."""
    L, B, Hq, Hkv, d = 96, 8, 4, 2, 8
    nb = L // B
    qb = rnd((nb, Hq, d), 55) + 0.5
    q = np.repeat(qb, B, axis=0)
    _, k, v = walk_inputs(L, Hq, Hkv, d, 56)
    a = prefill(q, k, v, B, tau, 0.3)
    b = prefill(q, k, v, B, tau, 0.3, variant="block_score")
    assert np.abs(a["o"] - b["o"]).max() < 1e-12 and np.abs(a["lse"] - b["lse"]).max() < 1e-12
    kc = np.repeat(rnd((nb, Hkv, d), 57), B, axis=0)
    vc = np.repeat(rnd((nb, Hkv, d), 58), B, axis=0)
    c_ = prefill(q, kc, vc, B, tau, 0.3, variant="block_score")
    ref, lse = dense_numpy(q, kc, vc, 0.3)
    assert np.abs(c_["o"] - ref).max() < 1e-12 and np.abs(c_["lse"] - lse).max() < 1e-12


@pytest.mark.parametrize("P,tau", [(0, 0.3), (7, 1.0), (0, -1.0)])
def test_block_score_matches_augmented_loops(P, tau):
    """The block-score pseudo-token logit is the block pair's mean token logit
    (E2's closed form, summed pair by pair here) plus ln |J|."""
    L, B, Hq, Hkv, d = 34, 4, 4, 2, 4
    q, k, v = walk_inputs(L, Hq, Hkv, d, 60, P)
    out = prefill(q, k, v, B, tau, 0.5, P=P, variant="block_score")
    assert (~out["keep"]).any()
    o, lse = brute.attend_augmented(q, k, v, out["keep"], 0.5, P, L, B, Hq // Hkv, block_score=True)
    assert np.abs(out["o"] - o).max() < 1e-12 and np.abs(out["lse"] - lse).max() < 1e-12
    mean = prefill(q, k, v, B, tau, 0.5, P=P)
    assert np.abs(out["o"] - mean["o"]).max() > 1e-6     # a different correction on these inputs
