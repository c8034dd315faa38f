"""GPU parity: the HIP path through the C ABI against the fp64 CPU oracle.

Kept lists must match bit-exactly except blocks whose oracle estimate lies
within 1e-3 of the threshold; outputs (evaluated by the oracle under the
GPU's validated kept lists) within max-abs 2e-2 / mean-abs 2e-3 for bf16 and
6e-2 / 6e-3 for fp8; lse within a per-element bound derived from the data
(fp_testutil.lse_bound)."""
import math
import sys

import numpy as np
import pytest
import torch

import oracle
import synth
from fp_testutil import (TOL, check_csr_wellformed, check_lse, lse_bound, check_sched, compare_masks, compare_outputs,
                         csr_to_keep, fixed_sched_groups)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fp():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import block_sparse_long_estimate_amd as m
    m._native.load()
    return m


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def to_dev(inp):
    dev = torch.device("cuda:0")
    mv = lambda t: None if t is None else t.to(dev)
    return mv(inp.q), mv(inp.k), mv(inp.v), mv(inp.q_scale), mv(inp.k_scale), mv(inp.v_scale)


def run_fixed(fp, inp, tau, block):
    q, k, v, qs, ks, vs = to_dev(inp)
    out = fp.sparse_prefill(q, k, v, block, tau, q_scale=qs, k_scale=ks, v_scale=vs)
    torch.cuda.synchronize()
    return {kk: (vv.cpu() if isinstance(vv, torch.Tensor) else vv) for kk, vv in out.items()}


def widen(inp, b):
    if inp.q.dtype == torch.bfloat16:
        return [oracle.widen_bf16(t[b]) for t in (inp.q, inp.k, inp.v)]
    return [oracle.widen_fp8(t[b].numpy(), s[b].numpy())
            for t, s in ((inp.q, inp.q_scale), (inp.k, inp.k_scale), (inp.v, inp.v_scale))]


def check_fixed(fp, inp, tau, block, rows=None, kind="bf16", check_pooled=True):
    """Full comparison of one fixed-shape run. rows: per-sequence list of
    (g, il) to evaluate E6 on (None = all)."""
    out = run_fixed(fp, inp, tau, block)
    B, S, Hq = inp.q.shape[0], inp.q.shape[1], inp.q.shape[2]
    Hkv = inp.k.shape[2]
    nb = -(-S // block)
    c = 1 / math.sqrt(128)
    rp, ci = out["row_ptr"].numpy(), out["col_idx"].numpy()
    check_csr_wellformed(rp, ci, lambda r: r % nb)
    counts = np.diff(rp)
    esz = 2 if inp.q.dtype == torch.bfloat16 else 1
    check_sched(out["sched"].numpy(), counts, fixed_sched_groups(B, Hkv, nb, block, esz))
    stats = []
    for b in range(B):
        q, k, v = widen(inp, b)
        ref = oracle.prefill(q, k, v, block, tau, c, with_output=False)
        if check_pooled:
            for name in ("qbar", "kbar", "vbar"):
                g = out[name][b].numpy()
                r = ref[name]
                assert np.abs(g - r).max() <= 1e-5 * max(1.0, np.abs(r).max()), name
            sg, sr = out["scores"][b].numpy(), ref["S"]
            fin = np.isfinite(sr)
            assert np.array_equal(fin, np.isfinite(sg))
            assert np.abs(sg[fin] - sr[fin]).max() <= 2e-4 * max(1.0, np.abs(sr[fin]).max())
        keep = csr_to_keep(rp, ci, b * Hkv * nb, Hkv, nb, nb)
        ndiff, nband = compare_masks(keep, ref["keep"], ref["R"], tau)
        o_ref, lse_ref = oracle.attend(q, k, v, keep, ref["kbar"], ref["vbar"], c, block, 0,
                                       rows=None if rows is None else rows[b])
        mx, mean = compare_outputs(out["o"][b].float().numpy(), o_ref, kind)
        check_lse(out["lse"][b].numpy(), lse_ref,
                  lse_bound(q, k, keep, ref["kbar"], lse_ref, c, block, 0, rows=None if rows is None else rows[b],
                            kind=kind))
        frac = keep.sum() / (Hkv * nb * (nb + 1) / 2)
        stats.append((frac, ndiff, nband, mx, mean))
        say(f"  seq {b}: kept {frac:.3%}, mask diffs {ndiff} (band {nband}), max|err| {mx:.2e}, mean {mean:.2e}")
    return out, stats


# ---------------------------------------------------------------------------
def test_config1_full(fp):
    """S=2048, GQA 4:1, iid N(0,1), 64x64 blocks, tau=4 (every block expected kept)."""
    cfg = synth.config(1)
    say("config 1")
    _, stats = check_fixed(fp, synth.gen_fixed(cfg), cfg.tau, cfg.block)
    assert stats[0][0] == 1.0


@pytest.mark.parametrize("tau", [0.01, 0.05])
def test_config1_shape_low_tau(fp, tau):
    """Config 1's shape at tau values that actually prune."""
    cfg = synth.config(1, tau=tau)
    say(f"config 1 shape, tau={tau}")
    _, stats = check_fixed(fp, synth.gen_fixed(cfg), tau, cfg.block)
    assert stats[0][0] < 1.0


@pytest.mark.parametrize("S,block,tau", [(4096 + 77, 128, 2.0), (4096 + 77, 128, 4.0),
                                         (3000, 64, 2.0), (1024, 128, 1.0)])
def test_walk_pruning(fp, S, block, tau):
    """Random-walk keys with sink and planted blocks: real pruning, the
    correction path, a ragged last block."""
    cfg = synth.config(2, S=S, Hq=8, Hkv=2, block=block, tau=tau)
    say(f"walk S={S} block={block} tau={tau}")
    _, stats = check_fixed(fp, synth.gen_fixed(cfg), tau, block)
    assert stats[0][0] < 1.0


def test_batch_of_two_equals_single_runs(fp):
    cfg = synth.config(2, S=2048 + 5, Hq=8, Hkv=2, batch=2, tau=2.0)
    inp = synth.gen_fixed(cfg)
    out, _ = check_fixed(fp, inp, cfg.tau, cfg.block)
    for b in range(2):
        one = synth.FixedInputs(cfg, inp.q[b:b + 1], inp.k[b:b + 1], inp.v[b:b + 1])
        o1 = run_fixed(fp, one, cfg.tau, cfg.block)
        assert torch.equal(o1["o"][0], out["o"][b])
        assert torch.equal(o1["lse"][0], out["lse"][b])


@pytest.mark.parametrize("tau", [float("inf"), -1.0])
def test_tau_limits(fp, tau):
    """tau=inf keeps every block (dense causal attention); tau<0 keeps only
    the sink and diagonal blocks (everything else through the correction)."""
    cfg = synth.config(2, S=2048 + 64 + 3, Hq=8, Hkv=2, tau=tau)
    inp = synth.gen_fixed(cfg)
    say(f"tau limit {tau}")
    out, stats = check_fixed(fp, inp, tau, cfg.block)
    nb = -(-cfg.S // cfg.block)
    counts = np.diff(out["row_ptr"].numpy())
    if tau == float("inf"):
        assert stats[0][0] == 1.0
        # dense causal attention, float32 on the CPU
        q = inp.q[0].float().permute(1, 0, 2)
        k = inp.k[0].float().repeat_interleave(4, dim=1).permute(1, 0, 2)
        v = inp.v[0].float().repeat_interleave(4, dim=1).permute(1, 0, 2)
        ref = torch.nn.functional.scaled_dot_product_attention(q[None], k[None], v[None], is_causal=True)
        err = (out["o"][0].float().permute(1, 0, 2) - ref[0]).abs()
        assert err.max() <= TOL["bf16"][0] and err.mean() <= TOL["bf16"][1]
    else:
        exp = np.array([min(i, 1) + 1 for i in range(nb)] * cfg.Hkv)
        assert np.array_equal(counts, exp)


def test_caller_supplied_oracle_mask(fp):
    """fp_sparse_prefill accepts any valid kept list: feed the oracle's."""
    cfg = synth.config(2, S=3072 + 11, Hq=8, Hkv=2, tau=2.0)
    inp = synth.gen_fixed(cfg)
    q, k, v, _, _, _ = to_dev(inp)
    p = fp.make_problem(q, k, v, cfg.block)
    qbar, kbar, vbar, scores = fp.fp_block_scores(p, q, k, v)
    qn, kn, vn = widen(inp, 0)
    ref = oracle.prefill(qn, kn, vn, cfg.block, cfg.tau)
    Hkv, nq, nb = ref["keep"].shape
    rows = [np.nonzero(ref["keep"][g, il])[0] for g in range(Hkv) for il in range(nq)]
    row_ptr = np.concatenate([[0], np.cumsum([len(r) for r in rows])]).astype(np.int32)
    col_idx = np.concatenate(rows).astype(np.int32)
    o, lse = fp.fp_sparse_prefill(p, q, k, v, kbar, vbar, torch.from_numpy(row_ptr).cuda(),
                                  torch.from_numpy(col_idx).cuda(), None)
    torch.cuda.synchronize()
    compare_outputs(o[0].float().cpu().numpy(), ref["o"], "bf16")


def test_run_twice_is_bit_identical(fp):
    cfg = synth.config(2, S=4096, Hq=8, Hkv=2, tau=2.0)
    inp = synth.gen_fixed(cfg)
    a = run_fixed(fp, inp, cfg.tau, cfg.block)
    b = run_fixed(fp, inp, cfg.tau, cfg.block)
    for key in ("scores", "row_ptr", "sched", "o", "lse"):
        assert torch.equal(a[key], b[key]), key
    n = int(a["row_ptr"][-1])
    assert torch.equal(a["col_idx"][:n], b["col_idx"][:n])


# ---------------------------------------------------------------------------
# fp8
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("S,tau", [(2048 + 40, 2.0), (4096, 4.0)])
def test_fp8_walk(fp, S, tau):
    cfg = synth.config(4, S=S, Hq=8, Hkv=2, tau=tau)
    say(f"fp8 walk S={S} tau={tau}")
    check_fixed(fp, synth.gen_fixed(cfg), tau, cfg.block, kind="fp8")


@pytest.mark.parametrize("Hq,Hkv", [(32, 8), (48, 16)])
def test_fp8_pool_head_groups(fp, Hq, Hkv):
    """fp8 pooling works on groups of 32 heads per workgroup: 32 query heads
    fill one group (one token lane, no LDS reduction: the headline layer's
    case), 48 leave a partial second group of 16; 8 and 16 KV heads split
    the tokens over 4 and 2 lanes. Pooled rows, scores, kept lists and
    outputs are compared."""
    cfg = synth.config(4, S=1024 + 300, Hq=Hq, Hkv=Hkv, tau=2.0, seed=31 + Hq)
    say(f"fp8 pooling head groups {Hq}/{Hkv}")
    check_fixed(fp, synth.gen_fixed(cfg), cfg.tau, cfg.block, kind="fp8")


@pytest.mark.parametrize("Hq,Hkv", [(32, 8), (48, 16)])
def test_paged_fp8_pool_head_groups(fp, Hq, Hkv):
    """The same head groupings through the paged entry point (fp8 codes in
    64-token pages, cached prefixes)."""
    cfg = synth.config(5, Hq=Hq, Hkv=Hkv, n_seqs=2, len_range=(600, 1500), page_size=64, tau=2.0,
                       dtype="fp8", seed=41 + Hq)
    L, P = synth.paged_lengths(cfg)
    say(f"paged fp8 pooling head groups {Hq}/{Hkv}: L={L.tolist()} P={P.tolist()}")
    check_paged(fp, synth.gen_paged(cfg, (L, P)), cfg.tau)


def test_fp8_block64_iid(fp):
    cfg = synth.config(1, S=1024 + 9, dtype="fp8", tau=0.05)
    say("fp8 iid block 64")
    check_fixed(fp, synth.gen_fixed(cfg), cfg.tau, cfg.block, kind="fp8")


# ---------------------------------------------------------------------------
# paged varlen
# ---------------------------------------------------------------------------
def run_paged(fp, inp, tau, softmax_scale=0.0):
    dev = torch.device("cuda:0")
    q, kc, vc, bt = inp.q.to(dev), inp.k_cache.to(dev), inp.v_cache.to(dev), inp.block_table.to(dev)
    sc = [None if t is None else t.to(dev) for t in (inp.q_scale, inp.k_scale, inp.v_scale)]
    vp = fp.make_varlen_problem(q, inp.cu_seqlens_q, inp.seqlens_k, kc, bt, inp.cfg.block,
                                softmax_scale=softmax_scale)
    o, lse, rp, ci = fp.fp_sparse_prefill_paged(vp, q, kc, vc, bt, tau, q_scale=sc[0], k_scale=sc[1],
                                                v_scale=sc[2])
    torch.cuda.synchronize()
    return o.cpu(), lse.cpu(), rp.cpu().numpy(), ci.cpu().numpy()


def check_paged(fp, inp, tau, sample_rows=None, softmax_scale=0.0):
    o, lse, rp, ci = run_paged(fp, inp, tau, softmax_scale)
    cfg = inp.cfg
    c = softmax_scale if softmax_scale > 0 else 1 / math.sqrt(128)
    kind = "fp8" if inp.q.dtype == torch.uint8 else "bf16"
    scales = dict(q_scale=inp.q_scale, k_scale=inp.k_scale, v_scale=inp.v_scale)
    refs = oracle.prefill_varlen(inp.q, inp.cu_seqlens_q, inp.seqlens_k, inp.k_cache, inp.v_cache,
                                 inp.block_table.numpy(), cfg.block, tau, c, with_output=False, **scales)
    row0 = 0
    for b, ref in enumerate(refs):
        L, P = int(inp.seqlens_k[b]), int(inp.prefix[b])
        Hkv, nq, nb = ref["keep"].shape
        if nq == 0:                             # no new rows: no kept-list rows, no outputs
            assert L == P
            continue
        keep = csr_to_keep(rp, ci, row0, Hkv, nq, nb)
        for r in range(Hkv * nq):
            cols = ci[rp[row0 + r]:rp[row0 + r + 1]]
            assert cols[0] == 0 and cols[-1] == ref["i0"] + r % nq and np.all(np.diff(cols) > 0)
        ndiff, nband = compare_masks(keep, ref["keep"], ref["R"], tau)
        lo, hi = int(inp.cu_seqlens_q[b]), int(inp.cu_seqlens_q[b + 1])
        qw, kw, vw, _ = oracle.varlen_sequence(inp.q, inp.cu_seqlens_q, inp.seqlens_k, inp.k_cache,
                                               inp.v_cache, inp.block_table.numpy(), b, **scales)
        rows = None if sample_rows is None else sample_rows(Hkv, nq)
        o_ref, lse_ref = oracle.attend(qw, kw, vw, keep, ref["kbar"], ref["vbar"], c, cfg.block, P, rows=rows)
        mx, mean = compare_outputs(o[lo:hi].float().numpy(), o_ref, kind)
        check_lse(lse[:, lo:hi].numpy(), lse_ref, lse_bound(qw, kw, keep, ref["kbar"], lse_ref, c, cfg.block, P,
                                                            rows=rows, kind=kind))
        say(f"  seq {b}: L={L} P={P} kept {keep.sum() / max(1, (np.tril(np.ones((nq, nb)), ref['i0']).sum()) * Hkv):.2%} "
            f"diffs {ndiff} (band {nband}) max|err| {mx:.2e} mean {mean:.2e}")
        row0 += Hkv * nq
    assert row0 == len(rp) - 1


@pytest.mark.parametrize("page,block", [(64, 128), (16, 128), (256, 128), (32, 64), (128, 64)])
def test_paged_varlen_small(fp, page, block):
    """Pages smaller than, equal to and larger than the block (a tile then
    starts mid-page), for both block sizes."""
    cfg = synth.config(5, Hq=8, Hkv=2, n_seqs=4, len_range=(300, 3500), page_size=page, block=block, tau=2.0)
    L, P = synth.paged_lengths(cfg)
    P[0] = 0                                    # one sequence without a cached prefix
    say(f"paged varlen page={page} block={block}: L={L.tolist()} P={P.tolist()}")
    check_paged(fp, synth.gen_paged(cfg, (L, P)), cfg.tau)


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
def test_paged_edge_sequences(fp, dtype):
    """A batch holding a sequence with no new rows (all cached), a one-token
    sequence, a cached prefix that ends on a block boundary, one that leaves a
    single new row, and a sequence one token past a block boundary."""
    cfg = synth.config(5, Hq=8, Hkv=2, n_seqs=5, tau=2.0, dtype=dtype, page_size=64)
    L = np.array([700, 1, 1024 + 300, 900, 2049])
    P = np.array([700, 0, 1024, 899, 0])
    say(f"paged edge sequences {dtype}: L={L.tolist()} P={P.tolist()}")
    check_paged(fp, synth.gen_paged(cfg, (L, P)), cfg.tau)


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
def test_paged_all_sequences_cached(fp, dtype):
    """A batch whose sequences are all fully cached has no present rows: the
    call writes row_ptr = [0] (no kept-list rows) and nothing else."""
    cfg = synth.config(5, Hq=8, Hkv=2, n_seqs=3, tau=2.0, dtype=dtype, page_size=64)
    L = np.array([700, 129, 2048])
    say(f"paged, every sequence cached {dtype}: L={L.tolist()}")
    inp = synth.gen_paged(cfg, (L, L.copy()))
    dev = torch.device("cuda:0")
    q, kc, vc, bt = inp.q.to(dev), inp.k_cache.to(dev), inp.v_cache.to(dev), inp.block_table.to(dev)
    sc = [None if t is None else t.to(dev) for t in (inp.q_scale, inp.k_scale, inp.v_scale)]
    vp = fp.make_varlen_problem(q, inp.cu_seqlens_q, inp.seqlens_k, kc, bt, cfg.block)
    assert vp.rows == 0 and q.shape[0] == 0
    o, lse, rp, ci = fp.fp_sparse_prefill_paged(vp, q, kc, vc, bt, cfg.tau, q_scale=sc[0], k_scale=sc[1],
                                                v_scale=sc[2])
    torch.cuda.synchronize()
    assert rp.shape == (1,) and int(rp.cpu()[0]) == 0
    assert o.shape[0] == 0 and lse.shape[1] == 0


@pytest.mark.parametrize("Hq,Hkv,block", [(8, 8, 128), (6, 2, 128), (16, 1, 64), (6, 2, 64)])
@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
def test_paged_gqa_ratios(fp, Hq, Hkv, block, dtype):
    """The paged path at G = 1, 3 and 16: with G = 3 a query block packs 384
    (block 128) or 192 (block 64) rows, so a slice is left partly empty."""
    cfg = synth.config(5, Hq=Hq, Hkv=Hkv, n_seqs=3, len_range=(200, 2500), page_size=32, block=block, tau=2.0,
                       dtype=dtype, seed=17 + Hq + Hkv)
    L, P = synth.paged_lengths(cfg)
    say(f"paged GQA {Hq}/{Hkv} block={block} {dtype}: L={L.tolist()} P={P.tolist()}")
    check_paged(fp, synth.gen_paged(cfg, (L, P)), cfg.tau)


@pytest.mark.parametrize("page,block", [(64, 128), (32, 64), (256, 128)])
def test_paged_varlen_small_fp8(fp, page, block):
    """fp8-e4m3 codes in the paged cache and packed queries, one scale per 128
    positions of each sequence (cached prefixes start mid-block)."""
    cfg = synth.config(5, Hq=8, Hkv=2, n_seqs=4, len_range=(300, 3500), page_size=page, block=block, tau=2.0,
                       dtype="fp8", seed=15)
    L, P = synth.paged_lengths(cfg)
    P[1] = 0
    say(f"paged varlen fp8 page={page} block={block}: L={L.tolist()} P={P.tolist()}")
    check_paged(fp, synth.gen_paged(cfg, (L, P)), cfg.tau)


@pytest.mark.parametrize("tau", [1.0, 3.0])
@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
def test_no_correction_variant(fp, tau, dtype):
    """The ablation without the mean correction, against the oracle's variant
    under the GPU's kept lists; the kept lists are those of the default run."""
    cfg = synth.config(2, S=4096 + 77, Hq=8, Hkv=2, seed=61, tau=tau, dtype=dtype)
    inp = synth.gen_fixed(cfg)
    dev = torch.device("cuda:0")
    mv = lambda t: None if t is None else t.to(dev)
    q, k, v = (t.to(dev) for t in (inp.q, inp.k, inp.v))
    sc = dict(q_scale=mv(inp.q_scale), k_scale=mv(inp.k_scale), v_scale=mv(inp.v_scale))
    a = fp.sparse_prefill(q, k, v, 128, tau, **sc)
    b = fp.sparse_prefill(q, k, v, 128, tau, correction=False, **sc)
    torch.cuda.synchronize()
    assert torch.equal(a["row_ptr"], b["row_ptr"])
    S, Hkv = cfg.S, cfg.Hkv
    nb = -(-S // 128)
    rp, ci = b["row_ptr"].cpu().numpy(), b["col_idx"].cpu().numpy()
    keep = csr_to_keep(rp, ci, 0, Hkv, nb, nb)
    assert (~keep[np.tril(np.ones((nb, nb), dtype=bool))[None].repeat(Hkv, 0)]).any()   # real pruning
    qd, kd, vd = widen(inp, 0)
    c = 1 / math.sqrt(128)
    ref = oracle.prefill(qd, kd, vd, 128, tau, c, with_output=False)
    o_ref, lse_ref = oracle.attend(qd, kd, vd, keep, ref["kbar"], ref["vbar"], c, 128, 0, correction=False)
    say(f"no-correction tau={tau} {dtype}")
    compare_outputs(b["o"][0].float().cpu().numpy(), o_ref, dtype)
    check_lse(b["lse"][0].cpu().numpy(), lse_ref,
              lse_bound(qd, kd, keep, ref["kbar"], lse_ref, c, 128, 0, correction=False, kind=dtype))
    assert not torch.equal(a["o"], b["o"])          # the correction changes the result


@pytest.mark.parametrize("L,page", [(3000, 64), (3000, 256), (33000, 16)])
def test_paged_equals_contiguous(fp, L, page):
    """A shuffled block table gives bit-identical results to contiguous storage.
    Pages of 256 tokens hold two 128-key tiles each (a tile starts mid-page);
    33000 tokens in 16-token pages need 2063 page ids, more than the kernel
    stages in LDS, so its tiles take the block-table path."""
    cfg = synth.config(5, Hq=8, Hkv=2, n_seqs=1, tau=2.0, page_size=page)
    say(f"paged == contiguous: L={L} page={page}")
    inp = synth.gen_paged(cfg, (np.array([L]), np.array([0])))
    o, lse, rp, ci = run_paged(fp, inp, cfg.tau)
    k, v = synth.unpage(inp, 0)
    fixed = synth.FixedInputs(cfg, inp.q[None], k[None], v[None])
    out = run_fixed(fp, fixed, cfg.tau, cfg.block)
    assert np.array_equal(rp, out["row_ptr"].numpy())
    assert torch.equal(o, out["o"][0])
    assert torch.equal(lse, out["lse"][0])


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
def test_paged_interleaved_kv_cache(fp, dtype):
    """K and V pages interleaved in one device tensor [pages, 2, page, Hkv, 128]
    (k_cache = cache[:, 0], v_cache = cache[:, 1], page stride twice a page):
    bit-identical to separate contiguous caches."""
    cfg = synth.config(5, Hq=8, Hkv=2, n_seqs=3, len_range=(300, 3000), tau=2.0, dtype=dtype)
    inp = synth.gen_paged(cfg)
    o, lse, rp, ci = run_paged(fp, inp, cfg.tau)
    dev = torch.device("cuda:0")
    cache = torch.stack([inp.k_cache, inp.v_cache], dim=1).to(dev)
    kc, vc = cache[:, 0], cache[:, 1]
    assert kc.stride(0) == 2 * inp.k_cache.stride(0) and kc.data_ptr() != vc.data_ptr()
    q, bt = inp.q.to(dev), inp.block_table.to(dev)
    sc = {n: None if t is None else t.to(dev)
          for n, t in (("q_scale", inp.q_scale), ("k_scale", inp.k_scale), ("v_scale", inp.v_scale))}
    vp = fp.make_varlen_problem(q, inp.cu_seqlens_q, inp.seqlens_k, kc, bt, cfg.block)
    o2, lse2, rp2, ci2 = fp.fp_sparse_prefill_paged(vp, q, kc, vc, bt, cfg.tau, **sc)
    torch.cuda.synchronize()
    rp2, ci2 = rp2.cpu().numpy(), ci2.cpu().numpy()
    assert np.array_equal(rp, rp2) and np.array_equal(ci[:rp[-1]], ci2[:rp[-1]])
    assert torch.equal(o, o2.cpu()) and torch.equal(lse, lse2.cpu())
    say(f"paged ({dtype}): interleaved K/V cache views bit-identical to separate caches")


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
def test_paged_unused_table_entries_not_read(fp, dtype):
    """Block-table entries past a sequence's last page point at an extra page
    of NaNs (a valid page id): results stay bit-identical, so no unused entry
    is followed."""
    cfg = synth.config(5, Hq=8, Hkv=2, n_seqs=3, len_range=(300, 3000), page_size=64, tau=2.0, dtype=dtype,
                       seed=29)
    inp = synth.gen_paged(cfg)
    o, lse, rp, ci = run_paged(fp, inp, cfg.tau)
    n_pages, page = inp.k_cache.shape[0], inp.k_cache.shape[1]
    nan_page = torch.full_like(inp.k_cache[:1], 0x7F) if dtype == "fp8" else torch.full_like(inp.k_cache[:1],
                                                                                               float("nan"))
    kc, vc = torch.cat([inp.k_cache, nan_page]), torch.cat([inp.v_cache, nan_page])
    bt = inp.block_table.clone()
    for b, L in enumerate(inp.seqlens_k):
        bt[b, -(-int(L) // page):] = n_pages
    assert (bt == n_pages).any()
    poisoned = synth.PagedInputs(inp.cfg, inp.q, kc, vc, bt, inp.cu_seqlens_q, inp.seqlens_k, inp.prefix, inp.meta,
                                 inp.q_scale, inp.k_scale, inp.v_scale)
    o2, lse2, rp2, ci2 = run_paged(fp, poisoned, cfg.tau)
    assert np.array_equal(rp, rp2) and np.array_equal(ci[:rp[-1]], ci2[:rp[-1]])
    assert torch.equal(o, o2) and torch.equal(lse, lse2)
    say(f"paged ({dtype}): unused block-table entries pointing at a NaN page change nothing")


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
def test_paged_slots_past_sequence_end_not_read(fp, dtype):
    """The slots of each sequence's last page past its length hold NaN (fp8:
    NaN codes): results stay bit-identical."""
    cfg = synth.config(5, Hq=8, Hkv=2, n_seqs=3, len_range=(300, 3000), page_size=64, tau=2.0, dtype=dtype,
                       seed=31)
    inp = synth.gen_paged(cfg)
    o, lse, rp, ci = run_paged(fp, inp, cfg.tau)
    page = inp.k_cache.shape[1]
    kc, vc = inp.k_cache.clone(), inp.v_cache.clone()
    poisoned_slots = 0
    for b, L in enumerate(inp.seqlens_k):
        L = int(L)
        if L % page:
            last = int(inp.block_table[b, (L - 1) // page])
            for c in (kc, vc):
                if dtype == "fp8":
                    c[last, L % page:] = 0x7F
                else:
                    c[last, L % page:] = float("nan")
            poisoned_slots += page - L % page
    assert poisoned_slots > 0
    poisoned = synth.PagedInputs(inp.cfg, inp.q, kc, vc, inp.block_table, inp.cu_seqlens_q, inp.seqlens_k,
                                 inp.prefix, inp.meta, inp.q_scale, inp.k_scale, inp.v_scale)
    o2, lse2, rp2, ci2 = run_paged(fp, poisoned, cfg.tau)
    assert np.array_equal(rp, rp2) and np.array_equal(ci[:rp[-1]], ci2[:rp[-1]])
    assert torch.equal(o, o2) and torch.equal(lse, lse2)
    say(f"paged ({dtype}): {poisoned_slots} NaN slots past the sequence ends change nothing")


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
def test_paged_softmax_scale(fp, dtype):
    """softmax_scale given explicitly (0.05, not 1/sqrt(d)) on the paged path:
    scores, kept lists and outputs against the oracle at the same scale."""
    cfg = synth.config(5, Hq=8, Hkv=2, n_seqs=3, len_range=(300, 3000), page_size=64, tau=2.0, dtype=dtype,
                       seed=37)
    L, P = synth.paged_lengths(cfg)
    say(f"paged softmax_scale 0.05 {dtype}: L={L.tolist()} P={P.tolist()}")
    check_paged(fp, synth.gen_paged(cfg, (L, P)), cfg.tau, softmax_scale=0.05)


def test_paged_fp8_equals_contiguous_fp8(fp):
    """The same fp8 codes and scales through the paged entry point (shuffled
    64-token pages) and the fixed-shape one: bit-identical results."""
    L = 5000 + 37
    cfg = synth.config(5, Hq=8, Hkv=2, n_seqs=1, tau=2.0, dtype="fp8")
    say(f"paged fp8 == contiguous fp8: L={L}")
    inp = synth.gen_paged(cfg, (np.array([L]), np.array([0])))
    o, lse, rp, ci = run_paged(fp, inp, cfg.tau)
    k, v = synth.unpage(inp, 0)
    nsb = -(-L // 128)
    fixed = synth.FixedInputs(cfg, inp.q[None], k[None], v[None], inp.q_scale[:, :, :nsb].contiguous(),
                              inp.k_scale[:, :, :nsb].contiguous(), inp.v_scale[:, :, :nsb].contiguous())
    out = run_fixed(fp, fixed, cfg.tau, cfg.block)
    assert np.array_equal(rp, out["row_ptr"].numpy())
    assert torch.equal(o, out["o"][0])
    assert torch.equal(lse, out["lse"][0])

