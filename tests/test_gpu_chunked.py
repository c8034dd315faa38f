"""GPU: chunked prefill through the pooled-KV cache (fp_sparse_prefill_paged_cached).

One sequence is prefilled in three chunks: each call's kept lists, outputs and
lse must equal, bit for bit, the plain paged entry point's on the same call
(which pools every key afresh); rows of query blocks complete within a chunk
must equal the one-shot prefill's rows bit for bit; the kept lists and outputs
must match the oracle's chunked prefill (pooled means carried across chunks)
to the usual parity bar; and the cache must hold the block means after the
last chunk. A batch whose sequences advance by different chunks is checked
call by call against the plain entry point."""
import math
import sys

import numpy as np
import pytest
import torch

import oracle
import synth
from fp_testutil import check_csr_wellformed, compare_masks, compare_outputs, csr_to_keep

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


def whole_sequence(L, page, block, dtype, seed=7, Hq=8, Hkv=2):
    """One sequence of L tokens, every row a query (P = 0), in a shuffled page cache."""
    cfg = synth.config(5, Hq=Hq, Hkv=Hkv, n_seqs=1, block=block, page_size=page, dtype=dtype, seed=seed)
    return synth.gen_paged(cfg, (np.array([L]), np.array([0])))


def call(fp, inp, dev, rows, ends_k, cached=None, tau=4.0):
    """One paged call over the sequences of inp: sequence b presents query rows
    rows[b] = (P_b, L_b) and sees keys [0, L_b). cached: (kbar_cache, vbar_cache)
    or None for the plain entry point."""
    q_parts, cu = [], [0]
    qs = inp.q.to(dev)
    off = np.concatenate([[0], np.cumsum(inp.seqlens_k)])   # rows of the whole-sequence q per sequence
    for b, (P, L) in enumerate(rows):
        q_parts.append(qs[off[b] + P:off[b] + L])
        cu.append(cu[-1] + L - P)
    q = torch.cat(q_parts).contiguous() if cu[-1] else torch.empty((0,) + tuple(qs.shape[1:]), dtype=qs.dtype,
                                                                       device=dev)
    cu = np.array(cu, dtype=np.int32)
    lk = np.array([L for _, L in rows], dtype=np.int32)
    kc, vc, bt = inp.k_cache.to(dev), inp.v_cache.to(dev), inp.block_table.to(dev)
    sc = [None if t is None else t.to(dev) for t in (inp.q_scale, inp.k_scale, inp.v_scale)]
    vp = fp.make_varlen_problem(q, cu, lk, kc, bt, inp.cfg.block)
    if cached is None:
        out = fp.fp_sparse_prefill_paged(vp, q, kc, vc, bt, tau, q_scale=sc[0], k_scale=sc[1], v_scale=sc[2])
    else:
        out = fp.fp_sparse_prefill_paged_cached(vp, q, kc, vc, bt, cached[0], cached[1], tau, q_scale=sc[0],
                                                k_scale=sc[1], v_scale=sc[2])
    torch.cuda.synchronize()
    o, lse, rp, ci = out
    n = int(rp[-1])
    return o.cpu(), lse.cpu(), rp.cpu().numpy(), ci[:n].cpu().numpy(), cu


def new_cache(fp, inp, dev):
    slots = fp.pooled_kv_slots(inp.k_cache, inp.cfg.block)
    shape = (slots, inp.cfg.Hkv, 128)
    # NaN-filled: a slot read before it was written would poison the outputs
    return (torch.full(shape, float("nan"), device=dev), torch.full(shape, float("nan"), device=dev))


CASES = [
    # L, chunk ends, page, block, dtype
    (5000, (1500, 3000, 5000), 64, 128, "bf16"),
    (4173, (1024, 2100, 4173), 256, 128, "bf16"),
    (3000, (700, 1601, 3000), 16, 64, "bf16"),
    (3500, (1280, 2600, 3500), 64, 128, "fp8"),
]


@pytest.mark.parametrize("L,ends,page,block,dtype", CASES,
                         ids=[f"L{c[0]}-{len(c[1])}chunks-p{c[2]}-b{c[3]}-{c[4]}" for c in CASES])
def test_three_chunks_equal_uncached_one_shot_and_oracle(fp, L, ends, page, block, dtype):
    dev = torch.device("cuda:0")
    say(f"chunked prefill L={L} ends={ends} page={page} block={block} {dtype}")
    inp = whole_sequence(L, page, block, dtype)
    tau, c, B = 4.0, 1 / math.sqrt(128), block
    kind = dtype
    cache = new_cache(fp, inp, dev)
    o1, lse1, rp1, ci1, _ = call(fp, inp, dev, [(0, L)], None, tau=tau)       # one-shot
    keep1 = csr_to_keep(rp1, ci1, 0, inp.cfg.Hkv, -(-L // B), -(-L // B))
    scales = dict(q_scale=inp.q_scale, k_scale=inp.k_scale, v_scale=inp.v_scale)
    qw, kw, vw, _ = oracle.varlen_sequence(inp.q, inp.cu_seqlens_q, inp.seqlens_k, inp.k_cache, inp.v_cache,
                                           inp.block_table.numpy(), 0, **scales)
    refs = oracle.prefill_chunked(qw, kw, vw, B, tau, ends, c=c, with_output=False)
    P = 0
    for n, (E, ref) in enumerate(zip(ends, refs)):
        o, lse, rp, ci, _ = call(fp, inp, dev, [(P, E)], None, cached=cache, tau=tau)
        o0, lse0, rp0, ci0, _ = call(fp, inp, dev, [(P, E)], None, tau=tau)
        # the same call without the cache: identical kept lists, outputs and lse
        assert np.array_equal(rp, rp0) and np.array_equal(ci, ci0)
        assert torch.equal(o, o0) and torch.equal(lse, lse0), f"chunk {n}: cached != uncached"
        Hkv, nq, nb = ref["keep"].shape
        i0 = P // B
        assert len(rp) == Hkv * nq + 1
        check_csr_wellformed(rp, ci, lambda r: i0 + r % nq)
        keep = csr_to_keep(rp, ci, 0, Hkv, nq, nb)
        ndiff, nband = compare_masks(keep, ref["keep"], ref["R"], tau)
        # rows of query blocks complete within the chunk equal the one-shot rows
        full = [i for i in range(i0, i0 + nq) if i * B >= P and (i + 1) * B <= E]
        if full:
            a, z = full[0], full[-1] + 1
            assert np.array_equal(keep[:, a - i0:z - i0], keep1[:, a:z, :nb])
            assert torch.equal(o[a * B - P:z * B - P], o1[a * B:z * B]), f"chunk {n}: rows differ from one-shot"
            assert torch.equal(lse[:, a * B - P:z * B - P], lse1[:, a * B:z * B])
        o_ref, _ = oracle.attend(qw[P:E], kw[:E], vw[:E], keep, ref["kbar"], ref["vbar"], c, B, P)
        mx, mean = compare_outputs(o.float().numpy(), o_ref, kind)
        say(f"  chunk {n}: rows [{P}, {E}) diffs {ndiff} (band {nband}) full blocks {len(full)} "
            f"max|err| {mx:.2e} mean {mean:.2e}")
        P = E
    # the cache holds every complete block's means (slot = page of its last token)
    spp = max(1, page // B)
    bt = inp.block_table.numpy()[0]
    kref, vref = oracle.pool_keys(kw, B), oracle.pool_keys(vw, B)
    kc, vc = cache[0].cpu().numpy(), cache[1].cpu().numpy()
    for j in range(L // B):
        e = (j + 1) * B - 1
        slot = int(bt[e // page]) * spp + (e % page) // B
        for got, want in ((kc[slot], kref[:, j]), (vc[slot], vref[:, j])):
            assert np.abs(got - want).max() <= 1e-5 * (1 + np.abs(want).max())
    # the cache is what the call reads: with its slots zeroed the last chunk changes
    cache[0].zero_(); cache[1].zero_()
    o, _, _, _, _ = call(fp, inp, dev, [(ends[-2], L)], None, cached=cache, tau=tau)
    o0, _, _, _, _ = call(fp, inp, dev, [(ends[-2], L)], None, tau=tau)
    assert not torch.equal(o, o0)


def test_batch_advancing_by_different_chunks(fp):
    """Three sequences prefilled together, each cut at its own points; in some
    calls a sequence presents no rows (it neither reads nor writes the cache).
    Every call equals the plain entry point on the same call."""
    dev = torch.device("cuda:0")
    cfg = synth.config(5, Hq=8, Hkv=2, n_seqs=3, block=128, page_size=32, dtype="bf16", seed=11)
    Ls = np.array([3000, 1800, 4500])
    inp = synth.gen_paged(cfg, (Ls, np.zeros(3, dtype=np.int64)))
    cuts = [(900, 900, 2200, 3000), (1800, 1800, 1800, 1800), (128, 1500, 3500, 4500)]
    cache = new_cache(fp, inp, dev)
    prev = [0, 0, 0]
    for n in range(4):
        rows = [(prev[b], cuts[b][n]) for b in range(3)]
        # a sequence with no new rows still needs L >= 1 keys: keep its last chunk's end
        o, lse, rp, ci, cu = call(fp, inp, dev, rows, None, cached=cache)
        o0, lse0, rp0, ci0, _ = call(fp, inp, dev, rows, None)
        say(f"  call {n}: rows {rows} kept {len(ci)}")
        assert np.array_equal(rp, rp0) and np.array_equal(ci, ci0)
        assert torch.equal(o, o0) and torch.equal(lse, lse0), f"call {n}: cached != uncached"
        prev = [cuts[b][n] for b in range(3)]
