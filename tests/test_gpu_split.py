"""GPU: split rows for problems too small to fill the chip (FP_SPLIT_SMALL_GRIDS).

With the split, each (row, slice) of a problem of at most 128 work units runs
as several workgroups over consecutive parts of its tile sequence, and a merge
pass combines their partial results. The kept lists do not change (the split
is E6 only); o and lse must meet the oracle at the usual parity bar and the
data-derived lse bound, stay within rounding of the unsplit run, and the
allocation-free entry point must give the workspace entry's results bit for
bit under the same split."""
import math
import sys

import numpy as np
import pytest
import torch

import oracle
import synth
from fp_testutil import check_lse, compare_masks, compare_outputs, csr_to_keep, lse_bound

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


def widen(inp, b):
    if inp.q.dtype == torch.bfloat16:
        return [oracle.widen_bf16(t[b]) for t in (inp.q, inp.k, inp.v)]
    return [oracle.widen_fp8(t[b].numpy(), s[b].numpy())
            for t, s in ((inp.q, inp.q_scale), (inp.k, inp.k_scale), (inp.v, inp.v_scale))]


def units(Hq, Hkv, S, block, batch=1):
    rows = batch * Hkv * -(-S // block)
    return -(-rows // 8) * 8 * -(-(Hq // Hkv) * block // 256)


CASES = [
    # config id, overrides, variant
    (1, dict(), "mean"),                                          # S=2048, 4/1, 64-token blocks: 8 parts
    (1, dict(tau=0.05), "mean"),
    (2, dict(S=1500, Hq=8, Hkv=2, tau=1.0), "mean"),
    (2, dict(S=700, Hq=16, Hkv=1, tau=2.0, block=64), "mean"),
    (2, dict(S=1029, Hq=4, Hkv=1, tau=1.0, batch=2), "mean"),
    (2, dict(S=1500, Hq=8, Hkv=2, tau=1.0), "none"),
    (2, dict(S=1500, Hq=8, Hkv=2, tau=1.0), "per_head"),
    (2, dict(S=1500, Hq=8, Hkv=2, tau=1.0), "block_score"),
    (2, dict(S=8192, Hq=1, Hkv=1, tau=float("inf"), block=64), "mean"),  # a part starting at tile 64 of 128
    (4, dict(S=2088, Hq=8, Hkv=2, tau=2.0), "mean"),              # fp8
    (4, dict(S=1000, Hq=4, Hkv=1, tau=1.0, block=64), "mean"),
]


@pytest.mark.parametrize("cid,kw,variant", CASES, ids=[f"cfg{c[0]}-{'-'.join(f'{k}{v}' for k, v in c[1].items())}-{c[2]}"
                                                       for c in CASES])
def test_split_rows_against_oracle_and_unsplit(fp, cid, kw, variant):
    cfg = synth.config(cid, **kw)
    kind = "fp8" if cid == 4 else "bf16"
    inp = synth.gen_fixed(cfg)
    say(f"split rows: config {cid} {kw} {variant} ({units(cfg.Hq, cfg.Hkv, cfg.S, cfg.block, cfg.batch)} units)")
    assert units(cfg.Hq, cfg.Hkv, cfg.S, cfg.block, cfg.batch) <= 128
    dev = torch.device("cuda:0")
    mv = lambda t: None if t is None else t.to(dev)
    q, k, v = mv(inp.q), mv(inp.k), mv(inp.v)
    sc = dict(q_scale=mv(inp.q_scale), k_scale=mv(inp.k_scale), v_scale=mv(inp.v_scale))
    one = fp.sparse_prefill(q, k, v, cfg.block, cfg.tau, variant=variant, **sc)
    spl = fp.sparse_prefill(q, k, v, cfg.block, cfg.tau, variant=variant, split_small=True, **sc)
    torch.cuda.synchronize()
    # the split changes E6 only
    assert torch.equal(one["row_ptr"], spl["row_ptr"])
    n = int(one["row_ptr"][-1])
    assert torch.equal(one["col_idx"][:n], spl["col_idx"][:n])
    # within rounding of the unsplit run (different summation order)
    d = (one["o"].float() - spl["o"].float()).abs()
    assert float(d.max()) <= (2e-2 if kind == "fp8" else 8e-3), float(d.max())
    assert float((one["lse"] - spl["lse"]).abs().max()) <= 1e-3
    # against the oracle, under the kept lists the GPU chose
    c = 1 / math.sqrt(128)
    rp, ci = spl["row_ptr"].cpu().numpy(), spl["col_idx"].cpu().numpy()
    per_head = variant == "per_head"
    H = cfg.Hq if per_head else cfg.Hkv
    nb = -(-cfg.S // cfg.block)
    for b in range(cfg.batch):
        qn, kn, vn = widen(inp, b)
        ref = oracle.prefill(qn, kn, vn, cfg.block, cfg.tau, c, with_output=False, variant=variant)
        keep = csr_to_keep(rp, ci, b * H * nb, H, nb, nb)
        compare_masks(keep, ref["keep"], ref["R"], cfg.tau)
        o_ref, lse_ref = oracle.attend(qn, kn, vn, keep, ref["kbar"], ref["vbar"], c, cfg.block, 0,
                                       correction=variant != "none",
                                       block_scores=ref["S"] if variant == "block_score" else None)
        mx, mean = compare_outputs(spl["o"][b].float().cpu().numpy(), o_ref, kind)
        if variant in ("mean", "none"):
            check_lse(spl["lse"][b].cpu().numpy(), lse_ref,
                      lse_bound(qn, kn, keep, ref["kbar"], lse_ref, c, cfg.block, 0, kind=kind,
                                correction=variant != "none"))
        say(f"  seq {b}: max|err| {mx:.2e} mean {mean:.2e}; split vs unsplit max|d| {float(d.max()):.2e}")


def test_split_noalloc_equals_workspace_entry(fp):
    """Under the split, fp_sparse_prefill_noalloc (partials in its static array)
    equals fp_sparse_prefill (partials in the workspace) bit for bit."""
    dev = torch.device("cuda:0")
    for cfg in (synth.config(1), synth.config(2, S=1029, Hq=4, Hkv=1, tau=1.0)):
        inp = synth.gen_fixed(cfg)
        q, k, v = inp.q.to(dev), inp.k.to(dev), inp.v.to(dev)
        ref = fp.sparse_prefill(q, k, v, cfg.block, cfg.tau, split_small=True)
        o = torch.full_like(ref["o"], float("nan"))
        lse = torch.full_like(ref["lse"], float("nan"))
        fp.fp_sparse_prefill_noalloc(ref["problem"], q, k, v, ref["kbar"], ref["vbar"], ref["row_ptr"],
                                     ref["col_idx"], ref["sched"], o=o, lse=lse)
        torch.cuda.synchronize()
        assert torch.equal(o, ref["o"]) and torch.equal(lse, ref["lse"])


def test_split_graph_replays(fp):
    """The split path (partials and merge in the workspace, no memset) captures
    into a HIP graph; every replay equals the eager run."""
    dev = torch.device("cuda:0")
    cfg = synth.config(2, S=1500, Hq=8, Hkv=2, tau=1.0)
    inp = synth.gen_fixed(cfg)
    q, k, v = inp.q.to(dev), inp.k.to(dev), inp.v.to(dev)
    eager = fp.sparse_prefill(q, k, v, cfg.block, cfg.tau, split_small=True)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fp.sparse_prefill(q, k, v, cfg.block, cfg.tau, split_small=True)    # warm
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        cap = fp.sparse_prefill(q, k, v, cfg.block, cfg.tau, split_small=True)
    for r in range(3):
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(cap["o"], eager["o"]) and torch.equal(cap["lse"], eager["lse"]), f"replay {r}"
        _ = torch.ones(1 << 20, device=dev).sum()                     # eager work between replays
        torch.cuda.synchronize()
