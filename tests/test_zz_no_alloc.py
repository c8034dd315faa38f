"""The allocation-free entry point (fp_sparse_prefill_noalloc) against
fp_sparse_prefill on the same kept lists: the same kernels run on the
library's static per-GPU scratch array instead of a caller workspace, so o
and lse must be bit-identical. Two calls in a row, the second on a smaller
problem (the array keeps the first call's contents), then a problem whose
rows reach whole summary sub-tiles, then fp8."""
import sys

import pytest
import torch

import synth

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, file=sys.stderr, flush=True)


@pytest.fixture(scope="module")
def fp():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import block_sparse_long_estimate_amd as m
    m._native.load()
    return m


def test_noalloc_equals_workspace_entry_point(fp):
    dev = torch.device("cuda:0")
    cases = [(synth.config(2, S=4096 + 77, Hq=8, Hkv=2, tau=2.0), "bf16"),
             (synth.config(2, S=1024 + 5, Hq=4, Hkv=1, tau=1.0, seed=9), "bf16"),
             # rows past 64 blocks: whole summary sub-tiles (per-lane offsets into the array)
             (synth.config(2, S=65 * 128 + 7, Hq=8, Hkv=2, tau=2.0, seed=5), "bf16"),
             (synth.config(4, S=2048 + 40, Hq=8, Hkv=2, tau=2.0), "fp8")]
    for cfg, kind in cases:
        say(f"noalloc S={cfg.S} {cfg.Hq}/{cfg.Hkv} tau={cfg.tau} {kind}")
        inp = synth.gen_fixed(cfg)
        mv = lambda t: None if t is None else t.to(dev)
        q, k, v = mv(inp.q), mv(inp.k), mv(inp.v)
        sc = dict(q_scale=mv(inp.q_scale), k_scale=mv(inp.k_scale), v_scale=mv(inp.v_scale))
        ref = fp.sparse_prefill(q, k, v, cfg.block, cfg.tau, **sc)
        o = torch.full_like(ref["o"], float("nan"))
        lse = torch.full_like(ref["lse"], float("nan"))
        fp.fp_sparse_prefill_noalloc(ref["problem"], q, k, v, ref["kbar"], ref["vbar"], ref["row_ptr"],
                                     ref["col_idx"], ref["sched"], o=o, lse=lse, **sc)
        torch.cuda.synchronize()
        assert torch.equal(o, ref["o"]), "o differs from fp_sparse_prefill"
        assert torch.equal(lse, ref["lse"]), "lse differs from fp_sparse_prefill"
