"""fp_estimate_select: pooling, block scores and the threshold in one call,
with the scores computed inside the selection from the pooled rows (no score
matrix in HBM). Its pooled rows, kept lists and schedule must equal those of
fp_block_scores + fp_select_blocks bit for bit (the scores are summed in the
same order), and therefore match the oracle outside the 1e-3 band."""
import math
import sys

import numpy as np
import pytest
import torch

import oracle
import synth
from fp_testutil import compare_masks, compare_outputs, csr_to_keep

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


def run_both(fp, inp, tau, block):
    dev = torch.device("cuda:0")
    mv = lambda t: None if t is None else t.to(dev)
    q, k, v = mv(inp.q), mv(inp.k), mv(inp.v)
    sc = dict(q_scale=mv(inp.q_scale), k_scale=mv(inp.k_scale), v_scale=mv(inp.v_scale))
    ref = fp.sparse_prefill(q, k, v, block, tau, **sc)
    fus = fp.sparse_prefill_fused(q, k, v, block, tau, **sc)
    torch.cuda.synchronize()
    for name in ("qbar", "kbar", "vbar", "row_ptr", "sched", "o", "lse"):
        assert torch.equal(ref[name], fus[name]), f"{name} differs between the fused and unfused paths"
    n = int(ref["row_ptr"][-1])
    assert torch.equal(ref["col_idx"][:n], fus["col_idx"][:n])
    return fus


CASES = [(synth.config(2, S=4096 + 77, Hq=8, Hkv=2, tau=2.0), "bf16"),
         (synth.config(2, S=3000, Hq=8, Hkv=2, block=64, tau=2.0), "bf16"),
         (synth.config(2, S=2500, Hq=6, Hkv=2, tau=1.0, seed=8), "bf16"),
         (synth.config(2, S=2048 + 9, Hq=16, Hkv=1, block=64, tau=1.5, seed=9), "bf16"),
         (synth.config(2, S=1500, Hq=2, Hkv=2, tau=1.0, seed=10, batch=2), "bf16"),
         (synth.config(2, S=700, Hq=8, Hkv=2, tau=float("inf")), "bf16"),
         (synth.config(2, S=700, Hq=8, Hkv=2, tau=-1.0), "bf16"),
         (synth.config(4, S=2048 + 40, Hq=8, Hkv=2, tau=2.0), "fp8"),
         (synth.config(1, S=1, tau=4.0), "bf16"),
         (synth.config(1, S=65, tau=0.05), "bf16")]


@pytest.mark.parametrize("cfg,kind", CASES,
                         ids=[f"S{c.S}-{c.Hq}x{c.Hkv}-b{c.block}-B{c.batch}-tau{c.tau}-{k}" for c, k in CASES])
def test_fused_equals_unfused_and_oracle(fp, cfg, kind):
    say(f"fused S={cfg.S} {cfg.Hq}/{cfg.Hkv} block {cfg.block} batch {cfg.batch} tau {cfg.tau} {kind}")
    inp = synth.gen_fixed(cfg)
    out = run_both(fp, inp, cfg.tau, cfg.block)
    nb = -(-cfg.S // cfg.block)
    rp, ci = out["row_ptr"].cpu().numpy(), out["col_idx"].cpu().numpy()
    c = 1 / math.sqrt(128)
    for b in range(cfg.batch):
        if kind == "bf16":
            qd, kd, vd = (oracle.widen_bf16(t[b]) for t in (inp.q, inp.k, inp.v))
        else:
            qd, kd, vd = (oracle.widen_fp8(t[b].numpy(), s_[b].numpy())
                          for t, s_ in ((inp.q, inp.q_scale), (inp.k, inp.k_scale), (inp.v, inp.v_scale)))
        ref = oracle.prefill(qd, kd, vd, cfg.block, cfg.tau, c, with_output=False)
        keep = csr_to_keep(rp, ci, b * cfg.Hkv * nb, cfg.Hkv, nb, nb)
        compare_masks(keep, ref["keep"], ref["R"], cfg.tau)


def test_fused_falls_back_past_1024_key_blocks(fp):
    """1025 key blocks do not fit the fused kernel's LDS: the call computes a
    score matrix in its workspace instead, with the same lists."""
    cfg = synth.config(2, S=1024 * 128 + 1, Hq=1, Hkv=1, tau=1.0, seed=12)
    say("fused fallback S=131073 1/1")
    run_both(fp, synth.gen_fixed(cfg), cfg.tau, cfg.block)
