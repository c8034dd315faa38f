"""The ablation variants against the oracle's variants: per-query-head kept
lists (E4 without the GQA union; rows per query head) and the block-score
correction (a pruned block's pseudo-token takes the block score as logit for
every row of its query block). Kept lists match except inside the 1e-3 band,
outputs within the bf16 / fp8 tolerances under the GPU's lists."""
import math
import sys

import numpy as np
import pytest
import torch

import oracle
import synth
from fp_testutil import check_lse, compare_masks, compare_outputs, lse_bound

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


def lists_to_keep(rp, ci, nrow_groups, nq, nb):
    keep = np.zeros((nrow_groups, nq, nb), dtype=bool)
    for g in range(nrow_groups):
        for il in range(nq):
            r = g * nq + il
            keep[g, il, ci[rp[r]:rp[r + 1]]] = True
    return keep


CASES = [(synth.config(2, S=4096 + 77, Hq=8, Hkv=2, tau=2.0), "bf16"),
         (synth.config(2, S=3000, Hq=6, Hkv=2, block=64, tau=1.5, seed=4), "bf16"),
         (synth.config(4, S=2048 + 40, Hq=8, Hkv=2, tau=2.0), "fp8")]


@pytest.mark.parametrize("variant", ["per_head", "block_score"])
@pytest.mark.parametrize("cfg,kind", CASES, ids=[f"S{c.S}-{c.Hq}x{c.Hkv}-b{c.block}-{k}" for c, k in CASES])
def test_variant_against_oracle(fp, cfg, kind, variant):
    say(f"variant {variant}: S={cfg.S} {cfg.Hq}/{cfg.Hkv} block {cfg.block} tau {cfg.tau} {kind}")
    inp = synth.gen_fixed(cfg)
    dev = torch.device("cuda:0")
    mv = lambda t: None if t is None else t.to(dev)
    q, k, v = mv(inp.q), mv(inp.k), mv(inp.v)
    sc = dict(q_scale=mv(inp.q_scale), k_scale=mv(inp.k_scale), v_scale=mv(inp.v_scale))
    out = fp.sparse_prefill(q, k, v, cfg.block, cfg.tau, variant=variant, **sc)
    if variant == "per_head":               # the fused selection makes the same per-head decisions
        fus = fp.sparse_prefill_fused(q, k, v, cfg.block, cfg.tau, variant=variant, **sc)
    torch.cuda.synchronize()
    nb = -(-cfg.S // cfg.block)
    rp, ci = out["row_ptr"].cpu().numpy(), out["col_idx"].cpu().numpy()
    if variant == "per_head":
        assert len(rp) - 1 == cfg.Hq * nb
        for key in ("row_ptr", "sched", "o", "lse"):
            assert torch.equal(fus[key], out[key]), key
    if kind == "bf16":
        qd, kd, vd = (oracle.widen_bf16(t[0]) for t in (inp.q, inp.k, inp.v))
    else:
        qd, kd, vd = (oracle.widen_fp8(t[0].numpy(), s_[0].numpy())
                      for t, s_ in ((inp.q, inp.q_scale), (inp.k, inp.k_scale), (inp.v, inp.v_scale)))
    c = 1 / math.sqrt(128)
    ref = oracle.prefill(qd, kd, vd, cfg.block, cfg.tau, c, with_output=False, variant=variant)
    groups = cfg.Hq if variant == "per_head" else cfg.Hkv
    keep = lists_to_keep(rp, ci, groups, nb, nb)
    ndiff, nband = compare_masks(keep, ref["keep"], ref["R"], cfg.tau)
    assert (~keep[np.tril(np.ones((nb, nb), dtype=bool))[None].repeat(groups, 0)]).any()   # real pruning
    o_ref, lse_ref = oracle.attend(qd, kd, vd, keep, ref["kbar"], ref["vbar"], c, cfg.block, 0,
                                   block_scores=ref["S"] if variant == "block_score" else None)
    mx, mean = compare_outputs(out["o"][0].float().cpu().numpy(), o_ref, kind)
    if variant == "per_head":
        per_group = keep.reshape(cfg.Hkv, cfg.Hq // cfg.Hkv, nb, nb)
        check_lse(out["lse"][0].cpu().numpy(), lse_ref,
                  lse_bound(qd, kd, per_group.any(axis=1), ref["kbar"], lse_ref, c, cfg.block, 0, kind=kind,
                            pruned=~per_group.all(axis=1)))
    else:
        # the pseudo-token logits are the fp32 block scores: their error is that of E2
        err = np.abs(out["lse"][0].cpu().numpy() - lse_ref)
        assert err.max() <= 2e-4 * max(1.0, np.abs(ref["S"][np.isfinite(ref["S"])]).max()) + 1e-3
    mean_out = fp.sparse_prefill(q, k, v, cfg.block, cfg.tau, **sc)
    torch.cuda.synchronize()
    assert not torch.equal(mean_out["o"], out["o"])          # a different result from the stated method
    say(f"  mask diffs {ndiff} (band {nband}) max|err| {mx:.2e} mean {mean:.2e}")
