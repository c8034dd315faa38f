"""The dense causal path (fp_dense_prefill): every key block of every row
attended on the sparse kernel's tile loop, with no estimate, selection or
correction -- this library's own dense baseline.

It must equal the oracle's E6 with every block kept (textbook causal softmax
attention), and fp_sparse_prefill on tau = +inf bit for bit (the same tiles in
the same order per row)."""
import math
import sys

import numpy as np
import pytest
import torch

import oracle
import synth
from fp_testutil import TOL, check_lse, compare_outputs, lse_bound

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


def to_dev(inp):
    dev = torch.device("cuda:0")
    mv = lambda t: None if t is None else t.to(dev)
    return mv(inp.q), mv(inp.k), mv(inp.v), dict(q_scale=mv(inp.q_scale), k_scale=mv(inp.k_scale),
                                                  v_scale=mv(inp.v_scale))


def widen(inp, b=0):
    if inp.q.dtype == torch.bfloat16:
        return [oracle.widen_bf16(t[b]) for t in (inp.q, inp.k, inp.v)]
    return [oracle.widen_fp8(t[b].numpy(), s[b].numpy())
            for t, s in ((inp.q, inp.q_scale), (inp.k, inp.k_scale), (inp.v, inp.v_scale))]


CASES = [(synth.config(2, S=2048 + 77, Hq=8, Hkv=2), "bf16"),
         (synth.config(1, S=1000), "bf16"),
         (synth.config(2, S=1536 + 3, Hq=6, Hkv=2, block=64), "bf16"),
         (synth.config(4, S=2048 + 40, Hq=8, Hkv=2), "fp8"),
         (synth.config(1, S=777, dtype="fp8"), "fp8")]


@pytest.mark.parametrize("cfg,kind", CASES, ids=[f"S{c.S}-{c.Hq}x{c.Hkv}-b{c.block}-{k}" for c, k in CASES])
def test_dense_against_oracle_and_sparse_tau_inf(fp, cfg, kind):
    inp = synth.gen_fixed(cfg)
    q, k, v, sc = to_dev(inp)
    say(f"dense S={cfg.S} {cfg.Hq}/{cfg.Hkv} block {cfg.block} {kind}")
    p = fp.make_problem(q, k, v, cfg.block)
    o, lse = fp.fp_dense_prefill(p, q, k, v, **sc)
    sp = fp.sparse_prefill(q, k, v, cfg.block, float("inf"), **sc)
    torch.cuda.synchronize()
    assert torch.equal(o, sp["o"]) and torch.equal(lse, sp["lse"]), "dense differs from tau = +inf"
    qd, kd, vd = widen(inp)
    c = 1 / math.sqrt(128)
    ref = oracle.prefill(qd, kd, vd, cfg.block, float("inf"), c)
    assert ref["keep"][np.tril(np.ones(ref["keep"].shape[1:], dtype=bool))[None].repeat(cfg.Hkv, 0)].all()
    mx, mean = compare_outputs(o[0].float().cpu().numpy(), ref["o"], kind)
    check_lse(lse[0].cpu().numpy(), ref["lse"],
              lse_bound(qd, kd, ref["keep"], ref["kbar"], ref["lse"], c, cfg.block, 0, kind=kind))
    say(f"  max|err| {mx:.2e} mean {mean:.2e}")


@pytest.mark.parametrize("S,Hq,block", [(130 * 128 + 5, 4, 128), (200 * 64 + 7, 2, 64)])
def test_long_rows_equal_dense(fp, S, Hq, block):
    """Rows keeping more than 64 and 128 blocks (the kernel holds a row's kept
    list 64 codes per register and reloads it as it goes): tau = +inf through
    the sparse path equals the dense path bit for bit, so every row visits
    its blocks 0..i in order across the reloads."""
    cfg = synth.config(2, S=S, Hq=Hq, Hkv=1, block=block)
    inp = synth.gen_fixed(cfg)
    q, k, v, sc = to_dev(inp)
    say(f"long rows S={S} {Hq}/1 block {block}")
    p = fp.make_problem(q, k, v, block)
    o, lse = fp.fp_dense_prefill(p, q, k, v, **sc)
    sp = fp.sparse_prefill(q, k, v, block, float("inf"), **sc)
    torch.cuda.synchronize()
    nb = -(-S // block)
    assert int(np.diff(sp["row_ptr"].cpu().numpy()).max()) == nb
    assert torch.equal(o, sp["o"]) and torch.equal(lse, sp["lse"]), "tau = +inf differs from dense"


def test_dense_against_torch_sdpa(fp):
    """An independent reference: torch's scaled_dot_product_attention (causal,
    float32, CPU) on the same bf16 inputs."""
    cfg = synth.config(2, S=1024 + 33, Hq=8, Hkv=2)
    inp = synth.gen_fixed(cfg)
    q, k, v, sc = to_dev(inp)
    p = fp.make_problem(q, k, v, cfg.block)
    o, _ = fp.fp_dense_prefill(p, q, k, v, with_lse=False)
    torch.cuda.synchronize()
    qq = inp.q[0].float().permute(1, 0, 2)
    kk = inp.k[0].float().repeat_interleave(4, dim=1).permute(1, 0, 2)
    vv = inp.v[0].float().repeat_interleave(4, dim=1).permute(1, 0, 2)
    ref = torch.nn.functional.scaled_dot_product_attention(qq[None], kk[None], vv[None], is_causal=True)
    err = (o[0].float().cpu().permute(1, 0, 2) - ref[0]).abs()
    assert err.max() <= TOL["bf16"][0] and err.mean() <= TOL["bf16"][1]
