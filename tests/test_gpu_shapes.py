"""GPU parity on shapes the headline workloads do not reach: other GQA
ratios (including ones whose packed rows leave part of a slice empty), tiny
and ragged sequence lengths, strided views of a fused qkv tensor, and a
non-default softmax scale. Same comparison rules as test_gpu_parity."""
import math

import numpy as np
import pytest
import torch

import oracle
import synth
from fp_testutil import check_lse, lse_bound, check_csr_wellformed, compare_masks, compare_outputs, csr_to_keep
from test_gpu_parity import check_fixed, fp, say, widen  # noqa: F401  (fp is a fixture)

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("Hq,Hkv", [(8, 8), (6, 2), (16, 2), (16, 1)])
@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
def test_gqa_ratios(fp, Hq, Hkv, dtype):
    """G = 1, 3, 8, 16. G = 3 packs 384 rows per query block: the second
    256-row slice is half empty."""
    cfg = synth.config(2, S=1536 + 45, Hq=Hq, Hkv=Hkv, seed=40 + Hq + Hkv, dtype=dtype)
    say(f"GQA {Hq}/{Hkv} {dtype} S={cfg.S}")
    inp = synth.gen_fixed(cfg)
    check_fixed(fp, inp, 3.0, 128, kind=dtype)


@pytest.mark.parametrize("Hq,Hkv", [(6, 2), (16, 1)])
@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
def test_gqa_ratios_block64(fp, Hq, Hkv, dtype):
    """64-token blocks at G = 3 (192 packed rows: one slice, a quarter empty)
    and G = 16 (1024 packed rows: four slices)."""
    cfg = synth.config(2, S=1536 + 45, Hq=Hq, Hkv=Hkv, block=64, seed=50 + Hq + Hkv, dtype=dtype)
    say(f"GQA {Hq}/{Hkv} block 64 {dtype} S={cfg.S}")
    inp = synth.gen_fixed(cfg)
    check_fixed(fp, inp, 3.0, 64, kind=dtype)


@pytest.mark.parametrize("S,block", [(1, 128), (5, 128), (127, 128), (128, 128), (129, 128),
                                     (1, 64), (63, 64), (65, 64), (300, 64)])
def test_tiny_and_ragged_lengths(fp, S, block):
    cfg = synth.config(1, S=S, block=block, seed=70 + S)
    say(f"S={S} block={block}")
    inp = synth.gen_fixed(cfg)
    check_fixed(fp, inp, 2.0, block)


@pytest.mark.parametrize("S", [1, 129, 700])
def test_fp8_tiny_and_ragged(fp, S):
    cfg = synth.config(2, S=S, Hq=8, Hkv=2, seed=90 + S, dtype="fp8")
    say(f"fp8 S={S}")
    inp = synth.gen_fixed(cfg)
    check_fixed(fp, inp, 2.0, 128, kind="fp8")


def test_fused_qkv_strides(fp):
    """q, k, v as views of one [batch, S, Hq + 2 Hkv, 128] tensor: the same
    results, bit for bit, as contiguous copies."""
    cfg = synth.config(2, S=2048 + 17, Hq=8, Hkv=2, seed=123, batch=2)
    inp = synth.gen_fixed(cfg)
    dev = torch.device("cuda:0")
    q, k, v = (t.to(dev) for t in (inp.q, inp.k, inp.v))
    fused = torch.cat([q, k, v], dim=2)                   # [B, S, 12, 128]
    qv, kv, vv = fused[:, :, :8], fused[:, :, 8:10], fused[:, :, 10:12]
    assert not qv.is_contiguous() and not kv.is_contiguous()
    a = fp.sparse_prefill(q, k, v, 128, 3.0)
    b = fp.sparse_prefill(qv, kv, vv, 128, 3.0)
    torch.cuda.synchronize()
    assert torch.equal(a["row_ptr"], b["row_ptr"])
    n = int(a["row_ptr"][-1])
    assert torch.equal(a["col_idx"][:n], b["col_idx"][:n])
    assert torch.equal(a["o"], b["o"])
    assert torch.equal(a["lse"], b["lse"])
    check_fixed(fp, inp, 3.0, 128)


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
def test_softmax_scale(fp, dtype):
    """softmax_scale given explicitly (not 1/sqrt(d))."""
    cscale = 0.05
    cfg = synth.config(2, S=2048 + 99, Hq=8, Hkv=2, seed=321, dtype=dtype)
    inp = synth.gen_fixed(cfg)
    dev = torch.device("cuda:0")
    mv = lambda t: None if t is None else t.to(dev)
    q, k, v = (t.to(dev) for t in (inp.q, inp.k, inp.v))
    tau = 2.0
    out = fp.sparse_prefill(q, k, v, 128, tau, softmax_scale=cscale, q_scale=mv(inp.q_scale),
                            k_scale=mv(inp.k_scale), v_scale=mv(inp.v_scale))
    torch.cuda.synchronize()
    S, Hkv = cfg.S, cfg.Hkv
    nb = -(-S // 128)
    rp, ci = out["row_ptr"].cpu().numpy(), out["col_idx"].cpu().numpy()
    check_csr_wellformed(rp, ci, lambda r: r % nb)
    qd, kd, vd = widen(inp, 0)
    ref = oracle.prefill(qd, kd, vd, 128, tau, cscale, with_output=False)
    assert np.abs(out["scores"][0].cpu().numpy()[np.isfinite(ref["S"])] - ref["S"][np.isfinite(ref["S"])]).max() \
        <= 2e-4 * max(1.0, np.abs(ref["S"][np.isfinite(ref["S"])]).max())
    keep = csr_to_keep(rp, ci, 0, Hkv, nb, nb)
    compare_masks(keep, ref["keep"], ref["R"], tau)
    o_ref, lse_ref = oracle.attend(qd, kd, vd, keep, ref["kbar"], ref["vbar"], cscale, 128, 0)
    compare_outputs(out["o"][0].float().cpu().numpy(), o_ref, dtype)
    check_lse(out["lse"][0].cpu().numpy(), lse_ref, lse_bound(qd, kd, keep, ref["kbar"], lse_ref, cscale, 128, 0,
                                                             kind=dtype))


@pytest.mark.parametrize("cid,S", [(2, 4096 + 33), (1, 2048)])
def test_fp32_output_derived_bound(fp, cid, S):
    """Diagnostic fp32 output. The bf16 result must be the bf16 rounding of it,
    bit for bit, and against the fp64 oracle (same kept lists) the error is
    bounded by the kernel's own roundings: P to bf16 (RNE, relative <= 2^-8
    per weight) and the pooled V to bf16 (relative <= 2^-8), each moving a
    weighted average by at most 2^-8 max|v|, so |o - o_ref| <= 2^-7 max|v|
    up to fp32 accumulation noise."""
    cfg = synth.config(cid, S=S, seed=555 + cid)
    inp = synth.gen_fixed(cfg)
    dev = torch.device("cuda:0")
    q, k, v = (t.to(dev) for t in (inp.q, inp.k, inp.v))
    tau, block = 2.0, cfg.block
    ob = fp.sparse_prefill(q, k, v, block, tau)
    of = fp.sparse_prefill(q, k, v, block, tau, out_fp32=True)
    torch.cuda.synchronize()
    assert of["o"].dtype == torch.float32
    assert torch.equal(ob["row_ptr"], of["row_ptr"])
    assert torch.equal(of["o"].to(torch.bfloat16), ob["o"])
    assert torch.equal(ob["lse"], of["lse"])
    nb = -(-S // block)
    rp, ci = of["row_ptr"].cpu().numpy(), of["col_idx"].cpu().numpy()
    qd, kd, vd = widen(inp, 0)
    c = 1 / math.sqrt(128)
    ref = oracle.prefill(qd, kd, vd, block, tau, c, with_output=False)
    keep = csr_to_keep(rp, ci, 0, cfg.Hkv, nb, nb)
    o_ref, _ = oracle.attend(qd, kd, vd, keep, ref["kbar"], ref["vbar"], c, block, 0)
    err = np.abs(of["o"][0].cpu().numpy() - o_ref)
    vmax = np.abs(vd).max()
    bound = 2.0 ** -7 * vmax + 1e-5
    say(f"fp32 out: max|err| {err.max():.3e} (bound {bound:.3e}), mean {err.mean():.3e}")
    assert err.max() <= bound


@pytest.mark.parametrize("block", [128, 64])
def test_fp32_output_fp8(fp, block):
    """Diagnostic fp32 output on fp8 inputs: the bf16 result is its bf16
    rounding, bit for bit, and against the fp64 oracle (same kept lists) the
    error is bounded by the kernel's roundings: P to E4M3 (RNE, relative
    <= 2^-4 per weight while normal; below the normal range an absolute
    2^-10 of the scaled weight), P of the correction and the pooled V to bf16
    (2^-8 each), so |o - o_ref| <= (2^-4 + 2^-7) max|v| plus the subnormal
    term, taken here as 2^-8 max|v|."""
    cfg = synth.config(2, S=3000 + 21, Hq=8, Hkv=2, block=block, seed=561 + block, dtype="fp8")
    inp = synth.gen_fixed(cfg)
    dev = torch.device("cuda:0")
    mv = lambda t: None if t is None else t.to(dev)
    q, k, v = (t.to(dev) for t in (inp.q, inp.k, inp.v))
    sc = dict(q_scale=mv(inp.q_scale), k_scale=mv(inp.k_scale), v_scale=mv(inp.v_scale))
    tau = 2.0
    ob = fp.sparse_prefill(q, k, v, block, tau, **sc)
    of = fp.sparse_prefill(q, k, v, block, tau, out_fp32=True, **sc)
    torch.cuda.synchronize()
    assert of["o"].dtype == torch.float32
    assert torch.equal(ob["row_ptr"], of["row_ptr"])
    assert torch.equal(of["o"].to(torch.bfloat16), ob["o"])
    assert torch.equal(ob["lse"], of["lse"])
    nb = -(-cfg.S // block)
    rp, ci = of["row_ptr"].cpu().numpy(), of["col_idx"].cpu().numpy()
    qd, kd, vd = widen(inp, 0)
    c = 1 / math.sqrt(128)
    ref = oracle.prefill(qd, kd, vd, block, tau, c, with_output=False)
    keep = csr_to_keep(rp, ci, 0, cfg.Hkv, nb, nb)
    o_ref, _ = oracle.attend(qd, kd, vd, keep, ref["kbar"], ref["vbar"], c, block, 0)
    err = np.abs(of["o"][0].cpu().numpy() - o_ref)
    vmax = np.abs(vd).max()
    bound = (2.0 ** -4 + 2.0 ** -7 + 2.0 ** -8) * vmax
    say(f"fp8 fp32 out block {block}: max|err| {err.max():.3e} (bound {bound:.3e}), mean {err.mean():.3e}")
    assert err.max() <= bound


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
@pytest.mark.parametrize("S,block", [(1000 + 77, 128), (700 + 5, 64)])
def test_no_reads_past_sequence_end(fp, dtype, S, block):
    """q, k and v are views of tensors whose tokens past S are NaN (fp8: NaN
    codes): every output, lse and kept list is bit-identical to the run on
    exact-size tensors, so the ragged last block reads nothing past the end."""
    cfg = synth.config(2, S=S, Hq=8, Hkv=2, block=block, seed=301 + block, dtype=dtype)
    inp = synth.gen_fixed(cfg)
    dev = torch.device("cuda:0")
    mv = lambda t: None if t is None else t.to(dev)
    qs, ks, vs = mv(inp.q_scale), mv(inp.k_scale), mv(inp.v_scale)

    def padded(t):
        big = torch.empty((t.shape[0], S + 300, t.shape[2], t.shape[3]), dtype=t.dtype, device=dev)
        if dtype == "fp8":
            big.fill_(0x7F)
        else:
            big.fill_(float("nan"))
        big[:, :S] = t.to(dev)
        return big[:, :S]

    a = fp.sparse_prefill(mv(inp.q), mv(inp.k), mv(inp.v), block, 2.0, q_scale=qs, k_scale=ks, v_scale=vs)
    b = fp.sparse_prefill(padded(inp.q), padded(inp.k), padded(inp.v), block, 2.0, q_scale=qs, k_scale=ks,
                          v_scale=vs)
    torch.cuda.synchronize()
    n = int(a["row_ptr"][-1])
    assert torch.equal(a["row_ptr"], b["row_ptr"]) and torch.equal(a["col_idx"][:n], b["col_idx"][:n])
    for key in ("qbar", "kbar", "vbar", "o", "lse"):
        assert torch.equal(a[key], b[key]), key
    assert torch.equal(torch.isinf(a["scores"]), torch.isinf(b["scores"]))
    fin = torch.isfinite(a["scores"])
    assert torch.equal(a["scores"][fin], b["scores"][fin])
    say(f"S={S} block={block} {dtype}: NaN tokens past the end change nothing")
