"""The whole path (fp_block_scores, fp_select_blocks, fp_sparse_prefill) and
the paged entry point captured once in a HIP graph and replayed: the library
allocates, frees and synchronises nothing and records no memset, so a capture
replays the same kernels on whatever the captured buffers hold. Every replay
is compared bit for bit with an eager run, with eager work and
synchronisations between the replays; one replay runs on new input values
copied into the captured input tensors. The last test runs two problems on
two streams at once against serial runs (no state shared between calls)."""
import numpy as np
import pytest
import torch

import synth
from test_gpu_parity import fp, run_paged, say  # noqa: F401  (fp is a fixture)

pytestmark = pytest.mark.gpu


def same(a, b):
    return a is None and b is None or torch.equal(a, b)


def test_fixed_path_graph_replays(fp):
    cfg = synth.config(2, S=4096 + 77, Hq=8, Hkv=2, seed=91, tau=2.0)
    a, b = synth.gen_fixed(cfg), synth.gen_fixed(synth.config(2, S=4096 + 77, Hq=8, Hkv=2, seed=92, tau=2.0))
    dev = torch.device("cuda:0")
    q, k, v = (t.to(dev) for t in (a.q, a.k, a.v))
    keys = ("row_ptr", "col_idx", "sched", "o", "lse", "scores")

    def eager(qq, kk, vv):
        out = fp.sparse_prefill(qq, kk, vv, 128, cfg.tau)
        torch.cuda.synchronize()
        n = int(out["row_ptr"][-1])
        return {key: (out[key][:n] if key == "col_idx" else out[key]).clone() for key in keys}

    ref_a = eager(q, k, v)
    side = torch.cuda.Stream()                    # default priority
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fp.sparse_prefill(q, k, v, 128, cfg.tau)  # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        cap = fp.sparse_prefill(q, k, v, 128, cfg.tau)

    def check(ref, label):
        n = int(cap["row_ptr"][-1])
        for key in keys:
            got = cap[key][:n] if key == "col_idx" else cap[key]
            assert same(got, ref[key]), f"{label}: {key} differs"

    for r in range(3):
        cap["o"].zero_()                          # eager work between replays
        cap["row_ptr"].fill_(-1)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        check(ref_a, f"replay {r}")
    # new values in the captured inputs
    qb, kb, vb = (t.to(dev) for t in (b.q, b.k, b.v))
    ref_b = eager(qb, kb, vb)
    q.copy_(qb), k.copy_(kb), v.copy_(vb)
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    check(ref_b, "replay on new inputs")
    say("fixed path: 4 graph replays bit-identical to eager runs")


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
def test_paged_path_graph_replays(fp, dtype):
    cfg = synth.config(5, Hq=8, Hkv=2, n_seqs=3, len_range=(300, 3000), tau=2.0, dtype=dtype)
    L, P = synth.paged_lengths(cfg)
    inp = synth.gen_paged(cfg, (L, P))
    dev = torch.device("cuda:0")
    q, kc, vc, bt = inp.q.to(dev), inp.k_cache.to(dev), inp.v_cache.to(dev), inp.block_table.to(dev)
    sc = {n: None if t is None else t.to(dev)
          for n, t in (("q_scale", inp.q_scale), ("k_scale", inp.k_scale), ("v_scale", inp.v_scale))}
    vp = fp.make_varlen_problem(q, inp.cu_seqlens_q, inp.seqlens_k, kc, bt, cfg.block)
    ws = torch.empty(vp.ws_bytes, dtype=torch.uint8, device=dev)
    o0, lse0, rp0, ci0 = fp.fp_sparse_prefill_paged(vp, q, kc, vc, bt, cfg.tau, workspace=ws, **sc)
    torch.cuda.synchronize()
    n = int(rp0[-1])
    ref = [t.clone() for t in (o0, lse0, rp0, ci0[:n])]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fp.fp_sparse_prefill_paged(vp, q, kc, vc, bt, cfg.tau, workspace=ws, **sc)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        o, lse, rp, ci = fp.fp_sparse_prefill_paged(vp, q, kc, vc, bt, cfg.tau, workspace=ws, **sc)
    for r in range(3):
        o.zero_()
        lse.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for got, want in zip((o, lse, rp, ci[:n]), ref):
            assert torch.equal(got, want), f"paged replay {r} differs"
    say(f"paged path ({dtype}): 3 graph replays bit-identical to the eager run")


def test_two_streams_at_once(fp):
    """The library keeps no state between calls: two problems of different
    shapes enqueued on two streams (default priority) at the same time give
    the same bits as when run one after the other."""
    dev = torch.device("cuda:0")
    cfgs = [synth.config(2, S=4096 + 77, Hq=8, Hkv=2, seed=401, tau=2.0),
            synth.config(2, S=3000 + 5, Hq=6, Hkv=2, block=64, seed=402, tau=3.0)]
    ins = [synth.gen_fixed(c) for c in cfgs]
    qkv = [tuple(t.to(dev) for t in (i.q, i.k, i.v)) for i in ins]
    keys = ("row_ptr", "sched", "o", "lse", "scores")

    def run(n):
        out = fp.sparse_prefill(*qkv[n], cfgs[n].block, cfgs[n].tau)
        return out

    serial = []
    for n in range(2):
        out = run(n)
        torch.cuda.synchronize()
        serial.append({k: out[k].clone() for k in keys} | {"col_idx": out["col_idx"][:int(out["row_ptr"][-1])].clone()})
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    for s in streams:
        s.wait_stream(torch.cuda.current_stream())
    outs = []
    for n, s in enumerate(streams):
        with torch.cuda.stream(s):
            outs.append(run(n))
    torch.cuda.synchronize()
    for n in range(2):
        for k in keys:
            assert torch.equal(outs[n][k], serial[n][k]), f"problem {n}: {k} differs"
        nnz = int(outs[n]["row_ptr"][-1])
        assert torch.equal(outs[n]["col_idx"][:nnz], serial[n]["col_idx"])
    say("two problems on two streams at once: bit-identical to serial runs")


def test_fused_path_graph_replays(fp):
    """fp_estimate_select + fp_sparse_prefill captured and replayed, at a
    length whose score rows need more than 64 KiB of LDS (the fused kernel
    raises its dynamic LDS limit at launch, also under capture)."""
    cfg = synth.config(2, S=600 * 128 + 5, Hq=4, Hkv=1, seed=93, tau=2.0)
    inp = synth.gen_fixed(cfg)
    dev = torch.device("cuda:0")
    q, k, v = (t.to(dev) for t in (inp.q, inp.k, inp.v))
    keys = ("row_ptr", "sched", "o", "lse")
    ref = fp.sparse_prefill(q, k, v, 128, cfg.tau)          # the three-call path, eager
    torch.cuda.synchronize()
    n = int(ref["row_ptr"][-1])
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fp.sparse_prefill_fused(q, k, v, 128, cfg.tau)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        cap = fp.sparse_prefill_fused(q, k, v, 128, cfg.tau)
    for r in range(3):
        cap["o"].zero_()
        cap["row_ptr"].fill_(-1)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for key in keys:
            assert torch.equal(cap[key], ref[key]), f"fused replay {r}: {key} differs"
        assert torch.equal(cap["col_idx"][:n], ref["col_idx"][:n])
    say("fused path: 3 graph replays bit-identical to the eager three-call path")
