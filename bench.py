"""Benchmark of the block-sparse prefill hot path on one MI355X.

One step = the whole path on one layer: fp_block_scores (pooling + block
scores), fp_select_blocks (threshold + CSR + schedule) and fp_sparse_prefill
(sparse attention + mean correction), on the S=131072, 32 query / 8 KV head,
head dim 128, 128x128-block, tau=4 bf16 workload (synthetic, seeded; inputs
resident in HBM before timing). The same path is also timed on the fp8-e4m3
version of the same tensors.

    python bench.py [--gpus 1] [--steps 10] [--warmup 3]

Prints one JSON line: dense-equivalent TFLOP/s of the bf16 step as `value`,
ms per layer, kept-block fraction, the attention kernel's MFMA roofline
fraction over the FLOPs of the kept blocks, and the single-threaded CPU
oracle's throughput on a bounded sample as `cpu_baseline`. Context legs on
the same tensors (skipped with --no-sweep): bf16 at tau 2, 6, 8, and tau=inf,
where every block is kept and the path is this library's own dense causal
attention. The paged varlen entry point is timed on its own 8-sequence
batch (skipped with --no-paged), and the S=2048 and S=32768 configurations
on their own (skipped with --no-configs). A chunked prefill of the same sequence in three chunks is timed
with and without the pooled-KV cache (skipped with --no-chunked). The error
of the sparse outputs against that dense attention is reported at tau 2, 4, 8 for four variants: mean
correction, none, per-query-head lists, block-score correction (skipped
with --no-ablation).
"""
from __future__ import annotations

import argparse
import ctypes
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_TFLOPS = {"bf16": 2500.0, "fp8": 5000.0}   # MI355X dense MFMA peaks
HBM_GBS = 8000.0


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kept_flops_from_csr(row_ptr, col_idx, nb, S, B, G, d, Hkv, batch):
    """4 d G x causal (t, s) pairs inside the kept block pairs; rows (b, g, i)."""
    counts = np.diff(row_ptr)
    rows = np.arange(len(counts))
    i_of_row = np.repeat(rows % nb, counts)
    j = col_idx[:row_ptr[-1]]
    ni = np.minimum((i_of_row + 1) * B, S) - i_of_row * B
    mj = np.minimum((j + 1) * B, S) - j * B
    pairs = np.where(j < i_of_row, ni * mj, ni * (ni + 1) // 2)
    kept = 4.0 * d * G * pairs.astype(np.float64).sum()
    # correction work: each row's pruned blocks are pseudo-tokens for its |I_i| rows
    i_all = rows % nb
    n_all = np.minimum((i_all + 1) * B, S) - i_all * B
    npr = (i_all + 1) - counts
    corr = 4.0 * d * G * float((n_all * npr).sum())
    return kept, corr


def varlen_flops(rp, ci, L, P, B, G, d, Hkv):
    """Kept, correction and dense-equivalent FLOPs of a varlen batch whose CSR
    rows are (b, g, il), il over the query blocks of [P_b, L_b) on the
    absolute block grid; causal (t, s) pairs counted exactly."""
    kept = corr = dense = 0.0
    row = 0
    for Lb, Pb in zip(L, P):
        Lb, Pb = int(Lb), int(Pb)
        i0, i1 = Pb // B, (Lb - 1) // B
        dense += 4.0 * d * G * Hkv * sum(t + 1 for t in range(Pb, Lb))
        for g in range(Hkv):
            for i in range(i0, i1 + 1):
                lo, hi = max(i * B, Pb), min((i + 1) * B, Lb)
                cols = ci[rp[row]:rp[row + 1]]
                row += 1
                for j in cols:
                    j = int(j)
                    if j < i:
                        kept += (hi - lo) * (min((j + 1) * B, Lb) - j * B)
                    else:                      # diagonal: s in [iB, t]
                        kept += sum(t - i * B + 1 for t in range(lo, hi))
                corr += (hi - lo) * ((i + 1) - len(cols))
    assert row == len(rp) - 1
    return 4.0 * d * G * kept, 4.0 * d * G * corr, dense


def time_paged(fp, N, steps, warmup, dtype="bf16"):
    """The paged varlen entry point (all stages in one call) on the 8-sequence
    batch of 4K-64K tokens with cached prefixes and 64-token pages; fp8: the
    same batch as E4M3FN codes with one scale per 128 positions."""
    import torch
    import synth
    cfg = synth.config(5, dtype=dtype)
    inp = synth.gen_paged(cfg)
    dev = torch.device("cuda:0")
    q, kc, vc, bt = inp.q.to(dev), inp.k_cache.to(dev), inp.v_cache.to(dev), inp.block_table.to(dev)
    sc = {n: None if t is None else t.to(dev)
          for n, t in (("q_scale", inp.q_scale), ("k_scale", inp.k_scale), ("v_scale", inp.v_scale))}
    vp = fp.make_varlen_problem(q, inp.cu_seqlens_q, inp.seqlens_k, kc, bt, cfg.block)
    ws = torch.empty(vp.ws_bytes, dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()
    for _ in range(warmup):
        out = fp.fp_sparse_prefill_paged(vp, q, kc, vc, bt, cfg.tau, workspace=ws, **sc)
    torch.cuda.synchronize()
    ts = []
    for _ in range(steps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        out = fp.fp_sparse_prefill_paged(vp, q, kc, vc, bt, cfg.tau, workspace=ws, **sc)
        e1.record(stream)
        ts.append((e0, e1))
    torch.cuda.synchronize()
    ms = [a.elapsed_time(b) for a, b in ts]
    rp, ci = out[2].cpu().numpy(), out[3].cpu().numpy()
    G = cfg.Hq // cfg.Hkv
    kept, corr, dense = varlen_flops(rp, ci, inp.seqlens_k, inp.prefix, cfg.block, G, 128, cfg.Hkv)
    nblk = sum(cfg.Hkv * sum(i + 1 for i in range(int(P) // cfg.block, (int(L) - 1) // cfg.block + 1))
               for L, P in zip(inp.seqlens_k, inp.prefix))
    t = float(np.median(ms))
    res = {"workload": f"{len(inp.seqlens_k)} sequences, L={inp.seqlens_k.tolist()}, "
                       f"cached prefix P={inp.prefix.tolist()}, {cfg.page_size}-token pages, "
                       f"32/8 heads, 128x128 blocks, tau={cfg.tau}",
           "ms_per_layer_median": round(t, 4), "steps": steps,
           "dense_equiv_tflops": round(dense / (t * 1e-3) / 1e12, 2),
           "kept_fraction": round(len(ci[:rp[-1]]) / nblk, 5),
           "kept_tflops_whole_call": round(kept / (t * 1e-3) / 1e12, 2),
           "mfma_util_kept_whole_call": round(kept / (t * 1e-3) / 1e12 / PEAK_TFLOPS[dtype], 4),
           "correction_tflop": round(corr / 1e12, 3)}
    del q, kc, vc, bt, ws, out, sc
    torch.cuda.empty_cache()
    return res


def time_chunked(fp, inp, tau, ends=(43690, 87380, 131072), page=64, reps=5):
    """Chunked prefill of the S=131072 sequence in three chunks through the
    paged entry points (the fixed-shape tensors moved into a shuffled cache of
    64-token pages): each chunk timed with the pooled-KV cache
    (fp_sparse_prefill_paged_cached: cached blocks are not re-pooled) and
    without it (fp_sparse_prefill_paged: all keys pooled on every call)."""
    import torch
    dev = torch.device("cuda:0")
    S, Hkv = inp.k.shape[1], inp.k.shape[2]
    assert ends[-1] == S and S % page == 0
    npg = S // page
    perm = torch.from_numpy(np.random.default_rng(5).permutation(npg)).to(dev)
    kc = torch.empty((npg, page, Hkv, 128), dtype=inp.k.dtype, device=dev)
    vc = torch.empty_like(kc)
    kc[perm] = inp.k[0].to(dev).view(npg, page, Hkv, 128)
    vc[perm] = inp.v[0].to(dev).view(npg, page, Hkv, 128)
    bt = perm.to(torch.int32).view(1, npg).contiguous()
    q = inp.q[0].to(dev)
    B = inp.cfg.block
    slots = fp.pooled_kv_slots(kc, B)
    kbc = torch.zeros((slots, Hkv, 128), device=dev)
    vbc = torch.zeros_like(kbc)
    stream = torch.cuda.current_stream()
    calls, P = [], 0
    for E in ends:
        qc = q[P:E].contiguous()
        vp = fp.make_varlen_problem(qc, np.array([0, E - P], dtype=np.int32), np.array([E], dtype=np.int32),
                                    kc, bt, B)
        ws = torch.empty(vp.ws_bytes, dtype=torch.uint8, device=dev)
        calls.append((P, E, vp, qc, ws))
        P = E

    def run(c, cached):
        _, _, vp, qc, ws = c
        if cached:
            return fp.fp_sparse_prefill_paged_cached(vp, qc, kc, vc, bt, kbc, vbc, tau, with_lse=False, workspace=ws)
        return fp.fp_sparse_prefill_paged(vp, qc, kc, vc, bt, tau, with_lse=False, workspace=ws)

    for c in calls:                              # fills the pooled cache chunk by chunk
        run(c, True)
        run(c, False)
    torch.cuda.synchronize()
    res = []
    for c in calls:
        row = {"rows": [c[0], c[1]]}
        for name, cached in (("ms_cached", True), ("ms_uncached", False)):
            ts = []
            for _ in range(reps):
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                run(c, cached)
                e1.record(stream)
                ts.append((e0, e1))
            torch.cuda.synchronize()
            row[name] = round(float(np.median([a.elapsed_time(b) for a, b in ts])), 4)
        res.append(row)
    del kc, vc, kbc, vbc, calls, q
    torch.cuda.empty_cache()
    return {"workload": f"S={S} in chunks ending at {list(ends)}, {page}-token shuffled pages, "
                        f"32/8 heads, 128x128 blocks, tau={tau}, bf16", "chunks": res}


def graph_replay_ms(fp, inp, tau, replays=20):
    """The whole path captured once in a HIP graph and replayed: median ms per
    replay (for small prefills, where launch overhead dominates)."""
    import torch
    dev = torch.device("cuda:0")
    q, k, v = inp.q.to(dev), inp.k.to(dev), inp.v.to(dev)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fp.sparse_prefill_fused(q, k, v, inp.cfg.block, tau)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fp.sparse_prefill_fused(q, k, v, inp.cfg.block, tau)
    g.replay()
    torch.cuda.synchronize()
    ts = []
    for _ in range(replays):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        g.replay()
        e1.record()
        ts.append((e0, e1))
    torch.cuda.synchronize()
    ms = float(np.median([a.elapsed_time(b) for a, b in ts]))
    del g, q, k, v
    torch.cuda.empty_cache()
    return ms


ABLATION_VARIANTS = ("mean", "none", "per_head", "block_score")


def ablation_vs_dense(fp, inp, taus=(2.0, 4.0, 8.0), chunk=8192):
    """Error of the sparse path against this library's dense causal attention
    (tau = inf: every block kept) on the same tensors, for the four variants
    of the method: the mean correction over GQA-union lists ("mean"), no
    correction ("none"), one list per query head with the mean correction
    ("per_head"), and the block score as each pruned block's logit
    ("block_score"). Max and mean |o - o_dense| (V is in units of max|V|),
    the relative Frobenius norm, the kept fraction of the causal block pairs
    (per list) and the wall time of one whole call (allocation included). A synthetic stand-in for the
    pages' accuracy claim, which needs trained weights to check."""
    import torch
    dev = torch.device("cuda:0")
    q, k, v = inp.q.to(dev), inp.k.to(dev), inp.v.to(dev)
    B = inp.cfg.block
    nb = -(-q.shape[1] // B)
    dense = fp.sparse_prefill(q, k, v, B, float("inf"), with_lse=False)["o"]
    ref_sq = 0.0
    for t0 in range(0, dense.shape[1], chunk):
        ref_sq += float(dense[:, t0:t0 + chunk].float().pow(2).sum())
    res = {}
    for tau in taus:
        row = {}
        for name in ABLATION_VARIANTS:
            fp.sparse_prefill(q, k, v, B, tau, with_lse=False, variant=name)   # warm
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            out = fp.sparse_prefill(q, k, v, B, tau, with_lse=False, variant=name)
            torch.cuda.synchronize()
            ms = (time.perf_counter() - t0) * 1e3
            o = out["o"]
            lists = out["row_ptr"].numel() - 1
            kept = int(out["row_ptr"][-1]) / (lists // nb * nb * (nb + 1) // 2)
            mx, sm, sq, n = 0.0, 0.0, 0.0, 0
            for t0 in range(0, o.shape[1], chunk):
                d = (o[:, t0:t0 + chunk].float() - dense[:, t0:t0 + chunk].float()).abs_()
                mx = max(mx, float(d.max()))
                sm += float(d.sum())
                sq += float(d.pow_(2).sum())
                n += d.numel()
            row[name] = {"max_abs": round(mx, 5), "mean_abs": round(sm / n, 6),
                         "rel_fro": round(math.sqrt(sq / ref_sq), 6), "kept": round(kept, 5),
                         "ms_call": round(ms, 2)}
            del out, o
            torch.cuda.empty_cache()
        res[str(tau)] = row
    del q, k, v, dense
    torch.cuda.empty_cache()
    return res


def plants_kept(metas, rp, ci, Hkv, nb):
    """How many of the planted (KV head, query block, key block) pairs of the
    synthetic inputs the produced kept lists hold, as [kept, planted]; rows
    of the fixed layout are (sequence, KV head, query block)."""
    kept = total = 0
    for b, meta in enumerate(metas):
        for g, ip, jp, _ in meta.plants:
            r = (b * Hkv + g) * nb + ip
            kept += int(jp in set(ci[rp[r]:rp[r + 1]].tolist()))
            total += 1
    return [kept, total]


def time_path(fp, N, inp, tau, steps, warmup, label, flush_bytes=0, keep_outputs=False, fused=True,
              split_small=False, sampler=None):
    """Run the path `warmup` + `steps` times; HIP events per stage on the
    current stream (the library launches on it). fused: fp_estimate_select +
    fp_sparse_prefill (no score matrix); otherwise the three calls
    fp_block_scores + fp_select_blocks + fp_sparse_prefill. flush_bytes > 0:
    before each timed step a buffer of that size is overwritten (outside the
    events), so L2 and the memory-side cache start cold. keep_outputs: also
    return the outputs of KV head 0's query heads (host, fp32) and lse.
    split_small: a problem too small for the chip splits its rows' tiles
    (FP_SPLIT_SMALL_GRIDS). sampler: started after the warm-up steps and
    stopped once the timed steps have finished."""
    import torch
    dev = torch.device("cuda:0")
    q, k, v = inp.q.to(dev), inp.k.to(dev), inp.v.to(dev)
    sc = [None if t is None else t.to(dev) for t in (inp.q_scale, inp.k_scale, inp.v_scale)]
    block = inp.cfg.block
    p = fp.make_problem(q, k, v, block, split_small=split_small)
    c = p.c
    f32 = dict(dtype=torch.float32, device=dev)
    i32 = dict(dtype=torch.int32, device=dev)
    qbar = torch.empty((c.batch, c.num_q_heads, p.nb, 128), **f32)
    kbar = torch.empty((c.batch, c.num_kv_heads, p.nb, 128), **f32)
    vbar = torch.empty((c.batch, c.num_kv_heads, p.nb, 128), **f32)
    scores = None if fused else torch.empty((c.batch, c.num_q_heads, p.nb, p.nb), **f32)
    row_ptr = torch.empty(p.rows + 1, **i32)
    col_idx = torch.empty(p.max_nnz, **i32)
    sched = torch.empty(p.rows, **i32)
    lib = N.load()
    ws = torch.empty(N.check_size(lib.fp_estimate_select_workspace_size(p.ref) if fused
                                  else lib.fp_workspace_size(p.ref)), dtype=torch.uint8, device=dev)
    ws2 = torch.empty(N.check_size(lib.fp_prefill_workspace_size(p.ref)), dtype=torch.uint8, device=dev)
    o = torch.empty((c.batch, c.seqlen, c.num_q_heads, 128), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((c.batch, c.num_q_heads, c.seqlen), **f32)
    P = lambda t: None if t is None else t.data_ptr()
    stream = torch.cuda.current_stream()
    sh = stream.cuda_stream

    def step():
        if fused:
            N.check(lib.fp_estimate_select(p.ref, P(q), P(k), P(v), P(sc[0]), P(sc[1]), P(sc[2]), float(tau),
                                           P(qbar), P(kbar), P(vbar), P(row_ptr), P(col_idx), p.max_nnz,
                                           P(sched), P(ws), ws.numel(), sh))
            ev[1].record(stream)
            ev[2].record(stream)
        else:
            N.check(lib.fp_block_scores(p.ref, P(q), P(k), P(v), P(sc[0]), P(sc[1]), P(sc[2]), P(qbar),
                                        P(kbar), P(vbar), P(scores), sh))
            ev[1].record(stream)
            N.check(lib.fp_select_blocks(p.ref, P(scores), float(tau), P(row_ptr), P(col_idx), p.max_nnz,
                                         P(sched), P(ws), ws.numel(), sh))
            ev[2].record(stream)
        N.check(lib.fp_sparse_prefill(p.ref, P(q), P(k), P(v), P(sc[0]), P(sc[1]), P(sc[2]), P(kbar),
                                      P(vbar), P(row_ptr), P(col_idx), P(sched), P(o), P(lse), P(ws2),
                                      ws2.numel(), sh))

    ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
    flush = torch.empty(flush_bytes, dtype=torch.uint8, device=dev) if flush_bytes else None
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    t_est, t_sel, t_att = [], [], []
    all0 = torch.cuda.Event(enable_timing=True)
    all1 = torch.cuda.Event(enable_timing=True)
    per = []
    if sampler is not None:
        sampler.start()
    all0.record(stream)
    for _ in range(steps):
        e = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
        ev = e
        if flush is not None:
            flush.fill_(1)
        e[0].record(stream)
        step()
        e[3].record(stream)
        per.append(e)
    all1.record(stream)
    torch.cuda.synchronize()
    if sampler is not None:
        sampler.stop()
    total_ms = all0.elapsed_time(all1)
    t_all = []
    for e in per:
        t_est.append(e[0].elapsed_time(e[1]))
        t_sel.append(e[1].elapsed_time(e[2]))
        t_att.append(e[2].elapsed_time(e[3]))
        t_all.append(e[0].elapsed_time(e[3]))
    rp = row_ptr.cpu().numpy()
    ci = col_idx[:int(rp[-1])].cpu().numpy()
    G = c.num_q_heads // c.num_kv_heads
    kept, corr = kept_flops_from_csr(rp, ci, p.nb, c.seqlen, block, G, 128, c.num_kv_heads, c.batch)
    dense = 4.0 * 128 * c.num_q_heads * c.batch * c.seqlen * (c.seqlen + 1) / 2.0
    nblk = c.batch * c.num_kv_heads * p.nb * (p.nb + 1) / 2.0
    res = dict(
        label=label,
        # with flushes in between, the bracket would time them too: use the per-step events
        ms_per_step=total_ms / steps if flush is None else float(np.mean(t_all)),
        ms_step_median=float(np.median(t_all)),
        ms_estimate=float(np.mean(t_est)), ms_select=float(np.mean(t_sel)),
        ms_attention=float(np.mean(t_att)), ms_attention_median=float(np.median(t_att)),
        kept_fraction=float(len(ci) / nblk),
        kept_tflop=kept / 1e12, correction_tflop=corr / 1e12, dense_tflop=dense / 1e12,
    )
    res["dense_equiv_tflops"] = dense / (res["ms_per_step"] * 1e-3) / 1e12
    if getattr(inp, "meta", None):
        res["plants_kept"] = plants_kept(inp.meta, rp, ci, c.num_kv_heads, p.nb)
    res["attn_kept_tflops"] = kept / (res["ms_attention"] * 1e-3) / 1e12
    res["attn_executed_tflops"] = (kept + corr) / (res["ms_attention"] * 1e-3) / 1e12
    # estimator: reads Q, K, V once and writes pooled rows (+ the full score
    # matrix on the three-call path); selection reads the causal half of the
    # scores there and writes the CSR and schedule
    esz = 1 if inp.q.dtype == torch.uint8 else 2
    n_s = 0 if scores is None else scores.numel()
    est_bytes = (q.numel() + k.numel() + v.numel()) * esz + (qbar.numel() + kbar.numel() + vbar.numel()
                                                             + n_s) * 4
    sel_bytes = n_s * 4 // 2 + (len(ci) + 3 * p.rows) * 4
    res["ms_estimate_select"] = res["ms_estimate"] + res["ms_select"]
    if fused:
        res["estimate_gbs"] = (est_bytes + sel_bytes) / (res["ms_estimate_select"] * 1e-3) / 1e9
        res["select_gbs"] = None
    else:
        res["estimate_gbs"] = est_bytes / (res["ms_estimate"] * 1e-3) / 1e9
        res["select_gbs"] = sel_bytes / (res["ms_select"] * 1e-3) / 1e9
    outs = None
    if keep_outputs:
        outs = (o[0, :, :G].float().cpu().numpy(), lse[0, :G].cpu().numpy())
    del q, k, v, qbar, kbar, vbar, scores, o, lse, ws, ws2, flush
    torch.cuda.empty_cache()
    return res, (rp, ci, outs)


def time_dense(fp, inp, steps, warmup):
    """fp_dense_prefill (this library's dense causal attention on the same
    kernel: every block kept, no estimate, selection or correction) on the
    same tensors; HIP events on the current stream."""
    import torch
    dev = torch.device("cuda:0")
    mv = lambda t: None if t is None else t.to(dev)
    q, k, v = mv(inp.q), mv(inp.k), mv(inp.v)
    sc = dict(q_scale=mv(inp.q_scale), k_scale=mv(inp.k_scale), v_scale=mv(inp.v_scale))
    cfg = inp.cfg
    p = fp.make_problem(q, k, v, cfg.block)
    o = torch.empty((1, cfg.S, cfg.Hq, 128), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((1, cfg.Hq, cfg.S), dtype=torch.float32, device=dev)
    for _ in range(warmup):
        fp.fp_dense_prefill(p, q, k, v, o=o, **sc)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    ev = []
    for _ in range(steps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        fp.fp_dense_prefill(p, q, k, v, o=o, **sc)
        e1.record(stream)
        ev.append((e0, e1))
    torch.cuda.synchronize()
    ms = sorted(a.elapsed_time(b) for a, b in ev)
    dense = 4.0 * 128 * cfg.Hq * cfg.S * (cfg.S + 1) / 2.0
    med = ms[len(ms) // 2]
    del q, k, v, o, lse
    torch.cuda.empty_cache()
    return {"ms_median": med, "tflops": dense / (med * 1e-3) / 1e12}


def cpu_baseline(inp, tau, rows_sample=768, gpu=None):
    """The fp64 oracle, as it stands, single-threaded, on a bounded sample of
    the same workload: E1-E5 for one KV head group (all query blocks) and E6
    for `rows_sample` (KV head, query block) rows spread over the sequence;
    projected to the whole layer in dense-equivalent TFLOP/s. With the GPU's
    CSR and KV head 0 outputs given, the same oracle results also give parity
    statistics for that sample (outside the timed parts)."""
    from threadpoolctl import threadpool_limits
    import oracle
    from oracle.core import pool_queries, pool_keys, block_scores, select, attend
    cfg = inp.cfg
    S, B, Hq, Hkv = cfg.S, cfg.block, cfg.Hq, cfg.Hkv
    G = Hq // Hkv
    c = 1 / math.sqrt(128)
    nb = -(-S // B)
    # one BLAS thread, and this thread pinned to one of the cores it may use
    prev = os.sched_getaffinity(0) if hasattr(os, "sched_getaffinity") else None
    core = min(prev) if prev else None
    if core is not None:
        os.sched_setaffinity(0, {core})
    try:
        with threadpool_limits(limits=1):
            g = 0
            q = oracle.widen_bf16(inp.q[0, :, g * G:(g + 1) * G])
            k = oracle.widen_bf16(inp.k[0, :, g:g + 1])
            v = oracle.widen_bf16(inp.v[0, :, g:g + 1])
            t0 = time.perf_counter()
            qb = pool_queries(q, B, 0, S)
            kb, vb = pool_keys(k, B), pool_keys(v, B)
            Sc = block_scores(qb, kb, c, 0)
            keep, R_or = select(Sc, G, tau, 0)
            t_est = time.perf_counter() - t0
            il_list = np.linspace(0, nb - 1, rows_sample).round().astype(int)
            t0 = time.perf_counter()
            o_or, lse_or = attend(q, k, v, keep, kb, vb, c, B, 0, rows=[(0, int(il)) for il in il_list])
            t_att = time.perf_counter() - t0
    finally:
        if core is not None:
            os.sched_setaffinity(0, prev)
    parity = None if gpu is None else sample_parity(gpu, keep, R_or, o_or, lse_or, il_list, nb, B, tau)
    # projection: estimator time per group x Hkv; E6 time per row (evenly spaced
    # rows average the linear growth of row cost in i) x all rows
    t_layer = t_est * Hkv + t_att / rows_sample * (Hkv * nb)
    dense = 4.0 * 128 * Hq * S * (S + 1) / 2.0
    return dict(value=dense / t_layer / 1e12, unit="TFLOP/s (dense-equivalent)", cores=1,
                kind="oracle", host_cores=os.cpu_count(), host_cpu=host_cpu_model(), pinned_core=core,
                sample=(f"E1-E5 for KV head 0 (4 query heads, all {nb} query blocks): {t_est:.2f} s; "
                        f"E6 for {rows_sample} evenly spaced query blocks of KV head 0: {t_att:.2f} s; "
                        f"projected layer time {t_layer:.0f} s (x{Hkv} heads, x{nb} rows)"),
                measured_s=t_est + t_att, projected_layer_s=t_layer, parity=parity)


def host_cpu_model() -> str:
    """The host CPU's model name (first "model name" line of /proc/cpuinfo)."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


MASK_BAND = 1e-3          # a block may differ from the oracle's only where |R + tau| <= this
O_TOL_MAX, O_TOL_MEAN = 2e-2, 2e-3


def sample_parity(gpu, keep, R, o_or, lse_or, il_list, nb, B, tau):
    """GPU vs oracle on the cpu_baseline sample (KV head 0): kept lists of all
    query blocks, and o / lse of the sampled query blocks whose list equals
    the oracle's (rows whose lists differ inside the band are valid results
    of another mask and are counted, not compared)."""
    rp, ci, (o_gpu, lse_gpu) = gpu
    keep_gpu = np.zeros((nb, nb), dtype=bool)
    for il in range(nb):                           # rows (b=0, g=0, il) come first
        keep_gpu[il, ci[rp[il]:rp[il + 1]]] = True
    diff = keep_gpu != keep[0]
    band = np.abs(R[0] + tau) <= MASK_BAND
    out_of_band = int((diff & ~band).sum())
    same = [int(il) for il in np.unique(il_list) if not diff[il].any()]
    err, lerr = [], []
    for il in same:
        lo, hi = il * B, min((il + 1) * B, o_gpu.shape[0])
        err.append(np.abs(o_gpu[lo:hi] - o_or[lo:hi]).ravel())
        lerr.append(np.abs(lse_gpu[:, lo:hi] - lse_or[:, lo:hi]).ravel())
    err = np.concatenate(err) if err else np.zeros(1)
    lerr = np.concatenate(lerr) if lerr else np.zeros(1)
    return {"kv_head": 0, "mask_blocks": int(nb * (nb + 1) // 2), "mask_differs_in_band": int(diff.sum()) - out_of_band,
            "mask_differs_out_of_band": out_of_band,
            "rows_compared": len(same), "rows_skipped_mask_differs": len(np.unique(il_list)) - len(same),
            "o_max_abs": float(err.max()), "o_mean_abs": float(err.mean()), "lse_max_abs": float(lerr.max()),
            "tolerance": {"o_max_abs": O_TOL_MAX, "o_mean_abs": O_TOL_MEAN, "mask_band": MASK_BAND},
            "ok": bool(out_of_band == 0 and err.max() <= O_TOL_MAX and err.mean() <= O_TOL_MEAN)}


TRAFFIC_FILE = {kind: os.path.join(ROOT, "profiles", f"attn_{kind}_S131072_tau4_traffic.md") for kind in ("bf16", "fp8")}
# the attention kernel and the selection stage that orders its work (both shape its traffic)
KERNEL_SOURCES = [os.path.join(ROOT, "block_sparse_long_estimate_amd", "csrc", f) for f in ("k_attn.hip", "attn_geom.h", "k_select.hip")]


def measured_traffic(S, tau, kind="bf16"):
    """HBM bytes per attention launch from the committed rocprofv3 FETCH_SIZE /
    WRITE_SIZE readings (scaled by a plain copy kernel's readings), or None
    when they were taken on another workload or another version of the
    kernel or selection source. The record is the `key: value` block of the
    summary."""
    import hashlib
    try:
        with open(TRAFFIC_FILE[kind]) as f:
            rec = {}
            for line in f:
                key, sep, val = line.strip().partition(": ")
                if sep and key in ("kernel_source_sha256", "seq_len", "tau", "hbm_bytes_per_launch"):
                    rec[key] = val.strip()
        h = hashlib.sha256()
        for path in KERNEL_SOURCES:
            with open(path, "rb") as f:
                h.update(f.read())
        digest = h.hexdigest()
        if (rec.get("kernel_source_sha256") != digest or int(rec["seq_len"]) != S
                or float(rec["tau"]) != tau):
            return None
        return int(rec["hbm_bytes_per_launch"])
    except (OSError, KeyError, ValueError):
        return None


def input_hashes(inputs):
    """SHA-256 of the bytes of every input tensor, per format (q, k, v and, for
    fp8, the per-block scales), so a run can be matched to its inputs."""
    import hashlib
    import torch
    out = {}
    for kind, inp in inputs.items():
        d = {}
        for name in ("q", "k", "v", "q_scale", "k_scale", "v_scale"):
            t = getattr(inp, name, None)
            if t is None:
                continue
            t = t.contiguous()
            raw = t.view(torch.int16) if t.dtype == torch.bfloat16 else t
            d[name] = hashlib.sha256(memoryview(raw.numpy()).cast("B")).hexdigest()
        out[kind] = d
    return out


class ClockSampler:
    """Samples the GFX clock (MHz) of the GPU torch uses, through amdsmi, on a
    background thread between start() and stop(). Best effort: when amdsmi is
    missing or cannot identify the device, `result()` says why instead."""

    def __init__(self, period_s=0.01):
        import threading
        self.period, self.samples, self.error, self.handle = period_s, [], None, None
        self._stop = threading.Event()
        self._thread = threading.Thread(target=self._run, daemon=True)
        try:
            import amdsmi
            import torch
            self._smi = amdsmi
            amdsmi.amdsmi_init()
            pr = torch.cuda.get_device_properties(0)
            bdf = f"{pr.pci_domain_id:04x}:{pr.pci_bus_id:02x}:{pr.pci_device_id:02x}"
            handles = amdsmi.amdsmi_get_processor_handles()
            for h in handles:
                if str(amdsmi.amdsmi_get_gpu_device_bdf(h)).lower().startswith(bdf):
                    self.handle = h
            if self.handle is None:
                self.error = f"no amdsmi device at {bdf} among {len(handles)}"
        except Exception as e:          # a reading, never a reason to fail the bench
            self.error = f"amdsmi: {e!r}"

    def _run(self):
        while not self._stop.is_set():
            try:
                self.samples.append(float(self._smi.amdsmi_get_clock_info(self.handle,
                                                                          self._smi.AmdSmiClkType.GFX)["clk"]))
            except Exception as e:
                self.error = f"amdsmi: {e!r}"
                return
            self._stop.wait(self.period)

    def start(self):
        if self.handle is not None:
            self._thread.start()

    def stop(self):
        self._stop.set()
        if self._thread.is_alive():
            self._thread.join()

    def result(self):
        if not self.samples:
            return {"error": self.error or "no samples"}
        x = np.array(self.samples)
        return {"gfx_mhz_median": float(np.median(x)), "gfx_mhz_min": float(x.min()),
                "gfx_mhz_max": float(x.max()), "samples": int(len(x)), "period_ms": self.period * 1e3}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--tau", type=float, default=4.0)
    ap.add_argument("--seqlen", type=int, default=131072)
    ap.add_argument("--no-fp8", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-paged", action="store_true", help="skip the paged varlen batch leg")
    ap.add_argument("--no-cold", action="store_true", help="skip the cold-cache leg")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the smaller fixed-shape configurations (S=2048 and S=32768)")
    ap.add_argument("--no-ablation", action="store_true",
                    help="skip the error-vs-dense comparison with and without the mean correction")
    ap.add_argument("--no-unfused", action="store_true",
                    help="skip the three-call path (fp_block_scores + fp_select_blocks, score matrix in HBM)")
    ap.add_argument("--no-dense", action="store_true",
                    help="skip the dense baseline legs (fp_dense_prefill in bf16 and fp8)")
    ap.add_argument("--no-chunked", action="store_true",
                    help="skip the chunked-prefill leg (three chunks, with and without the pooled-KV cache)")
    ap.add_argument("--only-chunked", action="store_true",
                    help="run only the chunked-prefill leg and print its result")
    ap.add_argument("--no-clock", action="store_true",
                    help="skip the clock leg (GFX clock sampled while the bf16 path runs back to back)")
    ap.add_argument("--no-sweep", action="store_true",
                    help="skip the context legs (bf16 at tau 2/6/8, and tau=inf: every block kept)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB (3 times): the reference "
                         "kernel for scaling rocprofv3 FETCH_SIZE / WRITE_SIZE readings")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the path shards by KV head with no exchange; see the design notes)", file=sys.stderr)
        sys.exit(2)

    import torch
    if args.copy_calibration:
        n = args.copy_calibration << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": n, "launches": 3}), flush=True)
        return
    import synth
    import block_sparse_long_estimate_amd as fp
    import block_sparse_long_estimate_amd._native as N
    N.load()
    assert torch.cuda.is_available(), "bench.py needs a GPU"

    cfg = synth.config(3, S=args.seqlen, tau=args.tau)
    t0 = time.time()
    inputs = synth.gen_fixed_multi(cfg, ("bf16",) if args.no_fp8 else ("bf16", "fp8"))
    log(f"generated S={cfg.S} inputs in {time.time() - t0:.1f} s")
    if args.only_chunked:
        print(json.dumps({"chunked_prefill_bf16": time_chunked(fp, inputs["bf16"], args.tau)}), flush=True)
        return
    bf, bf_csr = time_path(fp, N, inputs["bf16"], args.tau, args.steps, args.warmup, "bf16",
                           keep_outputs=not args.no_cpu_baseline)
    log(f"bf16: {json.dumps(bf)}")
    # the clock the chip holds under this load: sampled over back-to-back steps
    # of the same path, outside the timed steps above
    clock = None
    if not args.no_clock:
        cs = ClockSampler()
        time_path(fp, N, inputs["bf16"], args.tau, 80, 2, "bf16 clock", sampler=cs)
        clock = {**cs.result(), "during": "80 back-to-back steps of the bf16 path above (about 1 s)",
                 "source": "amdsmi GFX clock"}
        log(f"clock: {json.dumps(clock)}")
    # cold caches: a 1 GiB write before each step evicts L2 and the memory-side cache
    cold = None
    if not args.no_cold:
        cold, _ = time_path(fp, N, inputs["bf16"], args.tau, 5, 1, "bf16 cold", flush_bytes=1 << 30)
        log(f"bf16 cold: {json.dumps(cold)}")
    f8 = None
    if not args.no_fp8:
        f8, _ = time_path(fp, N, inputs["fp8"], args.tau, args.steps, args.warmup, "fp8")
        log(f"fp8: {json.dumps(f8)}")
    configs = {}
    if not args.no_configs:
        for cid in (1, 2):
            c = synth.config(cid)
            ci_inp = synth.gen_fixed(c)
            r, _ = time_path(fp, N, ci_inp, c.tau, 10, 3, f"config {cid}")
            configs[c.name] = {"seq_len": c.S, "heads": f"{c.Hq}/{c.Hkv}", "block": c.block, "tau": c.tau,
                               "ms_per_layer_median": round(r["ms_step_median"], 4),
                               "ms_attention_median": round(r["ms_attention_median"], 4),
                               "dense_equiv_tflops": round(r["dense_equiv_tflops"], 2),
                               "kept_fraction": round(r["kept_fraction"], 5),
                               "mfma_util_kept": round(r["attn_kept_tflops"] / PEAK_TFLOPS["bf16"], 4),
                               "ms_per_layer_graph_replay": round(graph_replay_ms(fp, ci_inp, c.tau), 4)}
            if cid == 1:
                # the same problem with its rows split over several workgroups (it has 32 units)
                rs, _ = time_path(fp, N, ci_inp, c.tau, 10, 3, f"config {cid} split", split_small=True)
                configs[c.name]["split_small"] = {"ms_per_layer_median": round(rs["ms_step_median"], 4),
                                                  "ms_attention_median": round(rs["ms_attention_median"], 4),
                                                  "mfma_util_kept": round(rs["attn_kept_tflops"] / PEAK_TFLOPS["bf16"],
                                                                          4)}
            log(f"config {cid}: {json.dumps(configs[c.name])}")
    paged = paged8 = None
    if not args.no_paged:
        paged = time_paged(fp, N, 5, 1)
        log(f"paged varlen: {json.dumps(paged)}")
        if not args.no_fp8:
            paged8 = time_paged(fp, N, 5, 1, "fp8")
            log(f"paged varlen fp8: {json.dumps(paged8)}")
    chunked = None
    if not args.no_chunked:
        chunked = time_chunked(fp, inputs["bf16"], args.tau)
        log(f"chunked prefill: {json.dumps(chunked)}")
    sweep, dense = {}, None
    if not args.no_sweep:
        for tau in (2.0, 6.0, 8.0):
            r, _ = time_path(fp, N, inputs["bf16"], tau, 5, 1, f"bf16 tau={tau}")
            sweep[str(tau)] = {"ms_per_layer": round(r["ms_per_step"], 4), "ms_attention": round(r["ms_attention"], 4),
                               "kept_fraction": round(r["kept_fraction"], 5), "plants_kept": r.get("plants_kept"),
                               "attn_kept_tflops": round(r["attn_kept_tflops"], 2)}
            log(f"sweep tau={tau}: {json.dumps(sweep[str(tau)])}")
        dense, _ = time_path(fp, N, inputs["bf16"], float("inf"), 2, 1, "bf16 dense")
        log(f"dense (tau=inf): {json.dumps(dense)}")
    three_call = {}
    if not args.no_unfused:
        # the same workload through the three-call path (score matrix in HBM)
        for kind in ("bf16", "fp8"):
            if kind not in inputs:
                continue
            r, _ = time_path(fp, N, inputs[kind], args.tau, 10, 3, f"{kind} three calls", fused=False)
            three_call[kind] = {"ms_per_layer_median": round(r["ms_step_median"], 4),
                                "ms_estimate": round(r["ms_estimate"], 4), "ms_select": round(r["ms_select"], 4),
                                "estimator_gbs": round(r["estimate_gbs"], 1),
                                "select_gbs": round(r["select_gbs"], 1)}
            log(f"three-call path {kind}: {json.dumps(three_call[kind])}")
    dense_base = {}
    if not args.no_dense:
        for kind, res in (("bf16", bf), ("fp8", f8)):
            if res is None:
                continue
            d = time_dense(fp, inputs[kind], 3, 1)
            dense_base[kind] = {"ms_attention_median": round(d["ms_median"], 4), "tflops": round(d["tflops"], 2),
                                "mfma_util": round(d["tflops"] / PEAK_TFLOPS[kind], 4),
                                "sparse_speedup_attention": round(d["ms_median"] / res["ms_attention_median"], 2),
                                "sparse_speedup_layer": round(d["ms_median"] / res["ms_step_median"], 2)}
            log(f"dense baseline {kind}: {json.dumps(dense_base[kind])}")
    ablation = None
    if not args.no_ablation:
        ablation = ablation_vs_dense(fp, inputs["bf16"])
        log(f"ablation vs dense: {json.dumps(ablation)}")
    cpu = None
    if not args.no_cpu_baseline:
        t0 = time.time()
        cpu = cpu_baseline(inputs["bf16"], args.tau, gpu=bf_csr)
        log(f"cpu baseline ({time.time() - t0:.1f} s): {json.dumps(cpu)}")

    att_peak = PEAK_TFLOPS["bf16"]
    line = {
        "metric": "prefill attn ms/layer + dense-equiv TFLOP/s at 128K GQA bf16/fp8; MFMA util",
        "value": round(bf["dense_equiv_tflops"], 2),
        "unit": "TFLOP/s (dense-equivalent)",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(bf["ms_per_step"], 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": f"one layer, S={cfg.S}, 32 query / 8 KV heads, head dim 128, "
                               f"128x128 blocks, tau={args.tau}, random-walk K/V with sink and "
                               f"16 planted blocks per KV head, seed {cfg.seed}",
                   "seq_len": cfg.S, "batch": 1, "tau": args.tau, "block": 128},
        "kept_fraction": round(bf["kept_fraction"], 5),
        "plants_kept": bf.get("plants_kept"),
        "path": "fp_estimate_select (pooling + fused block scores/threshold/CSR/schedule, no score matrix) "
                "+ fp_sparse_prefill",
        "ms_per_layer": {"total": round(bf["ms_per_step"], 4),
                         "estimate_select": round(bf["ms_estimate_select"], 4),
                         "attention": round(bf["ms_attention"], 4)},
        "ms_per_layer_median": {"total": round(bf["ms_step_median"], 4),
                                "attention": round(bf["ms_attention_median"], 4)},
        "mfma_util_kept": round(bf["attn_kept_tflops"] / att_peak, 4),
        "mfma_util_executed": round(bf["attn_executed_tflops"] / att_peak, 4),
        "estimate_select_gbs": round(bf["estimate_gbs"], 1),
        "estimate_select_hbm_frac": round(bf["estimate_gbs"] / HBM_GBS, 4),
        "roofline": {"bound": "mfma", "kernel": "attn_tile_kernel<128, bf16> (fp_sparse_prefill)",
                     "achieved": round(bf["attn_kept_tflops"], 2), "peak": att_peak,
                     "unit": "TFLOP/s", "frac": round(bf["attn_kept_tflops"] / att_peak, 4),
                     "traffic": measured_traffic(cfg.S, args.tau)},
    }
    if f8 is not None:
        line["fp8"] = {"ms_per_layer": round(f8["ms_per_step"], 4),
                       "dense_equiv_tflops": round(f8["dense_equiv_tflops"], 2),
                       "ms_attention": round(f8["ms_attention"], 4),
                       "kept_fraction": round(f8["kept_fraction"], 5),
                       "attn_kept_tflops": round(f8["attn_kept_tflops"], 2),
                       "mfma_util_kept": round(f8["attn_kept_tflops"] / PEAK_TFLOPS["fp8"], 4),
                       "ms_estimate_select": round(f8["ms_estimate_select"], 4),
                       "estimate_select_gbs": round(f8["estimate_gbs"], 1),
                       "traffic": measured_traffic(cfg.S, args.tau, "fp8"),
                       "roofline": {"bound": "mfma", "kernel": "attn_tile_kernel<128, fp8> (fp_sparse_prefill)",
                                    "achieved": round(f8["attn_kept_tflops"], 2), "peak": PEAK_TFLOPS["fp8"],
                                    "unit": "TFLOP/s", "frac": round(f8["attn_kept_tflops"] / PEAK_TFLOPS["fp8"], 4),
                                    "traffic": measured_traffic(cfg.S, args.tau, "fp8")},
                       "bf16_over_fp8_attention_time": round(bf["ms_attention_median"] / f8["ms_attention_median"], 3),
                       "bf16_over_fp8_context": "1.74x on H20 (47.26 / 27.19, the pages' speedups over "
                                                "FlashAttention-2 in fp8 and bf16), other hardware"}
    if clock is not None:
        line["gpu_clock"] = clock
    line["inputs_sha256"] = input_hashes(inputs)
    if cold is not None:
        line["cold_cache"] = {"runs": 5, "flush": "1 GiB written before each step",
                              "ms_per_layer_median": round(cold["ms_step_median"], 4),
                              "ms_attention_median": round(cold["ms_attention_median"], 4)}
    if configs:
        line["other_configs_bf16"] = configs
    if paged is not None:
        line["paged_varlen_bf16"] = paged
    if paged8:
        line["paged_varlen_fp8"] = paged8
    if chunked is not None:
        line["chunked_prefill_bf16"] = chunked
    if sweep:
        line["tau_sweep_bf16"] = sweep
    if dense is not None:
        # the same path with every block kept: this library's own dense causal attention
        line["dense_path_bf16"] = {"ms_per_layer": round(dense["ms_per_step"], 4),
                                   "ms_attention": round(dense["ms_attention"], 4),
                                   "attn_tflops": round(dense["attn_kept_tflops"], 2),
                                   "mfma_util": round(dense["attn_kept_tflops"] / att_peak, 4),
                                   "sparse_speedup": round(dense["ms_per_step"] / bf["ms_per_step"], 2)}
    if three_call:
        line["three_call_path"] = three_call
    if dense_base:
        # fp_dense_prefill: every block kept, no estimate/selection/correction
        dense_base["context"] = ("the pages' H20 speedups at 128K, for context only (other hardware, other "
                                 "dense kernels): 27.19x bf16 and 47.26x fp8 over FlashAttention-2, 30.49x fp8 "
                                 "over an FA3/4-aligned dense kernel")
        line["dense_baseline"] = dense_base
    if ablation is not None:
        line["error_vs_dense_bf16"] = ablation
    if cpu is not None:
        line["cpu_baseline"] = {k: cpu[k] for k in ("value", "unit", "cores", "kind", "sample", "host_cores",
                                                    "host_cpu", "pinned_core")}
        line["cpu_baseline"]["value"] = round(cpu["value"], 6)
        line["parity_sample"] = cpu["parity"]
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
