"""The whole fixed-shape path driven by a plain C99 program (tests/c/abi_run.c,
built by __graft_entry__.build()) through the C ABI, with its own hipMalloc'd
buffers and stream: its kept lists, schedule, outputs and lse must equal, bit
for bit, those of the Python binding on the same inputs, and match the oracle
like any other run."""
import os
import subprocess

import numpy as np
import pytest
import torch

import synth
from test_gpu_parity import check_fixed, fp, say  # noqa: F401  (fp is a fixture)

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
EXE = os.path.join(ROOT, "tests", "c", "abi_run")


@pytest.mark.parametrize("S,block", [(4096 + 77, 128), (2048 + 5, 64)])
def test_c_program_runs_the_whole_path(fp, tmp_path, S, block):
    assert os.path.exists(EXE), "tests/c/abi_run is missing: run __graft_entry__.build() first"
    cfg = synth.config(2, S=S, Hq=8, Hkv=2, block=block, seed=211 + block, tau=2.0)
    inp = synth.gen_fixed(cfg)
    for name, t in (("q", inp.q), ("k", inp.k), ("v", inp.v)):
        t[0].contiguous().view(torch.int16).numpy().tofile(str(tmp_path / f"{name}.bin"))
    (tmp_path / "meta.txt").write_text(f"{S} {cfg.Hq} {cfg.Hkv} {block} {cfg.tau}\n")
    say(f"C program: S={S} block={block}")
    r = subprocess.run([EXE, str(tmp_path)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0 and r.stdout.startswith("ok"), r.stdout + r.stderr

    dev = torch.device("cuda:0")
    q, k, v = (t.to(dev) for t in (inp.q, inp.k, inp.v))
    out = fp.sparse_prefill(q, k, v, block, cfg.tau)
    torch.cuda.synchronize()
    rp = out["row_ptr"].cpu().numpy()
    nnz = int(rp[-1])
    assert np.array_equal(np.fromfile(tmp_path / "row_ptr.bin", dtype=np.int32), rp)
    assert np.array_equal(np.fromfile(tmp_path / "col_idx.bin", dtype=np.int32), out["col_idx"][:nnz].cpu().numpy())
    assert np.array_equal(np.fromfile(tmp_path / "sched.bin", dtype=np.int32), out["sched"].cpu().numpy())
    o_c = np.fromfile(tmp_path / "o.bin", dtype=np.int16).reshape(S, cfg.Hq, 128)
    assert np.array_equal(o_c, out["o"][0].cpu().view(torch.int16).numpy())
    lse_c = np.fromfile(tmp_path / "lse.bin", dtype=np.float32).reshape(cfg.Hq, S)
    assert np.array_equal(lse_c.view(np.int32), out["lse"][0].cpu().numpy().view(np.int32))
    check_fixed(fp, inp, cfg.tau, block)


def test_c_program_runs_the_paged_path(fp, tmp_path):
    """fp_sparse_prefill_paged from C: a bf16 batch of three sequences with
    cached prefixes in a shuffled 32-token page pool."""
    from test_gpu_parity import check_paged, run_paged
    assert os.path.exists(EXE), "tests/c/abi_run is missing: run __graft_entry__.build() first"
    cfg = synth.config(5, Hq=8, Hkv=2, n_seqs=3, len_range=(300, 3000), page_size=32, tau=2.0, seed=223)
    L, P = synth.paged_lengths(cfg)
    P[2] = 0
    inp = synth.gen_paged(cfg, (L, P))
    n_pages, page = inp.k_cache.shape[0], inp.k_cache.shape[1]
    max_pages = inp.block_table.shape[1]
    inp.q.contiguous().view(torch.int16).numpy().tofile(str(tmp_path / "q.bin"))
    inp.k_cache.contiguous().view(torch.int16).numpy().tofile(str(tmp_path / "k_cache.bin"))
    inp.v_cache.contiguous().view(torch.int16).numpy().tofile(str(tmp_path / "v_cache.bin"))
    inp.block_table.contiguous().numpy().astype(np.int32).tofile(str(tmp_path / "block_table.bin"))
    np.asarray(inp.cu_seqlens_q, dtype=np.int32).tofile(str(tmp_path / "cu_seqlens_q.bin"))
    np.asarray(inp.seqlens_k, dtype=np.int32).tofile(str(tmp_path / "seqlens_k.bin"))
    (tmp_path / "meta.txt").write_text(
        f"{len(L)} {cfg.Hq} {cfg.Hkv} {cfg.block} {page} {n_pages} {max_pages} {cfg.tau}\n")
    say(f"C program, paged: L={L.tolist()} P={P.tolist()} page={page}")
    r = subprocess.run([EXE, "paged", str(tmp_path)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0 and r.stdout.startswith("ok"), r.stdout + r.stderr

    o, lse, rp, ci = run_paged(fp, inp, cfg.tau)
    nnz = int(rp[-1])
    nq = int(inp.cu_seqlens_q[-1])
    assert np.array_equal(np.fromfile(tmp_path / "row_ptr.bin", dtype=np.int32), rp)
    assert np.array_equal(np.fromfile(tmp_path / "col_idx.bin", dtype=np.int32), ci[:nnz])
    o_c = np.fromfile(tmp_path / "o.bin", dtype=np.int16).reshape(nq, cfg.Hq, 128)
    assert np.array_equal(o_c, o.view(torch.int16).numpy())
    lse_c = np.fromfile(tmp_path / "lse.bin", dtype=np.float32).reshape(cfg.Hq, nq)
    assert np.array_equal(lse_c.view(np.int32), lse.numpy().view(np.int32))
    check_paged(fp, inp, cfg.tau)
