"""Host-side pieces of bench.py (no GPU): the FLOP accounting from a CSR,
the sample parity statistics, the traffic record check and the one-GPU
guard."""
import os
import subprocess
import sys

import numpy as np

import bench
import oracle.core as oc

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def csr_from_keep(keep):
    """Rows (b = 0, g, i), ascending columns."""
    rp, ci = [0], []
    for g in range(keep.shape[0]):
        for il in range(keep.shape[1]):
            cols = np.nonzero(keep[g, il])[0]
            ci.extend(cols.tolist())
            rp.append(len(ci))
    return np.array(rp, dtype=np.int64), np.array(ci, dtype=np.int64)


def test_kept_and_correction_flops_match_oracle_counts():
    """S = 600 with 128-token blocks (ragged last block), 2 KV heads, G = 3."""
    S, B, Hkv, G, d = 600, 128, 2, 3, 128
    nb = -(-S // B)
    rng = np.random.default_rng(7)
    keep = np.zeros((Hkv, nb, nb), dtype=bool)
    for g in range(Hkv):
        for i in range(nb):
            keep[g, i, :i + 1] = rng.random(i + 1) < 0.5
            keep[g, i, 0] = keep[g, i, i] = True
    rp, ci = csr_from_keep(keep)
    kept, corr = bench.kept_flops_from_csr(rp, ci, nb, S, B, G, d, Hkv, 1)
    assert kept == oc.kept_flops(keep, 0, S, B, d, G)
    assert corr == oc.correction_flops(keep, 0, S, B, d, G)
    # every block kept: the dense causal count
    full = np.tril(np.ones((nb, nb), dtype=bool))[None].repeat(Hkv, 0)
    rp, ci = csr_from_keep(full)
    kept, corr = bench.kept_flops_from_csr(rp, ci, nb, S, B, G, d, Hkv, 1)
    assert kept == oc.dense_flops(0, S, d, G * Hkv)
    assert corr == 0.0


def _parity_case(nb=6, B=4, G=2, tau=1.0):
    rng = np.random.default_rng(3)
    S = nb * B
    R = -rng.random((1, nb, nb)) * 3.0
    keep = (R >= -tau)
    for i in range(nb):
        keep[0, i, 0] = keep[0, i, i] = True
        keep[0, i, i + 1:] = False
    o_or = rng.standard_normal((S, G, 8))
    lse_or = rng.standard_normal((G, S))
    rp, ci = csr_from_keep(keep)
    return S, R, keep, o_or, lse_or, rp, ci


def test_sample_parity_clean_and_perturbed():
    nb, B, tau = 6, 4, 1.0
    S, R, keep, o_or, lse_or, rp, ci = _parity_case(nb, B, tau=tau)
    il_list = np.arange(nb)
    st = bench.sample_parity((rp, ci, (o_or.copy(), lse_or.copy())), keep, R, o_or, lse_or, il_list, nb, B,
                             tau)
    assert st["ok"] and st["o_max_abs"] == 0.0 and st["rows_compared"] == nb
    assert st["mask_differs_in_band"] == 0 and st["mask_differs_out_of_band"] == 0
    # an output error above the bound in one row is reported and fails
    o_bad = o_or.copy()
    o_bad[2 * B, 1, 3] += 0.05
    st = bench.sample_parity((rp, ci, (o_bad, lse_or)), keep, R, o_or, lse_or, il_list, nb, B, tau)
    assert not st["ok"] and abs(st["o_max_abs"] - 0.05) < 1e-12


def test_sample_parity_mask_bands():
    nb, B, tau = 6, 4, 1.0
    S, R, keep, o_or, lse_or, rp, ci = _parity_case(nb, B, tau=tau)
    # flip one off-diagonal block of row 4: out of band unless R is within 1e-3 of -tau
    i, j = 4, 2
    keep2 = keep.copy()
    keep2[0, i, j] = not keep2[0, i, j]
    rp2, ci2 = csr_from_keep(keep2)
    R_far = R.copy()
    R_far[0, i, j] = -tau + 0.5
    st = bench.sample_parity((rp2, ci2, (o_or, lse_or)), keep, R_far, o_or, lse_or, np.arange(nb), nb, B, tau)
    assert st["mask_differs_out_of_band"] == 1 and not st["ok"]
    R_near = R.copy()
    R_near[0, i, j] = -tau + 5e-4
    st = bench.sample_parity((rp2, ci2, (o_or, lse_or)), keep, R_near, o_or, lse_or, np.arange(nb), nb, B, tau)
    assert st["mask_differs_in_band"] == 1 and st["mask_differs_out_of_band"] == 0
    assert st["rows_skipped_mask_differs"] == 1 and st["rows_compared"] == nb - 1 and st["ok"]


def test_traffic_record_requires_matching_workload():
    assert bench.measured_traffic(1234, 4.0) is None
    assert bench.measured_traffic(131072, 2.5) is None


def test_input_hashes_are_sha256_of_the_tensor_bytes():
    """The bench line's input hashes are plain SHA-256 over each tensor's
    bytes (bf16 as its 16-bit patterns, fp8 codes and fp32 scales as stored)."""
    import hashlib
    import synth
    out = bench.input_hashes({"bf16": synth.gen_fixed(synth.config(1)),
                              "fp8": synth.gen_fixed(synth.config(4, S=300, Hq=4, Hkv=1))})
    assert set(out["bf16"]) == {"q", "k", "v"}
    assert set(out["fp8"]) == {"q", "k", "v", "q_scale", "k_scale", "v_scale"}
    q = synth.gen_fixed(synth.config(1)).q
    assert out["bf16"]["q"] == hashlib.sha256(q.view(__import__("torch").int16).numpy().tobytes()).hexdigest()
    for d in out.values():
        assert all(len(h) == 64 for h in d.values())


def test_plants_kept_reads_the_row_of_each_plant():
    """Rows are (sequence, KV head, query block): a plant (g, i, j) is kept
    when column j is in row (b * Hkv + g) * nb + i."""
    from types import SimpleNamespace as NS
    Hkv, nb = 2, 4
    keep = np.zeros((2 * Hkv * nb, nb), dtype=bool)
    keep[(0 * Hkv + 1) * nb + 3, 1] = True            # sequence 0, head 1, block 3 keeps column 1
    keep[(1 * Hkv + 0) * nb + 2, 0] = True            # sequence 1, head 0, block 2 keeps column 0
    rp, ci = [0], []
    for r in range(keep.shape[0]):
        ci.extend(np.nonzero(keep[r])[0].tolist())
        rp.append(len(ci))
    metas = [NS(plants=[(1, 3, 1, 1.0), (1, 3, 2, 1.0)]), NS(plants=[(0, 2, 0, 1.0), (1, 2, 0, 1.0)])]
    assert bench.plants_kept(metas, np.array(rp), np.array(ci), Hkv, nb) == [2, 4]


def test_clock_sampler_reports_instead_of_failing_without_a_device():
    cs = bench.ClockSampler(period_s=0.001)
    cs.start()
    cs.stop()
    r = cs.result()
    assert "error" in r or r["samples"] >= 1


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stderr


def test_varlen_flops_match_oracle_counts():
    """Two sequences with cached prefixes that start mid-block."""
    B, Hkv, G, d = 64, 2, 2, 128
    L, P = [300, 200], [70, 0]
    rng = np.random.default_rng(11)
    rps, cis, keeps = [0], [], []
    for Lb, Pb in zip(L, P):
        i0, nq = oc.query_blocks(Pb, Lb, B)
        nb = oc.nblocks(Lb, B)
        keep = np.zeros((Hkv, nq, nb), dtype=bool)
        for g in range(Hkv):
            for il in range(nq):
                i = i0 + il
                keep[g, il, :i + 1] = rng.random(i + 1) < 0.5
                keep[g, il, 0] = keep[g, il, i] = True
                cols = np.nonzero(keep[g, il])[0]
                cis.extend(cols.tolist())
                rps.append(len(cis))
        keeps.append(keep)
    rp, ci = np.array(rps), np.array(cis)
    kept, corr, dense = bench.varlen_flops(rp, ci, L, P, B, G, d, Hkv)
    assert kept == sum(oc.kept_flops(k, Pb, Lb, B, d, G) for k, Lb, Pb in zip(keeps, L, P))
    assert corr == sum(oc.correction_flops(k, Pb, Lb, B, d, G) for k, Lb, Pb in zip(keeps, L, P))
    assert dense == sum(oc.dense_flops(Pb, Lb, d, G * Hkv) for Lb, Pb in zip(L, P))


def test_schedule_groups_rule():
    """The schedule-group rule on the benchmark shapes: S = 131072 with 8 KV
    heads pairs the heads in bf16 (64 MiB of K and V each) and takes four in
    fp8; S = 32768 and the longest single-head sequence form one group."""
    from fp_testutil import fixed_sched_groups
    g = fixed_sched_groups(1, 8, 1024, 128, 2)
    assert g.reshape(8, 1024)[:, 0].tolist() == [0, 0, 1, 1, 2, 2, 3, 3]
    g = fixed_sched_groups(1, 8, 1024, 128, 1)
    assert g.reshape(8, 1024)[:, 0].tolist() == [0, 0, 0, 0, 1, 1, 1, 1]
    assert fixed_sched_groups(1, 8, 256, 128, 2).max() == 0
    assert fixed_sched_groups(1, 1, 16384, 128, 2).max() == 0
