"""C-ABI checks that need no GPU: the library loads, exports every symbol the
header declares, sizes problems, and rejects bad arguments before any HIP call."""
import ctypes
import math
import os
import re

import numpy as np
import pytest

import block_sparse_long_estimate_amd._native as N

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fp_prefill.h")


def header_functions():
    with open(HEADER) as fh:
        text = fh.read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z0-9_]+\s*\*?\s*(fp_[a-z_]+)\s*\(", text, re.M)))


def test_library_exports_every_declared_symbol():
    lib = N.load()
    names = header_functions()
    assert len(names) >= 12
    assert set(names) == set(N.EXPORTS)
    for name in names:
        assert hasattr(lib, name), name
    assert b"gfx950" in lib.fp_version()


def problem(**kw):
    c = N.FpProblem()
    c.batch, c.seqlen, c.num_q_heads, c.num_kv_heads = 1, 1024, 8, 2
    c.head_dim, c.block, c.dtype, c.softmax_scale = 128, 128, 0, 0.0
    for name, H in (("q_stride", 8), ("k_stride", 2), ("v_stride", 2), ("o_stride", 8)):
        arr = getattr(c, name)
        arr[0], arr[1], arr[2] = 1024 * H * 128, H * 128, 128
    for k, v in kw.items():
        setattr(c, k, v)
    return c


def test_sizes():
    lib = N.load()
    p = problem()
    nb = 8
    assert lib.fp_num_rows(ctypes.byref(p)) == 2 * nb
    assert lib.fp_max_nnz(ctypes.byref(p)) == 2 * nb * (nb + 1) // 2
    assert lib.fp_workspace_size(ctypes.byref(p)) > 0
    p = problem(seqlen=1000, block=64)
    assert lib.fp_num_rows(ctypes.byref(p)) == 2 * 16


def test_largest_supported_sequence():
    """16384 blocks of 128 tokens is the longest sequence; one more token is refused."""
    lib = N.load()
    p = problem(seqlen=16384 * 128, num_q_heads=1, num_kv_heads=1)
    for arr in (p.q_stride, p.k_stride, p.v_stride, p.o_stride):
        arr[0], arr[1], arr[2] = 16384 * 128 * 128, 128, 128
    assert lib.fp_num_rows(ctypes.byref(p)) == 16384
    assert lib.fp_max_nnz(ctypes.byref(p)) == 16384 * 16385 // 2


@pytest.mark.parametrize("field,value,code", [
    ("num_q_heads", 7, N.FP_ERR_INVALID),          # Hq % Hkv != 0
    ("head_dim", 64, N.FP_ERR_UNSUPPORTED),
    ("block", 32, N.FP_ERR_UNSUPPORTED),
    ("block", 96, N.FP_ERR_UNSUPPORTED),
    ("dtype", 7, N.FP_ERR_UNSUPPORTED),
    ("batch", 0, N.FP_ERR_INVALID),
    ("seqlen", -5, N.FP_ERR_INVALID),
    ("seqlen", 0, N.FP_ERR_INVALID),                 # empty sequence
    ("seqlen", 16384 * 128 + 1, N.FP_ERR_UNSUPPORTED),   # one block past the 16384-block limit
    ("softmax_scale", float("nan"), N.FP_ERR_INVALID),
    ("num_kv_heads", 0, N.FP_ERR_INVALID),
])
def test_invalid_problems(field, value, code):
    lib = N.load()
    p = problem(**{field: value})
    assert lib.fp_num_rows(ctypes.byref(p)) == code
    assert len(lib.fp_last_error()) > 0
    fake = ctypes.c_void_p(1 << 20)
    assert lib.fp_block_scores(ctypes.byref(p), fake, fake, fake, None, None, None,
                               fake, fake, fake, fake, None) == code


def test_group_limit_and_block_count_limit():
    lib = N.load()
    p = problem(num_q_heads=34, num_kv_heads=2)       # G = 17
    assert lib.fp_num_rows(ctypes.byref(p)) == N.FP_ERR_UNSUPPORTED
    p = problem(seqlen=16385 * 128)
    assert lib.fp_num_rows(ctypes.byref(p)) == N.FP_ERR_UNSUPPORTED


def test_null_pointers_and_fp8_scales():
    lib = N.load()
    p = problem()
    fake = ctypes.c_void_p(1 << 20)
    assert lib.fp_block_scores(ctypes.byref(p), None, fake, fake, None, None, None,
                               fake, fake, fake, fake, None) == N.FP_ERR_INVALID
    assert b"NULL" in lib.fp_last_error()
    p8 = problem(dtype=1)
    for name, H in (("q_stride", 8), ("k_stride", 2), ("v_stride", 2)):
        arr = getattr(p8, name)
        arr[0], arr[1], arr[2] = 1024 * H * 128, H * 128, 128
    assert lib.fp_block_scores(ctypes.byref(p8), fake, fake, fake, None, None, None,
                               fake, fake, fake, fake, None) == N.FP_ERR_INVALID
    assert b"scale" in lib.fp_last_error()
    assert lib.fp_sparse_prefill(ctypes.byref(p), fake, fake, fake, None, None, None, fake, fake,
                                 None, fake, None, fake, None, fake, 1 << 30, None) == N.FP_ERR_INVALID
    # workspace below fp_prefill_workspace_size
    need = lib.fp_prefill_workspace_size(ctypes.byref(p))
    assert need == 3 * (1 * 2 * (1024 // 128)) * 128 * 2     # hi, lo, v copies, bf16
    assert lib.fp_sparse_prefill(ctypes.byref(p), fake, fake, fake, None, None, None, fake, fake,
                                 fake, fake, None, fake, None, fake, need - 1, None) == N.FP_ERR_CAPACITY
    assert b"workspace" in lib.fp_last_error()


def test_misaligned_strides_rejected():
    lib = N.load()
    p = problem()
    p.q_stride[1] = 8 * 128 + 4                      # 8-byte aligned only
    assert lib.fp_num_rows(ctypes.byref(p)) == N.FP_ERR_INVALID


def test_select_rejects_nan_tau_capacity_and_workspace():
    lib = N.load()
    p = problem()
    fake = ctypes.c_void_p(1 << 20)
    need = lib.fp_max_nnz(ctypes.byref(p))
    ws = lib.fp_workspace_size(ctypes.byref(p))
    assert lib.fp_select_blocks(ctypes.byref(p), fake, float("nan"), fake, fake, need, None,
                                fake, ws, None) == N.FP_ERR_INVALID
    assert b"NaN" in lib.fp_last_error()
    assert lib.fp_select_blocks(ctypes.byref(p), fake, 4.0, fake, fake, need - 1, None,
                                fake, ws, None) == N.FP_ERR_CAPACITY
    assert lib.fp_select_blocks(ctypes.byref(p), fake, 4.0, fake, fake, need, None,
                                fake, ws - 1, None) == N.FP_ERR_CAPACITY
    assert lib.fp_select_blocks(ctypes.byref(p), fake, 4.0, fake, fake, need, None,
                                ctypes.c_void_p((1 << 20) + 8), ws, None) == N.FP_ERR_INVALID


def vproblem(**kw):
    c = N.FpVarlenProblem()
    c.num_seqs, c.num_q_heads, c.num_kv_heads, c.head_dim = 3, 8, 2, 128
    c.block, c.page_size, c.dtype, c.softmax_scale = 128, 64, 0, 0.0
    c.max_pages_per_seq = 64
    c.q_stride[0], c.q_stride[1] = 8 * 128, 128
    c.kv_stride[0], c.kv_stride[1], c.kv_stride[2] = 64 * 2 * 128, 2 * 128, 128
    c.o_stride[0], c.o_stride[1] = 8 * 128, 128
    for k, v in kw.items():
        setattr(c, k, v)
    return c


def arr(x):
    a = np.ascontiguousarray(np.asarray(x, dtype=np.int32))
    return a, a.ctypes.data_as(ctypes.c_void_p)


def test_varlen_sizes_match_a_direct_count():
    lib = N.load()
    p = vproblem()
    cu, cup = arr([0, 300, 300, 1000])        # middle sequence has no new rows
    lk, lkp = arr([500, 200, 1000])
    rows = lib.fp_varlen_num_rows(ctypes.byref(p), cup, lkp)
    nnz = lib.fp_varlen_max_nnz(ctypes.byref(p), cup, lkp)
    exp_rows, exp_nnz = 0, 0
    for b in range(3):
        ql = cu[b + 1] - cu[b]
        if ql == 0:
            continue
        P = lk[b] - ql
        for i in range(P // 128, (lk[b] - 1) // 128 + 1):
            exp_rows += 2
            exp_nnz += 2 * (i + 1)
    assert rows == exp_rows and nnz == exp_nnz
    assert lib.fp_varlen_workspace_size(ctypes.byref(p), cup, lkp) > 0


@pytest.mark.parametrize("cu,lk,kw,code", [
    ([0, 300, 200, 1000], [500, 200, 1000], {}, N.FP_ERR_INVALID),     # cu not monotone
    ([0, 300, 400, 1000], [200, 200, 1000], {}, N.FP_ERR_INVALID),     # L < q_len
    ([1, 300, 400, 1000], [500, 200, 1000], {}, N.FP_ERR_INVALID),     # cu[0] != 0
    ([0, 300, 400, 1000], [500, 200, 1000], {"page_size": 48}, N.FP_ERR_UNSUPPORTED),
    ([0, 300, 400, 1000], [500, 200, 1000], {"dtype": 7}, N.FP_ERR_UNSUPPORTED),
    ([0, 300, 400, 1000], [500, 200, 1000], {"max_pages_per_seq": 8}, N.FP_ERR_INVALID),
    ([0, 300, 400, 1000], [500, 200, 1000], {"num_seqs": 0}, N.FP_ERR_INVALID),
])
def test_varlen_invalid(cu, lk, kw, code):
    lib = N.load()
    p = vproblem(**kw)
    _, cup = arr(cu)
    _, lkp = arr(lk)
    assert lib.fp_varlen_num_rows(ctypes.byref(p), cup, lkp) == code
    fake = ctypes.c_void_p(1 << 20)
    assert lib.fp_sparse_prefill_paged(ctypes.byref(p), fake, cup, lkp, fake, fake, fake, None, None, None,
                                       4.0, fake, fake, 1 << 30, fake, None, fake, 1 << 40, None) == code


def test_paged_rejects_nan_tau_capacity_workspace():
    lib = N.load()
    p = vproblem()
    _, cup = arr([0, 300, 400, 1000])
    _, lkp = arr([500, 200, 1000])
    fake = ctypes.c_void_p(1 << 20)
    nnz = lib.fp_varlen_max_nnz(ctypes.byref(p), cup, lkp)
    ws = lib.fp_varlen_workspace_size(ctypes.byref(p), cup, lkp)
    call = lambda tau, cap, wsb: lib.fp_sparse_prefill_paged(
        ctypes.byref(p), fake, cup, lkp, fake, fake, fake, None, None, None, tau, fake, fake, cap, fake, None,
        fake, wsb, None)
    assert call(float("nan"), nnz, ws) == N.FP_ERR_INVALID
    assert call(4.0, nnz - 1, ws) == N.FP_ERR_CAPACITY
    assert call(4.0, nnz, ws - 1) == N.FP_ERR_CAPACITY


def test_paged_fp8_needs_scales():
    """fp8 codes in the paged cache take q/k/v scales; a missing one is refused
    before any HIP call. fp8 also halves the byte strides the checks see."""
    lib = N.load()
    p = vproblem(dtype=N.FP_DTYPE_FP8_E4M3)
    _, cup = arr([0, 300, 400, 1000])
    _, lkp = arr([500, 200, 1000])
    nnz = lib.fp_varlen_max_nnz(ctypes.byref(p), cup, lkp)
    ws = lib.fp_varlen_workspace_size(ctypes.byref(p), cup, lkp)
    assert nnz > 0 and ws > 0
    fake = ctypes.c_void_p(1 << 20)
    for scales in ((None, fake, fake), (fake, None, fake), (fake, fake, None)):
        assert lib.fp_sparse_prefill_paged(ctypes.byref(p), fake, cup, lkp, fake, fake, fake, *scales, 4.0,
                                           fake, fake, nnz, fake, None, fake, ws, None) == N.FP_ERR_INVALID
    p.q_stride[1] = 8 + 128                       # 136 bytes per head row: not a multiple of 16
    assert lib.fp_varlen_num_rows(ctypes.byref(p), cup, lkp) == N.FP_ERR_INVALID


def test_paged_cached_needs_its_cache_and_checks_like_paged():
    """The pooled-KV entry point refuses a missing or misaligned cache and
    otherwise checks its arguments exactly as the plain paged one, before any
    HIP call."""
    lib = N.load()
    p = vproblem()
    _, cup = arr([0, 300, 400, 1000])
    _, lkp = arr([500, 200, 1000])
    nnz = lib.fp_varlen_max_nnz(ctypes.byref(p), cup, lkp)
    ws = lib.fp_varlen_workspace_size(ctypes.byref(p), cup, lkp)
    fake = ctypes.c_void_p(1 << 20)
    call = lambda kc, vc, tau=4.0, cap=nnz, wsb=ws: lib.fp_sparse_prefill_paged_cached(
        ctypes.byref(p), fake, cup, lkp, fake, fake, fake, None, None, None, kc, vc, tau, fake, fake, cap, fake,
        None, fake, wsb, None)
    assert call(None, fake) == N.FP_ERR_INVALID
    assert call(fake, None) == N.FP_ERR_INVALID
    assert call(fake, ctypes.c_void_p((1 << 20) + 4)) == N.FP_ERR_INVALID       # not 16-byte aligned
    assert "misaligned" in lib.fp_last_error().decode()
    assert call(fake, fake, tau=float("nan")) == N.FP_ERR_INVALID
    assert call(fake, fake, cap=nnz - 1) == N.FP_ERR_CAPACITY
    assert call(fake, fake, wsb=ws - 1) == N.FP_ERR_CAPACITY


def test_binding_checks_pooled_kv_cache():
    """The pooled-KV cache is fp32 [pages * max(1, page_size / block), Hkv, 128]."""
    import torch
    import block_sparse_long_estimate_amd as fp
    Hkv, pages = 2, 8
    q = torch.zeros((40, 4, 128), dtype=torch.bfloat16)
    for page, block, slots in ((16, 64, 8), (256, 64, 32), (64, 64, 8)):
        kc = torch.zeros((pages, page, Hkv, 128), dtype=torch.bfloat16)
        bt = torch.arange(pages, dtype=torch.int32).reshape(2, 4)
        cu, lk = np.array([0, 20, 40], dtype=np.int32), np.array([30, 50], dtype=np.int32)
        vp = fp.make_varlen_problem(q, cu, lk, kc, bt, block)
        assert fp.pooled_kv_slots(kc, block) == slots
        good = torch.zeros((slots, Hkv, 128))
        with pytest.raises(fp.FpError, match="kbar_cache has shape"):
            fp.fp_sparse_prefill_paged_cached(vp, q, kc, kc, bt, good[:-1], good, 1.0)
        with pytest.raises(fp.FpError, match="vbar_cache must be torch.float32"):
            fp.fp_sparse_prefill_paged_cached(vp, q, kc, kc, bt, good, good.bfloat16(), 1.0)
        with pytest.raises(fp.FpError, match="vbar_cache is required"):
            fp.fp_sparse_prefill_paged_cached(vp, q, kc, kc, bt, good, None, 1.0)


def test_variant_validation():
    """variant (the ablation of the mean correction) sits where the padding was."""
    lib = N.load()
    assert ctypes.sizeof(N.FpProblem) == 144
    assert lib.fp_num_rows(ctypes.byref(problem(variant=N.FP_VARIANT_NO_CORRECTION))) > 0
    assert lib.fp_num_rows(ctypes.byref(problem(variant=7))) == N.FP_ERR_UNSUPPORTED
    # per-head lists: one row per (query head, query block), sizes follow
    base = problem()
    ph = problem(variant=N.FP_VARIANT_PER_HEAD_LISTS)
    G = base.num_q_heads // base.num_kv_heads
    assert lib.fp_num_rows(ctypes.byref(ph)) == G * lib.fp_num_rows(ctypes.byref(base))
    assert lib.fp_max_nnz(ctypes.byref(ph)) == G * lib.fp_max_nnz(ctypes.byref(base))
    assert lib.fp_workspace_size(ctypes.byref(ph)) > lib.fp_workspace_size(ctypes.byref(base))
    assert lib.fp_prefill_workspace_size(ctypes.byref(ph)) == lib.fp_prefill_workspace_size(ctypes.byref(base))


def test_split_validation_and_workspace():
    """split (FP_SPLIT_SMALL_GRIDS) only changes E6 on problems of at most 128
    (row, 256-row slice) units: the prefill workspace then holds each part's
    partial results (256 rows x (128 + 2) floats); larger problems, and the
    default FP_SPLIT_OFF, need only the summary operands."""
    lib = N.load()
    assert lib.fp_num_rows(ctypes.byref(problem(split=7))) == N.FP_ERR_UNSUPPORTED
    assert lib.fp_num_rows(ctypes.byref(problem(reserved_=1))) == N.FP_ERR_INVALID
    ws = lambda **kw: lib.fp_prefill_workspace_size(ctypes.byref(problem(**kw)))
    # 16 rows (8 query blocks x 2 KV heads) x 2 slices (G = 4, 128-token blocks) = 32 units: 8 parts
    assert ws(split=N.FP_SPLIT_SMALL_GRIDS) - ws() == 16 * 2 * 8 * 256 * 130 * 4
    # S = 2048, 4/1 heads, 64-token blocks: 32 rows x 1 slice = 32 units: 8 parts
    small = dict(seqlen=2048, num_q_heads=4, num_kv_heads=1, block=64)
    for name, H in (("q_stride", 4), ("k_stride", 1), ("v_stride", 1), ("o_stride", 4)):
        small[name] = (ctypes.c_int64 * 3)(2048 * H * 128, H * 128, 128)
    assert ws(split=N.FP_SPLIT_SMALL_GRIDS, **small) - ws(**small) == 32 * 8 * 256 * 130 * 4
    # 128K tokens, 8 query / 2 KV heads: 2048 rows x 2 slices, far more than the chip: no split
    big = dict(seqlen=131072)
    for name, H in (("q_stride", 8), ("k_stride", 2), ("v_stride", 2), ("o_stride", 8)):
        big[name] = (ctypes.c_int64 * 3)(131072 * H * 128, H * 128, 128)
    assert ws(split=N.FP_SPLIT_SMALL_GRIDS, **big) == ws(**big)
    # the allocation-free entry point's static array holds the largest split's partial results
    assert 256 * 256 * 130 * 4 + 3 * 256 * 256 <= N.FP_NOALLOC_SCRATCH_BYTES


def test_block_score_variant_takes_scores():
    """The block-score variant runs through fp_sparse_prefill_scored only; the
    other entry points refuse it, and the scored entry refuses other variants
    (all before any HIP call)."""
    lib = N.load()
    fake = ctypes.c_void_p(1 << 20)
    args = [fake] * 3 + [None] * 3 + [fake] * 4 + [None, fake, None, fake, 1 << 30, None]
    bs = problem(variant=N.FP_VARIANT_BLOCK_SCORE)
    assert lib.fp_sparse_prefill(ctypes.byref(bs), *args) == N.FP_ERR_INVALID
    assert b"fp_sparse_prefill_scored" in lib.fp_last_error()
    assert lib.fp_sparse_prefill_scored(ctypes.byref(problem()), *args) == N.FP_ERR_INVALID
    assert b"FP_VARIANT_BLOCK_SCORE" in lib.fp_last_error()


def test_out_dtype_validation():
    lib = N.load()
    assert ctypes.sizeof(N.FpProblem) == 144
    p = problem(out_dtype=1)
    assert lib.fp_num_rows(ctypes.byref(p)) == N.FP_ERR_UNSUPPORTED
    p = problem(out_dtype=N.FP_OUT_FP32)
    assert lib.fp_num_rows(ctypes.byref(p)) > 0          # 128-element rows: 512-byte aligned
    p.o_stride[1] = 8 * 128 + 2                           # 8-byte aligned fp32 rows only
    assert lib.fp_num_rows(ctypes.byref(p)) == N.FP_ERR_INVALID



def test_binding_rejects_mismatched_cache_views():
    """The Python binding checks that V shares K's strides and dtype and that
    both match the strides the problem was sized with, before any device call."""
    import torch
    import block_sparse_long_estimate_amd as fp
    Hkv, page, pages = 2, 16, 8
    q = torch.zeros((40, 4, 128), dtype=torch.bfloat16)
    cache = torch.zeros((pages, 2, page, Hkv, 128), dtype=torch.bfloat16)
    kc, vc = cache[:, 0], cache[:, 1]
    bt = torch.arange(pages, dtype=torch.int32).reshape(2, 4)
    cu, lk = np.array([0, 20, 40], dtype=np.int32), np.array([30, 50], dtype=np.int32)
    vp = fp.make_varlen_problem(q, cu, lk, kc, bt, 64)
    with pytest.raises(fp.FpError, match="v_cache has strides"):
        fp.fp_sparse_prefill_paged(vp, q, kc, vc.contiguous(), bt, 1.0)
    with pytest.raises(fp.FpError, match="v_cache must be torch.bfloat16"):
        fp.fp_sparse_prefill_paged(vp, q, kc, vc.float(), bt, 1.0)
    with pytest.raises(fp.FpError, match="k_cache has strides"):
        fp.fp_sparse_prefill_paged(vp, q, kc.contiguous(), vc.contiguous(), bt, 1.0)
    # a permuted cache (head dim not contiguous) and a v_cache with fewer pages
    with pytest.raises(fp.FpError, match="last dim must be contiguous"):
        fp.fp_sparse_prefill_paged(vp, q, kc.transpose(2, 3).contiguous().transpose(2, 3), vc, bt, 1.0)
    with pytest.raises(fp.FpError, match="share one shape"):
        fp.fp_sparse_prefill_paged(vp, q, kc, vc[:4], bt, 1.0)
    with pytest.raises(fp.FpError, match="q: last dim must be contiguous"):
        fp.fp_sparse_prefill_paged(vp, q.transpose(1, 2).contiguous().transpose(1, 2), kc, vc, bt, 1.0)
    with pytest.raises(fp.FpError, match="q must be torch.bfloat16"):
        fp.fp_sparse_prefill_paged(vp, q.to(torch.uint8), kc, vc, bt, 1.0)


def test_plain_c_program_uses_the_abi(tmp_path):
    """tests/c/abi_host.c: the header compiled as C99 (-Wall -Wextra -Werror),
    linked against the in-tree library, sizing and argument checks called from C."""
    import shutil
    import subprocess
    gcc = shutil.which("gcc")
    assert gcc, "gcc is required for the C ABI check"
    libdir = os.path.dirname(N.LIB_PATH)
    exe = str(tmp_path / "abi_host")
    cmd = [gcc, "-std=c99", "-Wall", "-Wextra", "-Werror", "-I", os.path.join(ROOT, "include"),
           os.path.join(ROOT, "tests", "c", "abi_host.c"), "-L", libdir, "-lfp_prefill",
           f"-Wl,-rpath,{libdir}", "-lm", "-o", exe]
    b = subprocess.run(cmd, capture_output=True, text=True, timeout=120)
    assert b.returncode == 0, b.stderr
    r = subprocess.run([exe], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0 and r.stdout.strip() == "ok", r.stdout + r.stderr


def test_abi_host_code_under_sanitizers(tmp_path):
    """The library's host code (argument checks, sizing, workspace carving)
    built with AddressSanitizer and UndefinedBehaviorSanitizer (host pass
    only: -Xarch_host), driven by tests/c/abi_host.c built the same way. No
    GPU: every call in the program returns before any device work."""
    import shutil
    import subprocess
    from concurrent.futures import ThreadPoolExecutor
    hipcc, clang = "/opt/rocm/bin/hipcc", "/opt/rocm/llvm/bin/clang"
    if not (os.path.exists(hipcc) and os.path.exists(clang)):
        pytest.skip("ROCm hipcc/clang not found")
    csrc = os.path.join(ROOT, "block_sparse_long_estimate_amd", "csrc")
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=undefined"]
    flags = ["--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC", "-Xclang", "-target-feature",
             "-Xclang", "-packed-fp32-ops", "-Wno-unused-command-line-argument"]

    def compile_one(name):
        obj = str(tmp_path / (name + ".o"))
        extra = san if name == "abi" else []        # the host-side checks live in abi.hip
        r = subprocess.run([hipcc] + flags + extra + ["-c", os.path.join(csrc, name + ".hip"), "-o", obj],
                           capture_output=True, text=True, timeout=600)
        assert r.returncode == 0, r.stderr[-2000:]
        return obj

    with ThreadPoolExecutor(4) as ex:
        objs = list(ex.map(compile_one, ["abi", "k_estimate", "k_select", "k_attn"]))
    lib = str(tmp_path / "libfp_prefill.so")
    r = subprocess.run([hipcc] + flags + san + ["-shared"] + objs + ["-o", lib], capture_output=True, text=True,
                       timeout=300)
    assert r.returncode == 0, r.stderr[-2000:]
    exe = str(tmp_path / "abi_host")
    r = subprocess.run([clang, "-std=c99", "-Wall", "-Wextra", "-Werror", "-g", "-fsanitize=address,undefined",
                        "-fno-sanitize-recover=undefined", "-I", os.path.join(ROOT, "include"),
                        os.path.join(ROOT, "tests", "c", "abi_host.c"), "-L", str(tmp_path), "-lfp_prefill",
                        f"-Wl,-rpath,{tmp_path}", "-lm", "-o", exe], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr[-2000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120, env=env)
    assert r.returncode == 0 and r.stdout.strip() == "ok", r.stdout + r.stderr[-3000:]


def test_binding_argument_checks():
    """The binding refuses, before any device call, tensors that the kernels
    would misread: mixed q/k/v dtypes, missing or misshapen fp8 scales,
    scales on bf16 inputs, non-int32 kept lists or block tables, and host
    (CPU) tensors, whose addresses would fault the GPU."""
    import torch
    import block_sparse_long_estimate_amd as fp
    S, Hq, Hkv = 300, 4, 2
    q = torch.zeros((1, S, Hq, 128), dtype=torch.bfloat16)
    k = torch.zeros((1, S, Hkv, 128), dtype=torch.bfloat16)
    with pytest.raises(fp.FpError, match="must all be bfloat16"):
        fp.make_problem(q, k.to(torch.uint8), k, 128)
    with pytest.raises(fp.FpError, match="expected"):
        fp.make_problem(q, k[:, :200], k[:, :200], 128)
    p = fp.make_problem(q, k, k, 128)
    with pytest.raises(fp.FpError, match="fp8 inputs only"):
        fp.fp_block_scores(p, q, k, k, q_scale=torch.ones(1, Hq, 3))
    with pytest.raises(fp.FpError, match="on the GPU"):
        fp.fp_block_scores(p, q, k, k)
    q8, k8 = q.to(torch.uint8), k.to(torch.uint8)
    p8 = fp.make_problem(q8, k8, k8, 128)
    ks = torch.ones(1, Hkv, 3)
    with pytest.raises(fp.FpError, match="q_scale is required"):
        fp.fp_block_scores(p8, q8, k8, k8, None, ks, ks)
    with pytest.raises(fp.FpError, match="shape"):
        fp.fp_block_scores(p8, q8, k8, k8, torch.ones(1, Hq, 2), ks, ks)
    with pytest.raises(fp.FpError, match="float32"):
        fp.fp_block_scores(p8, q8, k8, k8, torch.ones(1, Hq, 3, dtype=torch.float64), ks, ks)
    # q/k/v must match the problem they were described with
    with pytest.raises(fp.FpError, match="q has shape"):
        fp.fp_block_scores(p, q[:, :200], k, k)
    with pytest.raises(fp.FpError, match="k must be torch.bfloat16"):
        fp.fp_block_scores(p, q, k.float(), k)
    with pytest.raises(fp.FpError, match="v has strides"):
        fp.fp_block_scores(p, q, k, torch.zeros((1, S, 2 * Hkv, 128), dtype=torch.bfloat16)[:, :, :Hkv])
    # fp_select_blocks reads scores as fp32 [batch, Hq, nb, nb]
    with pytest.raises(fp.FpError, match="scores has shape"):
        fp.fp_select_blocks(p, torch.zeros(1, Hq, 3, 2), 1.0)
    with pytest.raises(fp.FpError, match="scores must be torch.float32"):
        fp.fp_select_blocks(p, torch.zeros(1, Hq, 3, 3, dtype=torch.float64), 1.0)
    # fp_sparse_prefill: pooled rows fp32 [batch, Hkv, nb, 128], o per the problem's out dtype and strides
    kb = torch.zeros(1, Hkv, 3, 128)
    rp = torch.zeros(p.rows + 1, dtype=torch.int32)
    ci = torch.zeros(p.max_nnz, dtype=torch.int32)
    with pytest.raises(fp.FpError, match="kbar has shape"):
        fp.fp_sparse_prefill(p, q, k, k, torch.zeros(1, Hkv, 2, 128), kb, rp, ci)
    with pytest.raises(fp.FpError, match="vbar must be torch.float32"):
        fp.fp_sparse_prefill(p, q, k, k, kb, kb.double(), rp, ci)
    with pytest.raises(fp.FpError, match="o must be torch.bfloat16"):
        fp.fp_sparse_prefill(p, q, k, k, kb, kb, rp, ci, o=torch.zeros(1, S, Hq, 128))
    pf = fp.make_problem(q, k, k, 128, out_fp32=True)
    with pytest.raises(fp.FpError, match="o must be torch.float32"):
        fp.fp_sparse_prefill(pf, q, k, k, kb, kb, rp, ci, o=torch.zeros(1, S, Hq, 128, dtype=torch.bfloat16))
    with pytest.raises(fp.FpError, match="o has shape"):
        fp.fp_sparse_prefill(p, q, k, k, kb, kb, rp, ci, o=torch.zeros(1, S, Hq, 64, dtype=torch.bfloat16))
    ostr = torch.zeros(1, S, Hq, 256, dtype=torch.bfloat16)[..., :128]
    po = fp.make_problem(q, k, k, 128, o=ostr)
    with pytest.raises(fp.FpError, match="strided o"):
        fp.fp_sparse_prefill(po, q, k, k, kb, kb, rp, ci)
    with pytest.raises(fp.FpError, match="o has strides"):
        fp.fp_sparse_prefill(po, q, k, k, kb, kb, rp, ci, o=torch.zeros(1, S, Hq, 128, dtype=torch.bfloat16))
    rp = torch.zeros(p.rows + 1, dtype=torch.int64)
    with pytest.raises(fp.FpError, match="row_ptr must be torch.int32"):
        fp.fp_sparse_prefill(p, q, k, k, kb, kb, rp, rp)
    # paged: the block table must be int32 [num_seqs, max_pages]
    cache = torch.zeros((8, 16, Hkv, 128), dtype=torch.bfloat16)
    qp = torch.zeros((40, Hq, 128), dtype=torch.bfloat16)
    bt = torch.arange(8, dtype=torch.int32).reshape(2, 4)
    cu, lk = np.array([0, 20, 40], dtype=np.int32), np.array([30, 50], dtype=np.int32)
    vp = fp.make_varlen_problem(qp, cu, lk, cache, bt, 64)
    with pytest.raises(fp.FpError, match="block_table must be torch.int32"):
        fp.fp_sparse_prefill_paged(vp, qp, cache, cache, bt.long(), 1.0)
    with pytest.raises(fp.FpError, match="packed"):
        fp.fp_sparse_prefill_paged(vp, qp[:30], cache, cache, bt, 1.0)
    with pytest.raises(fp.FpError, match="on the GPU"):
        fp.fp_sparse_prefill_paged(vp, qp, cache, cache, bt, 1.0)


def test_noalloc_rejects_problems_beyond_its_scratch():
    """The allocation-free entry point refuses, before any HIP call, a problem
    whose summary operands exceed its static scratch array (batch x KV heads
    x blocks above FP_NOALLOC_MAX_POOLED_ROWS), and accepts the argument
    checks of fp_sparse_prefill."""
    lib = N.load()
    nb = 1024
    p = problem(seqlen=nb * 128, num_q_heads=8, num_kv_heads=8)
    for arr in (p.q_stride, p.k_stride, p.v_stride, p.o_stride):
        arr[0], arr[1], arr[2] = nb * 128 * 8 * 128, 8 * 128, 128
    p.batch = N.FP_NOALLOC_MAX_POOLED_ROWS // (8 * nb) + 1
    fake = ctypes.c_void_p(1 << 20)          # never dereferenced: the call fails before any device work
    args = [fake] * 3 + [None] * 3 + [fake] * 4 + [None, fake, None, None]
    rc = lib.fp_sparse_prefill_noalloc(ctypes.byref(p), *args)
    assert rc == N.FP_ERR_CAPACITY
    assert b"static" in lib.fp_last_error()
    p.batch = 1
    args_null = [fake] * 3 + [None] * 3 + [None] + [fake] * 3 + [None, fake, None, None]
    assert lib.fp_sparse_prefill_noalloc(ctypes.byref(p), *args_null) == N.FP_ERR_INVALID


def test_dense_entry_point_checks():
    """fp_dense_prefill validates its problem and pointers before any HIP call."""
    lib = N.load()
    p = problem()
    fake = ctypes.c_void_p(1 << 20)
    assert lib.fp_dense_prefill(ctypes.byref(p), None, fake, fake, None, None, None, fake, None, None) \
        == N.FP_ERR_INVALID
    p8 = problem(dtype=N.FP_DTYPE_FP8_E4M3)
    for arr in (p8.q_stride, p8.k_stride, p8.v_stride):
        arr[0], arr[1], arr[2] = arr[0] // 2, arr[1] // 2, arr[2] // 2
    assert lib.fp_dense_prefill(ctypes.byref(p8), fake, fake, fake, None, None, None, fake, None, None) \
        == N.FP_ERR_INVALID
    assert b"scale" in lib.fp_last_error()
    bad = problem(head_dim=64)
    assert lib.fp_dense_prefill(ctypes.byref(bad), fake, fake, fake, None, None, None, fake, None, None) \
        == N.FP_ERR_UNSUPPORTED
