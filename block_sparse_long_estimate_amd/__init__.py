"""Block-sparse causal GQA prefill attention for AMD MI355X (gfx950).

Thin Python binding over the C ABI of libfp_prefill.so (include/fp_prefill.h):
it builds the problem descriptors from torch tensors, allocates outputs with
torch, and passes raw device pointers plus torch's current HIP stream. Every
step of the method runs in the library's HIP kernels; there is no fallback.

Entry points (same names as the C ABI):
  fp_block_scores          pooling + block scores (E1-E2)
  fp_select_blocks         max-based dynamic threshold -> CSR kept lists (E3-E5)
  fp_sparse_prefill        sparse attention + mean correction (E6)
  fp_sparse_prefill_paged  all of it for a paged varlen batch
  fp_sparse_prefill_noalloc  fp_sparse_prefill without a workspace (static scratch)
  fp_dense_prefill         dense causal attention on the same kernel (the baseline)
  fp_estimate_select       E1-E5 without a score matrix (fused estimate + selection)
and sparse_prefill(), which chains the first three.
"""
from __future__ import annotations

import ctypes
import math
from dataclasses import dataclass
from typing import Optional, Tuple

import numpy as np
import torch

from . import _native as N
from ._native import FpError, FpProblem, FpVarlenProblem

__all__ = [
    "FpError", "Problem", "make_problem", "fp_block_scores", "fp_select_blocks",
    "fp_sparse_prefill", "fp_sparse_prefill_paged", "sparse_prefill", "version",
    "make_varlen_problem", "fp_sparse_prefill_noalloc", "fp_dense_prefill", "fp_estimate_select",
    "sparse_prefill_fused", "fp_sparse_prefill_scored", "VARIANTS", "fp_sparse_prefill_paged_cached",
    "pooled_kv_slots",
]


def version() -> str:
    return N.load().fp_version().decode()


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    """Device address of t; the kernels read and write through it, so t must
    live on the current GPU (a host pointer would fault the device)."""
    if t is None:
        return None
    if not t.is_cuda:
        raise FpError(N.FP_ERR_INVALID, "every tensor argument must be on the GPU (got a CPU tensor)")
    if t.device.index != torch.cuda.current_device():
        raise FpError(N.FP_ERR_INVALID,
                      f"tensor on {t.device}, but the current device is cuda:{torch.cuda.current_device()}")
    return t.data_ptr()


def _check(t: Optional[torch.Tensor], name: str, dtype: torch.dtype, shape=None, required: bool = False):
    """dtype, contiguity and (optionally) shape of an argument the C ABI reads
    as a packed array."""
    if t is None:
        if required:
            raise FpError(N.FP_ERR_INVALID, f"{name} is required")
        return
    if t.dtype != dtype:
        raise FpError(N.FP_ERR_INVALID, f"{name} must be {dtype} (got {t.dtype})")
    if not t.is_contiguous():
        raise FpError(N.FP_ERR_INVALID, f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise FpError(N.FP_ERR_INVALID, f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


def _check_view(t: Optional[torch.Tensor], name: str, dtype: torch.dtype, shape, strides=None):
    """A strided tensor the kernels address through the problem's strides:
    dtype, shape, a contiguous last dimension and (when given) the leading
    strides the problem descriptor was built with must all match."""
    if t is None:
        raise FpError(N.FP_ERR_INVALID, f"{name} is required")
    if t.dtype != dtype:
        raise FpError(N.FP_ERR_INVALID, f"{name} must be {dtype} (got {t.dtype})")
    if tuple(t.shape) != tuple(shape):
        raise FpError(N.FP_ERR_INVALID, f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.stride(-1) != 1:
        raise FpError(N.FP_ERR_INVALID, f"{name}: last dim must be contiguous")
    if strides is not None and tuple(t.stride()[:len(strides)]) != tuple(strides):
        raise FpError(N.FP_ERR_INVALID, f"{name} has strides {tuple(t.stride())}, but the problem was "
                                        f"built with {tuple(strides)}")


def _check_qkv(p: "Problem", q, k, v):
    c = p.c
    dt = torch.uint8 if p.fp8 else torch.bfloat16
    _check_view(q, "q", dt, (c.batch, c.seqlen, c.num_q_heads, 128), tuple(c.q_stride))
    _check_view(k, "k", dt, (c.batch, c.seqlen, c.num_kv_heads, 128), tuple(c.k_stride))
    _check_view(v, "v", dt, (c.batch, c.seqlen, c.num_kv_heads, 128), tuple(c.v_stride))


def _check_scales(fp8: bool, nseq: int, Hq: int, Hkv: int, nsb: int, q_scale, k_scale, v_scale):
    if not fp8:
        if any(t is not None for t in (q_scale, k_scale, v_scale)):
            raise FpError(N.FP_ERR_INVALID, "scales are for fp8 inputs only")
        return
    for name, t, H in (("q_scale", q_scale, Hq), ("k_scale", k_scale, Hkv), ("v_scale", v_scale, Hkv)):
        _check(t, name, torch.float32, (nseq, H, nsb), required=True)


def _stream() -> int:
    return torch.cuda.current_stream().cuda_stream


@dataclass
class Problem:
    c: FpProblem
    nb: int
    rows: int
    max_nnz: int
    fp8: bool

    @property
    def ref(self):
        return ctypes.byref(self.c)


VARIANTS = {"mean": N.FP_VARIANT_MEAN_CORRECTION, "none": N.FP_VARIANT_NO_CORRECTION,
            "per_head": N.FP_VARIANT_PER_HEAD_LISTS, "block_score": N.FP_VARIANT_BLOCK_SCORE}


def make_problem(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, block: int,
                 softmax_scale: float = 0.0, o: Optional[torch.Tensor] = None,
                 out_fp32: bool = False, correction: bool = True, variant: Optional[str] = None,
                 split_small: bool = False) -> Problem:
    """Descriptor of a fixed-shape batch: q [batch, S, Hq, 128], k/v [batch, S, Hkv, 128]
    (bf16, or uint8 E4M3FN codes), last dim contiguous. out_fp32: fp_sparse_prefill
    writes o in float32 (diagnostic) instead of bfloat16. correction=False: the
    ablation without the mean correction (pruned blocks dropped). variant: one of
    VARIANTS ("mean" is E1-E6 as stated; "none", "per_head" and "block_score"
    are ablations). split_small: a problem too small to fill the chip splits each
    row's tiles over several workgroups (FP_SPLIT_SMALL_GRIDS; lower latency, but
    the rounding then depends on the problem's size)."""
    if variant is None:
        variant = "mean" if correction else "none"
    if variant not in VARIANTS:
        raise FpError(N.FP_ERR_INVALID, f"unknown variant {variant!r} (one of {sorted(VARIANTS)})")
    fp8 = q.dtype == torch.uint8
    if q.dtype not in (torch.bfloat16, torch.uint8) or k.dtype != q.dtype or v.dtype != q.dtype:
        raise FpError(N.FP_ERR_INVALID, f"q, k, v must all be bfloat16 or all uint8 E4M3FN codes "
                                        f"(got {q.dtype}, {k.dtype}, {v.dtype})")
    if q.dim() != 4 or k.dim() != 4 or k.shape != v.shape or q.shape[:2] != k.shape[:2]:
        raise FpError(N.FP_ERR_INVALID, f"q [batch, S, Hq, d] and k, v [batch, S, Hkv, d] expected "
                                        f"(got {tuple(q.shape)}, {tuple(k.shape)}, {tuple(v.shape)})")
    c = FpProblem()
    c.out_dtype = N.FP_OUT_FP32 if out_fp32 else N.FP_OUT_BF16
    c.variant = VARIANTS[variant]
    c.split = N.FP_SPLIT_SMALL_GRIDS if split_small else N.FP_SPLIT_OFF
    c.batch, c.seqlen, c.num_q_heads, c.head_dim = q.shape[0], q.shape[1], q.shape[2], q.shape[3]
    c.num_kv_heads = k.shape[2]
    c.block = block
    c.dtype = N.FP_DTYPE_FP8_E4M3 if fp8 else N.FP_DTYPE_BF16
    c.softmax_scale = softmax_scale
    for name, t in (("q_stride", q), ("k_stride", k), ("v_stride", v), ("o_stride", o if o is not None else q)):
        st = t.stride()
        if t.stride(-1) != 1:
            raise FpError(N.FP_ERR_INVALID, f"{name[0]}: last dim must be contiguous")
        arr = getattr(c, name)
        arr[0], arr[1], arr[2] = st[0], st[1], st[2]
    if o is None:
        # o is allocated contiguous [batch, S, Hq, 128]
        S, Hq, d = q.shape[1], q.shape[2], q.shape[3]
        c.o_stride[0], c.o_stride[1], c.o_stride[2] = S * Hq * d, Hq * d, d
    lib = N.load()
    rows = N.check_size(lib.fp_num_rows(ctypes.byref(c)))
    nnz = N.check_size(lib.fp_max_nnz(ctypes.byref(c)))
    return Problem(c, (q.shape[1] + block - 1) // block, rows, nnz, fp8)


def fp_block_scores(p: Problem, q, k, v, q_scale=None, k_scale=None, v_scale=None):
    """E1-E2 -> (qbar, kbar, vbar, scores), fp32 device tensors."""
    c = p.c
    _check_qkv(p, q, k, v)
    _check_scales(p.fp8, c.batch, c.num_q_heads, c.num_kv_heads, (c.seqlen + 127) // 128, q_scale, k_scale,
                  v_scale)
    dev = q.device
    f32 = dict(dtype=torch.float32, device=dev)
    qbar = torch.empty((c.batch, c.num_q_heads, p.nb, 128), **f32)
    kbar = torch.empty((c.batch, c.num_kv_heads, p.nb, 128), **f32)
    vbar = torch.empty((c.batch, c.num_kv_heads, p.nb, 128), **f32)
    scores = torch.empty((c.batch, c.num_q_heads, p.nb, p.nb), **f32)
    N.check(N.load().fp_block_scores(p.ref, _ptr(q), _ptr(k), _ptr(v), _ptr(q_scale), _ptr(k_scale),
                                     _ptr(v_scale), _ptr(qbar), _ptr(kbar), _ptr(vbar), _ptr(scores),
                                     _stream()))
    return qbar, kbar, vbar, scores


def fp_select_blocks(p: Problem, scores: torch.Tensor, tau: float, with_sched: bool = True,
                     workspace: Optional[torch.Tensor] = None):
    """E3-E5 -> (row_ptr, col_idx, sched) int32 device tensors (col_idx has
    capacity max_nnz; its first row_ptr[-1] entries are valid)."""
    c = p.c
    _check(scores, "scores", torch.float32, (c.batch, c.num_q_heads, p.nb, p.nb), required=True)
    dev = scores.device
    i32 = dict(dtype=torch.int32, device=dev)
    row_ptr = torch.empty(p.rows + 1, **i32)
    col_idx = torch.empty(p.max_nnz, **i32)
    sched = torch.empty(p.rows, **i32) if with_sched else None
    lib = N.load()
    ws_bytes = N.check_size(lib.fp_workspace_size(p.ref))
    if workspace is None:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    N.check(lib.fp_select_blocks(p.ref, _ptr(scores), float(tau), _ptr(row_ptr), _ptr(col_idx),
                                 p.max_nnz, _ptr(sched), _ptr(workspace), workspace.numel(),
                                 _stream()))
    return row_ptr, col_idx, sched


def fp_sparse_prefill(p: Problem, q, k, v, kbar, vbar, row_ptr, col_idx, sched=None,
                      q_scale=None, k_scale=None, v_scale=None, with_lse: bool = True,
                      o: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None):
    """E6 -> (o like q in bf16, or fp32 for an out_fp32 problem; lse fp32 [batch, Hq, S] or None)."""
    c = p.c
    _check_qkv(p, q, k, v)
    _check_scales(p.fp8, c.batch, c.num_q_heads, c.num_kv_heads, (c.seqlen + 127) // 128, q_scale, k_scale,
                  v_scale)
    pooled = (c.batch, c.num_kv_heads, p.nb, 128)
    _check(kbar, "kbar", torch.float32, pooled, required=True)
    _check(vbar, "vbar", torch.float32, pooled, required=True)
    _check(row_ptr, "row_ptr", torch.int32, (p.rows + 1,), required=True)
    _check(col_idx, "col_idx", torch.int32, required=True)
    _check(sched, "sched", torch.int32, (p.rows,))
    odt = torch.float32 if c.out_dtype == N.FP_OUT_FP32 else torch.bfloat16
    oshape = (c.batch, c.seqlen, c.num_q_heads, 128)
    if o is None:
        if tuple(c.o_stride) != (c.seqlen * c.num_q_heads * 128, c.num_q_heads * 128, 128):
            raise FpError(N.FP_ERR_INVALID, "the problem was built for a strided o: pass that o")
        o = torch.empty(oshape, dtype=odt, device=q.device)
    else:
        _check_view(o, "o", odt, oshape, tuple(c.o_stride))
    lse = torch.empty((c.batch, c.num_q_heads, c.seqlen), dtype=torch.float32,
                      device=q.device) if with_lse else None
    lib = N.load()
    if workspace is None:
        workspace = torch.empty(N.check_size(lib.fp_prefill_workspace_size(p.ref)), dtype=torch.uint8,
                                device=q.device)
    N.check(lib.fp_sparse_prefill(p.ref, _ptr(q), _ptr(k), _ptr(v), _ptr(q_scale), _ptr(k_scale),
                                  _ptr(v_scale), _ptr(kbar), _ptr(vbar), _ptr(row_ptr),
                                  _ptr(col_idx), _ptr(sched), _ptr(o), _ptr(lse), _ptr(workspace),
                                  workspace.numel(), _stream()))
    return o, lse


def fp_estimate_select(p: Problem, q, k, v, tau: float, q_scale=None, k_scale=None, v_scale=None,
                       with_sched: bool = True, workspace: Optional[torch.Tensor] = None):
    """E1-E5 without a score matrix -> (qbar, kbar, vbar, row_ptr, col_idx, sched);
    the kept lists equal fp_block_scores + fp_select_blocks bit for bit."""
    c = p.c
    _check_qkv(p, q, k, v)
    _check_scales(p.fp8, c.batch, c.num_q_heads, c.num_kv_heads, (c.seqlen + 127) // 128, q_scale, k_scale,
                  v_scale)
    dev = q.device
    f32 = dict(dtype=torch.float32, device=dev)
    i32 = dict(dtype=torch.int32, device=dev)
    qbar = torch.empty((c.batch, c.num_q_heads, p.nb, 128), **f32)
    kbar = torch.empty((c.batch, c.num_kv_heads, p.nb, 128), **f32)
    vbar = torch.empty((c.batch, c.num_kv_heads, p.nb, 128), **f32)
    row_ptr = torch.empty(p.rows + 1, **i32)
    col_idx = torch.empty(p.max_nnz, **i32)
    sched = torch.empty(p.rows, **i32) if with_sched else None
    lib = N.load()
    if workspace is None:
        workspace = torch.empty(N.check_size(lib.fp_estimate_select_workspace_size(p.ref)), dtype=torch.uint8,
                                device=dev)
    N.check(lib.fp_estimate_select(p.ref, _ptr(q), _ptr(k), _ptr(v), _ptr(q_scale), _ptr(k_scale), _ptr(v_scale),
                                   float(tau), _ptr(qbar), _ptr(kbar), _ptr(vbar), _ptr(row_ptr), _ptr(col_idx),
                                   p.max_nnz, _ptr(sched), _ptr(workspace), workspace.numel(), _stream()))
    return qbar, kbar, vbar, row_ptr, col_idx, sched


def sparse_prefill_fused(q, k, v, block: int, tau: float, softmax_scale: float = 0.0,
                         q_scale=None, k_scale=None, v_scale=None, with_lse: bool = True,
                         out_fp32: bool = False, correction: bool = True, variant: Optional[str] = None,
                         split_small: bool = False):
    """The path in two calls: fp_estimate_select (no score matrix) then
    fp_sparse_prefill. Returns a dict of device tensors. (The block-score
    variant needs the score matrix: use sparse_prefill.)"""
    p = make_problem(q, k, v, block, softmax_scale, out_fp32=out_fp32, correction=correction, variant=variant,
                     split_small=split_small)
    qbar, kbar, vbar, row_ptr, col_idx, sched = fp_estimate_select(p, q, k, v, tau, q_scale, k_scale, v_scale)
    o, lse = fp_sparse_prefill(p, q, k, v, kbar, vbar, row_ptr, col_idx, sched,
                               q_scale, k_scale, v_scale, with_lse)
    return dict(problem=p, qbar=qbar, kbar=kbar, vbar=vbar, row_ptr=row_ptr, col_idx=col_idx, sched=sched,
                o=o, lse=lse)


def fp_dense_prefill(p: Problem, q, k, v, q_scale=None, k_scale=None, v_scale=None, with_lse: bool = True,
                     o: Optional[torch.Tensor] = None):
    """Dense causal attention on the same kernel (every block kept; no
    estimate, selection or correction) -> (o, lse)."""
    c = p.c
    _check_qkv(p, q, k, v)
    _check_scales(p.fp8, c.batch, c.num_q_heads, c.num_kv_heads, (c.seqlen + 127) // 128, q_scale, k_scale,
                  v_scale)
    odt = torch.float32 if c.out_dtype == N.FP_OUT_FP32 else torch.bfloat16
    oshape = (c.batch, c.seqlen, c.num_q_heads, 128)
    if o is None:
        if tuple(c.o_stride) != (c.seqlen * c.num_q_heads * 128, c.num_q_heads * 128, 128):
            raise FpError(N.FP_ERR_INVALID, "the problem was built for a strided o: pass that o")
        o = torch.empty(oshape, dtype=odt, device=q.device)
    else:
        _check_view(o, "o", odt, oshape, tuple(c.o_stride))
    lse = torch.empty((c.batch, c.num_q_heads, c.seqlen), dtype=torch.float32,
                      device=q.device) if with_lse else None
    N.check(N.load().fp_dense_prefill(p.ref, _ptr(q), _ptr(k), _ptr(v), _ptr(q_scale), _ptr(k_scale),
                                      _ptr(v_scale), _ptr(o), _ptr(lse), _stream()))
    return o, lse


def fp_sparse_prefill_noalloc(p: Problem, q, k, v, kbar, vbar, row_ptr, col_idx, sched=None,
                              q_scale=None, k_scale=None, v_scale=None, o: Optional[torch.Tensor] = None,
                              lse: Optional[torch.Tensor] = None):
    """fp_sparse_prefill without a workspace: the library's static per-GPU
    scratch array holds the summary operands. o (and lse, if wanted) are the
    caller's, so nothing is allocated here either when they are passed; o is
    allocated only when omitted. Calls that overlap on one GPU race."""
    c = p.c
    _check_qkv(p, q, k, v)
    _check_scales(p.fp8, c.batch, c.num_q_heads, c.num_kv_heads, (c.seqlen + 127) // 128, q_scale, k_scale,
                  v_scale)
    pooled = (c.batch, c.num_kv_heads, p.nb, 128)
    _check(kbar, "kbar", torch.float32, pooled, required=True)
    _check(vbar, "vbar", torch.float32, pooled, required=True)
    _check(row_ptr, "row_ptr", torch.int32, (p.rows + 1,), required=True)
    _check(col_idx, "col_idx", torch.int32, required=True)
    _check(sched, "sched", torch.int32, (p.rows,))
    _check(lse, "lse", torch.float32, (c.batch, c.num_q_heads, c.seqlen))
    odt = torch.float32 if c.out_dtype == N.FP_OUT_FP32 else torch.bfloat16
    oshape = (c.batch, c.seqlen, c.num_q_heads, 128)
    if o is None:
        if tuple(c.o_stride) != (c.seqlen * c.num_q_heads * 128, c.num_q_heads * 128, 128):
            raise FpError(N.FP_ERR_INVALID, "the problem was built for a strided o: pass that o")
        o = torch.empty(oshape, dtype=odt, device=q.device)
    else:
        _check_view(o, "o", odt, oshape, tuple(c.o_stride))
    N.check(N.load().fp_sparse_prefill_noalloc(p.ref, _ptr(q), _ptr(k), _ptr(v), _ptr(q_scale), _ptr(k_scale),
                                               _ptr(v_scale), _ptr(kbar), _ptr(vbar), _ptr(row_ptr),
                                               _ptr(col_idx), _ptr(sched), _ptr(o), _ptr(lse), _stream()))
    return o, lse


def fp_sparse_prefill_scored(p: Problem, q, k, v, scores, vbar, row_ptr, col_idx, sched=None,
                             q_scale=None, k_scale=None, v_scale=None, with_lse: bool = True,
                             o: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None):
    """E6 under the block-score correction (a problem of variant
    "block_score"): pruned blocks stand in with logit S[h,i,j] + ln|block| ->
    (o, lse)."""
    c = p.c
    _check_qkv(p, q, k, v)
    _check_scales(p.fp8, c.batch, c.num_q_heads, c.num_kv_heads, (c.seqlen + 127) // 128, q_scale, k_scale,
                  v_scale)
    _check(scores, "scores", torch.float32, (c.batch, c.num_q_heads, p.nb, p.nb), required=True)
    _check(vbar, "vbar", torch.float32, (c.batch, c.num_kv_heads, p.nb, 128), required=True)
    _check(row_ptr, "row_ptr", torch.int32, (p.rows + 1,), required=True)
    _check(col_idx, "col_idx", torch.int32, required=True)
    _check(sched, "sched", torch.int32, (p.rows,))
    odt = torch.float32 if c.out_dtype == N.FP_OUT_FP32 else torch.bfloat16
    oshape = (c.batch, c.seqlen, c.num_q_heads, 128)
    if o is None:
        if tuple(c.o_stride) != (c.seqlen * c.num_q_heads * 128, c.num_q_heads * 128, 128):
            raise FpError(N.FP_ERR_INVALID, "the problem was built for a strided o: pass that o")
        o = torch.empty(oshape, dtype=odt, device=q.device)
    else:
        _check_view(o, "o", odt, oshape, tuple(c.o_stride))
    lse = torch.empty((c.batch, c.num_q_heads, c.seqlen), dtype=torch.float32,
                      device=q.device) if with_lse else None
    lib = N.load()
    if workspace is None:
        workspace = torch.empty(N.check_size(lib.fp_prefill_workspace_size(p.ref)), dtype=torch.uint8,
                                device=q.device)
    N.check(lib.fp_sparse_prefill_scored(p.ref, _ptr(q), _ptr(k), _ptr(v), _ptr(q_scale), _ptr(k_scale),
                                         _ptr(v_scale), _ptr(scores), _ptr(vbar), _ptr(row_ptr), _ptr(col_idx),
                                         _ptr(sched), _ptr(o), _ptr(lse), _ptr(workspace), workspace.numel(),
                                         _stream()))
    return o, lse


def sparse_prefill(q, k, v, block: int, tau: float, softmax_scale: float = 0.0,
                   q_scale=None, k_scale=None, v_scale=None, with_lse: bool = True,
                   out_fp32: bool = False, correction: bool = True, variant: Optional[str] = None,
                   split_small: bool = False):
    """All three stages on the current stream. Returns a dict of device tensors."""
    p = make_problem(q, k, v, block, softmax_scale, out_fp32=out_fp32, correction=correction, variant=variant,
                     split_small=split_small)
    qbar, kbar, vbar, scores = fp_block_scores(p, q, k, v, q_scale, k_scale, v_scale)
    row_ptr, col_idx, sched = fp_select_blocks(p, scores, tau)
    if p.c.variant == N.FP_VARIANT_BLOCK_SCORE:
        o, lse = fp_sparse_prefill_scored(p, q, k, v, scores, vbar, row_ptr, col_idx, sched,
                                          q_scale, k_scale, v_scale, with_lse)
    else:
        o, lse = fp_sparse_prefill(p, q, k, v, kbar, vbar, row_ptr, col_idx, sched,
                                   q_scale, k_scale, v_scale, with_lse)
    return dict(problem=p, qbar=qbar, kbar=kbar, vbar=vbar, scores=scores, row_ptr=row_ptr,
                col_idx=col_idx, sched=sched, o=o, lse=lse)


# ---------------------------------------------------------------------------
# paged varlen
# ---------------------------------------------------------------------------
@dataclass
class VarlenProblem:
    c: FpVarlenProblem
    cu: np.ndarray
    lk: np.ndarray
    rows: int
    max_nnz: int
    ws_bytes: int

    @property
    def ref(self):
        return ctypes.byref(self.c)

    def host_ptrs(self):
        return (self.cu.ctypes.data_as(ctypes.c_void_p), self.lk.ctypes.data_as(ctypes.c_void_p))


def make_varlen_problem(q: torch.Tensor, cu_seqlens_q, seqlens_k, k_cache: torch.Tensor,
                        block_table: torch.Tensor, block: int = 128,
                        softmax_scale: float = 0.0) -> VarlenProblem:
    c = FpVarlenProblem()
    cu = np.ascontiguousarray(np.asarray(cu_seqlens_q, dtype=np.int32))
    lk = np.ascontiguousarray(np.asarray(seqlens_k, dtype=np.int32))
    c.num_seqs = len(lk)
    c.num_q_heads, c.head_dim = q.shape[1], q.shape[2]
    c.num_kv_heads = k_cache.shape[2]
    c.block = block
    c.page_size = k_cache.shape[1]
    c.dtype = N.FP_DTYPE_FP8_E4M3 if q.dtype == torch.uint8 else N.FP_DTYPE_BF16
    c.softmax_scale = softmax_scale
    c.max_pages_per_seq = block_table.shape[1]
    c.q_stride[0], c.q_stride[1] = q.stride(0), q.stride(1)
    c.kv_stride[0], c.kv_stride[1], c.kv_stride[2] = k_cache.stride(0), k_cache.stride(1), k_cache.stride(2)
    Hq = q.shape[1]
    c.o_stride[0], c.o_stride[1] = Hq * 128, 128
    lib = N.load()
    cup, lkp = cu.ctypes.data_as(ctypes.c_void_p), lk.ctypes.data_as(ctypes.c_void_p)
    rows = N.check_size(lib.fp_varlen_num_rows(ctypes.byref(c), cup, lkp))
    nnz = N.check_size(lib.fp_varlen_max_nnz(ctypes.byref(c), cup, lkp))
    ws = N.check_size(lib.fp_varlen_workspace_size(ctypes.byref(c), cup, lkp))
    return VarlenProblem(c, cu, lk, rows, nnz, ws)


def _paged_call(entry: str, vp: VarlenProblem, q, k_cache, v_cache, block_table, tau, with_lse, workspace,
                q_scale, k_scale, v_scale, pooled=()):
    c = vp.c
    dt = torch.uint8 if c.dtype == N.FP_DTYPE_FP8_E4M3 else torch.bfloat16
    if q.dim() != 3 or q.shape[0] != int(vp.cu[-1]) or q.shape[1] != c.num_q_heads:
        raise FpError(N.FP_ERR_INVALID, f"q must be packed [{int(vp.cu[-1])}, {c.num_q_heads}, 128] "
                                        f"(got {tuple(q.shape)})")
    _check_view(q, "q", dt, (int(vp.cu[-1]), c.num_q_heads, 128), tuple(c.q_stride))
    if k_cache.dim() != 4 or tuple(v_cache.shape) != tuple(k_cache.shape):
        raise FpError(N.FP_ERR_INVALID, f"k_cache and v_cache must share one shape [pages, page_size, Hkv, 128] "
                                        f"(got {tuple(k_cache.shape)} and {tuple(v_cache.shape)})")
    cshape = (k_cache.shape[0], c.page_size, c.num_kv_heads, 128)
    _check_view(k_cache, "k_cache", dt, cshape, tuple(c.kv_stride))
    _check_view(v_cache, "v_cache", dt, cshape, tuple(c.kv_stride))
    _check(block_table, "block_table", torch.int32, (c.num_seqs, c.max_pages_per_seq), required=True)
    nsb = (c.max_pages_per_seq * c.page_size + 127) // 128
    _check_scales(c.dtype == N.FP_DTYPE_FP8_E4M3, c.num_seqs, c.num_q_heads, c.num_kv_heads, nsb,
                  q_scale, k_scale, v_scale)
    if pooled:
        slots = k_cache.shape[0] * max(1, c.page_size // c.block)
        for t, name in zip(pooled, ("kbar_cache", "vbar_cache")):
            _check(t, name, torch.float32, (slots, c.num_kv_heads, 128), required=True)
    dev = q.device
    i32 = dict(dtype=torch.int32, device=dev)
    row_ptr = torch.empty(vp.rows + 1, **i32)
    col_idx = torch.empty(max(vp.max_nnz, 1), **i32)
    o = torch.empty((q.shape[0], q.shape[1], 128), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((q.shape[1], q.shape[0]), dtype=torch.float32, device=dev) if with_lse else None
    if workspace is None:
        workspace = torch.empty(vp.ws_bytes, dtype=torch.uint8, device=dev)
    cup, lkp = vp.host_ptrs()
    N.check(getattr(N.load(), entry)(vp.ref, _ptr(q), cup, lkp, _ptr(k_cache), _ptr(v_cache),
                                     _ptr(block_table), _ptr(q_scale), _ptr(k_scale), _ptr(v_scale),
                                     *[_ptr(t) for t in pooled], float(tau), _ptr(row_ptr),
                                     _ptr(col_idx), vp.max_nnz, _ptr(o), _ptr(lse),
                                     _ptr(workspace), workspace.numel(), _stream()))
    return o, lse, row_ptr, col_idx


def fp_sparse_prefill_paged(vp: VarlenProblem, q, k_cache, v_cache, block_table, tau: float,
                            with_lse: bool = True, workspace: Optional[torch.Tensor] = None,
                            q_scale=None, k_scale=None, v_scale=None):
    """E1-E6 on a paged varlen batch -> (o, lse, row_ptr, col_idx). fp8
    (uint8 E4M3FN codes) takes fp32 scales [num_seqs, H, nsb], one per 128
    positions of each sequence."""
    return _paged_call("fp_sparse_prefill_paged", vp, q, k_cache, v_cache, block_table, tau, with_lse,
                       workspace, q_scale, k_scale, v_scale)


def pooled_kv_slots(k_cache: torch.Tensor, block: int) -> int:
    """Slots of the pooled-KV cache beside a page cache [pages, page_size, Hkv, 128]:
    one per page, or page_size / block per page when pages hold several blocks."""
    return k_cache.shape[0] * max(1, k_cache.shape[1] // block)


def fp_sparse_prefill_paged_cached(vp: VarlenProblem, q, k_cache, v_cache, block_table, kbar_cache,
                                   vbar_cache, tau: float, with_lse: bool = True,
                                   workspace: Optional[torch.Tensor] = None,
                                   q_scale=None, k_scale=None, v_scale=None):
    """fp_sparse_prefill_paged with the pooled-KV cache kbar_cache / vbar_cache
    (fp32 [pooled_kv_slots(k_cache, block), Hkv, 128], kept across calls):
    complete blocks of each sequence's cached prefix are read from it, and
    complete blocks this call pools are written to it."""
    return _paged_call("fp_sparse_prefill_paged_cached", vp, q, k_cache, v_cache, block_table, tau, with_lse,
                       workspace, q_scale, k_scale, v_scale, pooled=(kbar_cache, vbar_cache))
