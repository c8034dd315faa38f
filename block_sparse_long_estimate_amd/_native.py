"""ctypes view of the C ABI in include/fp_prefill.h (no torch types cross it)."""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_NAME = "libfp_prefill.so"
# FP_PREFILL_LIB selects another build of the same library (same ABI).
LIB_PATH = os.environ.get("FP_PREFILL_LIB") or os.path.join(_HERE, LIB_NAME)

FP_OK = 0
FP_ERR_INVALID = -1
FP_ERR_UNSUPPORTED = -2
FP_ERR_CAPACITY = -3
FP_ERR_HIP = -4
FP_DTYPE_BF16 = 0
FP_DTYPE_FP8_E4M3 = 1
FP_OUT_BF16 = 0
FP_OUT_FP32 = 2
FP_VARIANT_MEAN_CORRECTION = 0
FP_VARIANT_NO_CORRECTION = 1
FP_VARIANT_PER_HEAD_LISTS = 2
FP_VARIANT_BLOCK_SCORE = 3
FP_SPLIT_OFF = 0
FP_SPLIT_SMALL_GRIDS = 1

EXPORTS = (
    "fp_version", "fp_last_error", "fp_num_rows", "fp_max_nnz", "fp_workspace_size",
    "fp_prefill_workspace_size",
    "fp_block_scores", "fp_select_blocks", "fp_sparse_prefill",
    "fp_varlen_num_rows", "fp_varlen_max_nnz", "fp_varlen_workspace_size",
    "fp_sparse_prefill_paged", "fp_sparse_prefill_noalloc", "fp_dense_prefill",
    "fp_estimate_select", "fp_estimate_select_workspace_size", "fp_sparse_prefill_scored",
    "fp_sparse_prefill_paged_cached",
)
FP_NOALLOC_MAX_POOLED_ROWS = 32768
FP_NOALLOC_SCRATCH_BYTES = 36 << 20


class FpProblem(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32), ("seqlen", ctypes.c_int32),
        ("num_q_heads", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32), ("block", ctypes.c_int32), ("dtype", ctypes.c_int32),
        ("softmax_scale", ctypes.c_float),
        ("q_stride", ctypes.c_int64 * 3), ("k_stride", ctypes.c_int64 * 3),
        ("v_stride", ctypes.c_int64 * 3), ("o_stride", ctypes.c_int64 * 3),
        ("out_dtype", ctypes.c_int32), ("variant", ctypes.c_int32),
        ("split", ctypes.c_int32), ("reserved_", ctypes.c_int32),
    ]


class FpVarlenProblem(ctypes.Structure):
    _fields_ = [
        ("num_seqs", ctypes.c_int32), ("num_q_heads", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
        ("block", ctypes.c_int32), ("page_size", ctypes.c_int32), ("dtype", ctypes.c_int32),
        ("softmax_scale", ctypes.c_float), ("max_pages_per_seq", ctypes.c_int32),
        ("pad_", ctypes.c_int32),
        ("q_stride", ctypes.c_int64 * 2), ("kv_stride", ctypes.c_int64 * 3),
        ("o_stride", ctypes.c_int64 * 2),
    ]


_lib = None


def load() -> ctypes.CDLL:
    """Load the in-tree HIP library; raise if it was not built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it first "
                           "(python -c 'import __graft_entry__ as g; g.build()')")
    lib = ctypes.CDLL(LIB_PATH)
    P = ctypes.POINTER(FpProblem)
    VP = ctypes.POINTER(FpVarlenProblem)
    vp, i32p = ctypes.c_void_p, ctypes.c_void_p
    lib.fp_version.restype = ctypes.c_char_p
    lib.fp_last_error.restype = ctypes.c_char_p
    for name in ("fp_num_rows", "fp_max_nnz", "fp_workspace_size", "fp_prefill_workspace_size",
                 "fp_estimate_select_workspace_size"):
        f = getattr(lib, name)
        f.restype, f.argtypes = ctypes.c_int64, [P]
    for name in ("fp_varlen_num_rows", "fp_varlen_max_nnz", "fp_varlen_workspace_size"):
        f = getattr(lib, name)
        f.restype, f.argtypes = ctypes.c_int64, [VP, i32p, i32p]
    lib.fp_block_scores.restype = ctypes.c_int
    lib.fp_block_scores.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp]
    lib.fp_select_blocks.restype = ctypes.c_int
    lib.fp_select_blocks.argtypes = [P, vp, ctypes.c_float, vp, vp, ctypes.c_int64, vp, vp,
                                     ctypes.c_size_t, vp]
    lib.fp_sparse_prefill.restype = ctypes.c_int
    lib.fp_sparse_prefill.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                      ctypes.c_size_t, vp]
    lib.fp_estimate_select.restype = ctypes.c_int
    lib.fp_estimate_select.argtypes = [P, vp, vp, vp, vp, vp, vp, ctypes.c_float, vp, vp, vp, vp, vp,
                                       ctypes.c_int64, vp, vp, ctypes.c_size_t, vp]
    lib.fp_sparse_prefill_scored.restype = ctypes.c_int
    lib.fp_sparse_prefill_scored.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                             ctypes.c_size_t, vp]
    lib.fp_dense_prefill.restype = ctypes.c_int
    lib.fp_dense_prefill.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, vp]
    lib.fp_sparse_prefill_noalloc.restype = ctypes.c_int
    lib.fp_sparse_prefill_noalloc.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp]
    lib.fp_sparse_prefill_paged.restype = ctypes.c_int
    lib.fp_sparse_prefill_paged.argtypes = [VP, vp, i32p, i32p, vp, vp, vp, vp, vp, vp, ctypes.c_float,
                                            vp, vp, ctypes.c_int64, vp, vp, vp, ctypes.c_size_t, vp]
    lib.fp_sparse_prefill_paged_cached.restype = ctypes.c_int
    lib.fp_sparse_prefill_paged_cached.argtypes = [VP, vp, i32p, i32p, vp, vp, vp, vp, vp, vp, vp, vp,
                                                   ctypes.c_float, vp, vp, ctypes.c_int64, vp, vp, vp,
                                                   ctypes.c_size_t, vp]
    _lib = lib
    return lib


class FpError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"[{code}] {msg}")
        self.code = code


def check(rc: int) -> None:
    if rc != FP_OK:
        raise FpError(rc, load().fp_last_error().decode())


def check_size(v: int) -> int:
    if v < 0:
        raise FpError(int(v), load().fp_last_error().decode())
    return int(v)
