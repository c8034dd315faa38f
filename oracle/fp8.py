"""OCP 8-bit floating point E4M3FN decode, written from the OCP FP8 specification
(4 exponent bits with bias 7, 3 mantissa bits, no infinities, S.1111.111 is
NaN, largest finite 448). Test infrastructure only.

The pages say only that the operator supports FP8 inference (lode.cx page,
operator paragraph; aimodeling.com page, "Operator alignment" bullet); the
codec and per-128-token scales are this library's stated format.
"""
from __future__ import annotations

import numpy as np


def _decode_one(code: int) -> float:
    sign = -1.0 if code & 0x80 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return float("nan")
    if e == 0:
        return sign * (m / 8.0) * 2.0 ** (1 - 7)        # subnormal
    return sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)


_TABLE = np.array([_decode_one(c) for c in range(256)], dtype=np.float64)


def decode_e4m3(codes: np.ndarray) -> np.ndarray:
    """uint8 codes -> float64 values."""
    return _TABLE[np.asarray(codes, dtype=np.uint8)]


def widen_fp8(codes: np.ndarray, scales: np.ndarray, block: int = 128, pos0: int = 0) -> np.ndarray:
    """codes [T, H, d] uint8 for positions pos0 .. pos0 + T - 1 and scales
    [H, nsb] float32 (one per 128 positions, nsb >= ceil((pos0 + T)/block))
    -> float64 values code * scale (the scale of the token's 128-position
    block)."""
    T = codes.shape[0]
    x = decode_e4m3(codes)
    sc = np.asarray(scales, dtype=np.float64)             # [H, nsb]
    per_tok = np.repeat(sc, block, axis=1)[:, pos0:pos0 + T]   # [H, T]
    assert per_tok.shape[1] == T
    return x * per_tok.T[:, :, None]
