"""Exact decoders for the storage types of the MLA decode inputs (oracle side).

[Issue] Sec. 1 "Environment" and Sec. 4.1 "Arguments": the KV cache and q are
``float8_e4m3fn`` (OCP FP8, 4 exponent bits with bias 7, 3 mantissa bits, no
infinities, NaN only for the all-ones exponent+mantissa pattern); o is
``bfloat16``.  The bf16 run of the mixed-length workload stores q and the pool
as bfloat16.

The e4m3fn table is built from the bit formula, not from any library cast, so
that the exhaustive comparison against torch in the tests is a real pin.
"""

from __future__ import annotations

import numpy as np

E4M3FN_MAX = 448.0


def _e4m3fn_value(code: int) -> float:
    """Value of one float8_e4m3fn code (0..255) from its bit fields."""
    sign = -1.0 if (code >> 7) & 1 else 1.0
    exp = (code >> 3) & 0xF
    man = code & 0x7
    if exp == 0xF and man == 0x7:
        return float("nan")
    if exp == 0:  # subnormal: (m / 8) * 2^(1 - 7)
        return sign * (man / 8.0) * 2.0 ** -6
    return sign * (1.0 + man / 8.0) * 2.0 ** (exp - 7)


E4M3FN_TABLE = np.array([_e4m3fn_value(c) for c in range(256)], dtype=np.float64)
E4M3FN_TABLE.setflags(write=False)


def decode_e4m3fn(codes: np.ndarray) -> np.ndarray:
    """float8_e4m3fn codes (uint8 array) -> float64 array of the same shape."""
    codes = np.asarray(codes)
    if codes.dtype != np.uint8:
        raise TypeError(f"e4m3fn codes must be uint8, got {codes.dtype}")
    return E4M3FN_TABLE[codes]


def decode_bf16(codes: np.ndarray) -> np.ndarray:
    """bfloat16 codes (uint16 array) -> float64, exactly.

    A bfloat16 is the upper half of an IEEE binary32, so widening the code by 16
    zero bits gives the binary32 bit pattern of the same value.
    """
    codes = np.asarray(codes)
    if codes.dtype != np.uint16:
        raise TypeError(f"bf16 codes must be uint16, got {codes.dtype}")
    wide = codes.astype(np.uint32) << np.uint32(16)
    with np.errstate(invalid="ignore"):  # NaN codes stay NaN
        return wide.view(np.float32).astype(np.float64)


def decode_fp32(codes: np.ndarray) -> np.ndarray:
    """binary32 values (float32 array, or uint32 bit patterns) -> float64."""
    codes = np.asarray(codes)
    if codes.dtype == np.uint32:
        codes = codes.view(np.float32)
    if codes.dtype != np.float32:
        raise TypeError(f"fp32 input must be float32 or uint32, got {codes.dtype}")
    return codes.astype(np.float64)


def decode(codes: np.ndarray, dtype: str) -> np.ndarray:
    """Decode raw codes of storage type ``dtype`` ('fp8', 'bf16' or 'fp32')."""
    if dtype == "fp8":
        return decode_e4m3fn(codes)
    if dtype == "bf16":
        return decode_bf16(codes)
    if dtype == "fp32":
        return decode_fp32(codes)
    raise ValueError(f"unknown storage dtype {dtype!r}")
