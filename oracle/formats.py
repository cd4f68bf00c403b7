"""Decoders of the stored number formats, written from the format definitions.

bf16: the upper 16 bits of an IEEE-754 binary32 value (1 sign, 8 exponent,
7 fraction bits); decoding pads 16 zero bits below and widens to float64,
which is exact.

fp8 E4M3 (the OCP "E4M3FN" encoding the fine-grained FP8 scheme relies on;
"DeepSeekMoE架构解析" section 4.3 names the tile/block-scaled FP8 format, and
this library's workloads store one fp32 scale per output row): 1 sign bit,
4 exponent bits with bias 7, 3 mantissa bits; exponent field 0 encodes
subnormals m/8 * 2^-6; the all-ones exponent with mantissa 7 is NaN; there is
no infinity; the largest finite magnitude is 1.75 * 2^8 = 448.
"""

from __future__ import annotations

import numpy as np


def bf16_to_f64(u16: np.ndarray) -> np.ndarray:
    u16 = np.asarray(u16)
    if u16.dtype != np.uint16:
        raise TypeError("bf16 values are passed as their uint16 bit patterns")
    return (u16.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def f64_to_bf16_bits(v: np.ndarray) -> np.ndarray:
    """Round float64 values to bf16 (round to nearest, ties to even), in one
    step from float64: a bf16 number has 8 significant bits and the binary32
    exponent range, so the spacing at v is 2^(e-8) for |v| in [2^(e-1), 2^e),
    and never below 2^-133 (the bf16 subnormal spacing). Finite inputs within
    the binary32 range. Returns the uint16 bit patterns."""
    v = np.asarray(v, dtype=np.float64)
    if not np.all(np.isfinite(v)):
        raise ValueError("finite values only")
    _, ex = np.frexp(v)
    q = np.ldexp(1.0, np.maximum(ex - 8, -133))
    r = np.rint(v / q) * q                     # rint: round half to even
    r32 = r.astype(np.float32)
    if not np.array_equal(r32.astype(np.float64), r):
        raise ValueError("value outside the bf16 range")
    return (r32.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def _e4m3_value(code: int) -> float:
    sign = -1.0 if (code >> 7) & 1 else 1.0
    exp = (code >> 3) & 0xF
    man = code & 0x7
    if exp == 0xF and man == 0x7:
        return float("nan")
    if exp == 0:
        return sign * (man / 8.0) * 2.0 ** (-6)
    return sign * (1.0 + man / 8.0) * 2.0 ** (exp - 7)


E4M3_TABLE = np.array([_e4m3_value(c) for c in range(256)], dtype=np.float64)


def e4m3_to_f64(u8: np.ndarray) -> np.ndarray:
    u8 = np.asarray(u8)
    if u8.dtype != np.uint8:
        raise TypeError("fp8 values are passed as their uint8 codes")
    return E4M3_TABLE[u8]


def decode_stored(arr: np.ndarray, row_scale: np.ndarray | None = None) -> np.ndarray:
    """Stored array -> float64. uint16 = bf16 bits, uint8 = e4m3 codes (times
    the fp32 scale of each row, i.e. of the last-but-one axis), float32 as is."""
    arr = np.asarray(arr)
    if arr.dtype == np.uint16:
        out = bf16_to_f64(arr)
    elif arr.dtype == np.uint8:
        if row_scale is None:
            raise ValueError("fp8 codes need their per-row scales")
        out = e4m3_to_f64(arr) * np.asarray(row_scale, dtype=np.float64)[..., None]
    elif arr.dtype == np.float32 or arr.dtype == np.float64:
        out = arr.astype(np.float64)
    else:
        raise TypeError(f"unsupported stored dtype {arr.dtype}")
    if not np.all(np.isfinite(out)):
        raise ValueError("inputs must be finite")
    return out
