"""Number formats, decoded from their definitions (oracle side).

* bfloat16: the upper 16 bits of an IEEE-754 binary32.
* OCP 8-bit floating point, E4M3FN variant (OCP "8-bit Floating Point
  Specification (OFP8)" rev. 1.0): 1 sign bit, 4 exponent bits with bias 7,
  3 mantissa bits; exponent field 0 encodes subnormals m/8 * 2^-6; there are
  no infinities and S.1111.111 is NaN, so the largest finite value is
  1.75 * 2^8 = 448.
"""
from __future__ import annotations

import numpy as np


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def e4m3fn_value(code: int) -> float:
    """Value of one E4M3FN code, computed from the field definitions."""
    code = int(code) & 0xFF
    s = -1.0 if code & 0x80 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return float("nan")
    if e == 0:
        return s * (m / 8.0) * 2.0 ** (1 - 7)
    return s * (1.0 + m / 8.0) * 2.0 ** (e - 7)


E4M3FN_TABLE = np.array([e4m3fn_value(c) for c in range(256)], dtype=np.float64)


def e4m3fn_to_f64(codes: np.ndarray) -> np.ndarray:
    return E4M3FN_TABLE[np.asarray(codes, dtype=np.uint8)]


def dequant_block128(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """W[i, j] = e4m3fn(codes[i, j]) * scales[i // 128, j // 128] in float64."""
    q = e4m3fn_to_f64(codes)
    rows, cols = q.shape
    s = np.asarray(scales, dtype=np.float64)
    if s.shape != ((rows + 127) // 128, (cols + 127) // 128):
        raise ValueError("scale grid does not match 128x128 blocks")
    full = np.repeat(np.repeat(s, 128, axis=0), 128, axis=1)[:rows, :cols]
    return q * full
