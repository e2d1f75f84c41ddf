"""OCP FP8 E4M3FN decoding, from the format definition (test infrastructure).

The Sage page ("bsa_attn_sm120_blk64_sage_fwd", Parameters: v_fp8) stores V as
"FP8 E4M3".  We read that as the OCP 8-bit E4M3 "FN" variant: 1 sign bit, 4
exponent bits with bias 7, 3 mantissa bits, no infinities, and NaN only for the
all-ones exponent-and-mantissa pattern.  Largest finite magnitude 448.
"""
from __future__ import annotations

import numpy as np


def e4m3_value(code: int) -> float:
    """Exact value of one E4M3FN code (0..255) as a Python float."""
    code = int(code) & 0xFF
    sign = -1.0 if (code >> 7) & 1 else 1.0
    exp = (code >> 3) & 0xF
    man = code & 0x7
    if exp == 0xF and man == 0x7:
        return float("nan")
    if exp == 0:                       # subnormal: 2^(1-bias) * m/8
        return sign * (man / 8.0) * 2.0 ** (1 - 7)
    return sign * (1.0 + man / 8.0) * 2.0 ** (exp - 7)


_TABLE = np.array([e4m3_value(c) for c in range(256)], dtype=np.float64)


def e4m3_decode(codes: np.ndarray) -> np.ndarray:
    """Decode an array of uint8 codes to float64."""
    return _TABLE[np.asarray(codes, dtype=np.uint8)]
