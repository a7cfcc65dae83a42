"""Exact decoders for the cache element formats (oracle side, test infrastructure).

The pages only say the cache is "fp8" ("perf(mla): chunk the non-FP4
gather_kv_b_proj over KV", description and table; the HK kernel files are named
``*_fp8_fp8``). The reading taken: OCP e4m3fn, the format whose largest finite
value is 448, so a per-tensor scale of ``amax / 448`` maps the tensor onto the
full range. Layout of a byte: 1 sign bit, 4 exponent bits (bias 7), 3 mantissa
bits. Exponent 0 is subnormal (``m/8 * 2**-6``); exponent 15 with mantissa 7 is
NaN; there is no infinity.

bf16 is the top half of an IEEE binary32, so widening is exact.
"""

import math

import numpy as np


def _e4m3fn_value(byte: int) -> float:
    sign = -1.0 if (byte >> 7) & 1 else 1.0
    exponent = (byte >> 3) & 0xF
    mantissa = byte & 0x7
    if exponent == 0xF and mantissa == 0x7:
        return math.nan
    if exponent == 0:
        return sign * (mantissa / 8.0) * 2.0 ** -6
    return sign * (1.0 + mantissa / 8.0) * 2.0 ** (exponent - 7)


# Table of all 256 byte values, built from the bit formula above (float64).
E4M3FN_VALUES = np.array([_e4m3fn_value(b) for b in range(256)], dtype=np.float64)


def decode_e4m3fn(raw) -> np.ndarray:
    """Decode e4m3fn bytes (any integer array) to exact float64 values."""
    return E4M3FN_VALUES[np.asarray(raw, dtype=np.uint8)]


def bf16_bits_to_f64(bits) -> np.ndarray:
    """Widen bf16 bit patterns (uint16) to float64, exactly."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)
