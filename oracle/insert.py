"""Reference for the decode epilogue that produces this path's inputs: query
concatenation and latent-cache insert (test infrastructure).

Page "[Perf][Kimi-K3] Cut MLA decode concat/cache epilogue latency" (Purpose and
its list of changes): one fused kernel sits between the absorbed-query GEMM and
the decode attention. It joins the query parts ``ql_nope`` and ``q_pe`` into the
576-wide query and writes each new token's latent row into the cache at
``slot_mapping``, reading the scales and a rope table; its rows are (token,
head + 1): H query rows and one cache row per token. The page prints no
per-element arithmetic. The readings taken here:

* ``q[t, h, 0:512] = ql_nope[t, h]`` and ``q[t, h, 512:576] = q_pe[t, h]``, a
  bit copy of bf16 values; ``q_pe`` is not rotated here.
* The cache row of token t goes to slot ``slot_mapping[t]``; a negative slot
  means no write (a padding token). Columns 0:512 are ``kv_c[t]``, columns
  512:576 are ``rope(k_pe[t])`` at ``positions[t]``.
* Rope uses a table ``cos_sin[pos] = (cos[0:32], sin[0:32])`` of float32 and
  rotates 32 pairs (x, y), either interleaved (2i, 2i+1) or split halves
  (i, i + 32): ``x' = x c - y s`` and ``y' = y c + x s``. Each product is
  rounded to float32, then the sum; there is no fused multiply-add.
* bf16 cache: round to nearest, ties to even, of the float32 value. fp8 cache:
  e4m3fn of ``value / kv_scale`` (a float32 division), saturated to +-448,
  nearest with ties to the even code; NaN becomes 0x7f.

Every function here is written from these definitions in plain numpy and is
pinned in ``tests/test_oracle_insert.py``.
"""

import numpy as np

from .fp8 import E4M3FN_VALUES

LATENT = 512
ROPE = 64
ROW = LATENT + ROPE

# Positive finite e4m3fn values in code order 0x00 .. 0x7e (increasing).
_POS_VALUES = E4M3FN_VALUES[:0x7F].astype(np.float64)


def bf16_bits_to_f32(bits) -> np.ndarray:
    """bf16 bit patterns (uint16) to float32, exactly."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def f32_to_bf16_rne(x) -> np.ndarray:
    """float32 to bf16 bits: keep the top 16 bits, rounding to nearest with ties
    to even on the 16 bits dropped. NaN becomes the quiet NaN with its sign."""
    x = np.asarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    nan = np.isnan(x)
    out = rounded.astype(np.uint16)
    out[nan] = ((u[nan] >> 16).astype(np.uint16) & np.uint16(0x8000)) | np.uint16(0x7FC0)
    return out


def f32_to_e4m3fn(x) -> np.ndarray:
    """float32 to e4m3fn codes: the nearest finite value, ties to the even code,
    magnitudes beyond 448 saturated to 448, the sign kept (-0 -> 0x80), NaN -> 0x7f."""
    x = np.asarray(x, dtype=np.float32)
    a = np.minimum(np.abs(x.astype(np.float64)), 448.0)
    hi = np.searchsorted(_POS_VALUES, a, side="left")  # first value >= a
    hi = np.minimum(hi, 0x7E)
    lo = np.maximum(hi - 1, 0)
    d_hi = _POS_VALUES[hi] - a
    d_lo = a - _POS_VALUES[lo]
    pick_lo = (d_lo < d_hi) | ((d_lo == d_hi) & (lo % 2 == 0))
    code = np.where(pick_lo, lo, hi).astype(np.uint8)
    code = np.where(np.signbit(x), code | np.uint8(0x80), code).astype(np.uint8)
    return np.where(np.isnan(x), np.uint8(0x7F), code).astype(np.uint8)


def rope_f32(x, cos, sin, neox: bool) -> np.ndarray:
    """Rotate the 32 pairs of each 64-wide row of x (float32 [..., 64]) by the
    angles whose cosines and sines are cos, sin (float32 [..., 32])."""
    x = np.asarray(x, dtype=np.float32)
    cos = np.asarray(cos, dtype=np.float32)
    sin = np.asarray(sin, dtype=np.float32)
    if neox:
        first, second = x[..., :32], x[..., 32:]
    else:
        first, second = x[..., 0::2], x[..., 1::2]
    a = (first * cos) - (second * sin)   # float32 products, then the float32 difference
    b = (second * cos) + (first * sin)
    out = np.empty_like(x)
    if neox:
        out[..., :32], out[..., 32:] = a, b
    else:
        out[..., 0::2], out[..., 1::2] = a, b
    return out


def qcat_cache_insert_reference(ql_nope, q_pe, kv_c, k_pe, positions, cos_sin, slot_mapping, cache,
                                kv_dtype: str, kv_scale: float, neox: bool):
    """Returns (q, cache, status) after the epilogue.

    ql_nope uint16 [T, H, 512], q_pe uint16 [T, H, 64], kv_c uint16 [T, 512],
    k_pe uint16 [T, 64] (bf16 bits); positions int [T]; cos_sin float32 [P, 64];
    slot_mapping int [T]; cache uint16 [S, 576] (bf16) or uint8 [S, 576] (fp8),
    copied, not modified. status bit 1: a slot at or past the cache end; bit 2:
    a position outside the table (that token's cache row is not written)."""
    ql_nope = np.asarray(ql_nope, dtype=np.uint16)
    q_pe = np.asarray(q_pe, dtype=np.uint16)
    T = ql_nope.shape[0]
    q = np.concatenate([ql_nope, q_pe], axis=-1)
    out = np.array(cache, copy=True)
    status = 0
    for t in range(T):
        slot = int(slot_mapping[t])
        if slot < 0:
            continue
        if slot >= out.shape[0]:
            status |= 1
            continue
        pos = int(positions[t])
        if not 0 <= pos < cos_sin.shape[0]:
            status |= 2
            continue
        latent = bf16_bits_to_f32(kv_c[t])
        rot = rope_f32(bf16_bits_to_f32(k_pe[t]), cos_sin[pos, :32], cos_sin[pos, 32:], neox)
        if kv_dtype == "bf16":
            out[slot, :LATENT] = np.asarray(kv_c[t], dtype=np.uint16)
            out[slot, LATENT:] = f32_to_bf16_rne(rot)
        elif kv_dtype == "fp8_e4m3fn":
            s = np.float32(kv_scale)
            out[slot, :LATENT] = f32_to_e4m3fn(latent / s)
            out[slot, LATENT:] = f32_to_e4m3fn(rot / s)
        else:
            raise ValueError(kv_dtype)
    return q, out, status
