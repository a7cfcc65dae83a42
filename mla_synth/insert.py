"""Seeded inputs for the decode epilogue (query concat + latent-cache insert).

Recipe (deterministic for a given seed; each part from its own stream
``default_rng([seed, 20 + part])``):

* ``ql_nope [T, H, 512]``, ``q_pe [T, H, 64]``, ``kv_c [T, 512]``, ``k_pe [T, 64]``
  ~ N(0, 1) in float32, rounded to bf16 (RNE, by torch);
* a rope table ``cos_sin [P, 64]``: for position p and pair i < 32,
  ``cos(p * 10000^(-i/32))`` then ``sin(...)``, computed in float64 and rounded to
  float32 (the usual rotary frequencies over 64 dims; the pages give none);
* ``positions [T]`` uniform in [0, P); ``slot_mapping [T]``: distinct slots from a
  permutation of the cache, every ``pad_every``-th token set to -1 (padding);
* the cache before the call: random bytes, so untouched rows are checked too;
* fp8 ``kv_scale = float32(amax / 448)`` over ``kv_c`` and ``k_pe``.
"""

from dataclasses import dataclass

import numpy as np
import torch

FP8_MAX = 448.0


@dataclass
class InsertCase:
    num_tokens: int
    num_heads: int
    kv_dtype: str
    kv_scale: float
    num_slots: int
    rope_positions: int
    neox: bool
    ql_nope: np.ndarray       # uint16 [T, H, 512]
    q_pe: np.ndarray          # uint16 [T, H, 64]
    kv_c: np.ndarray          # uint16 [T, 512]
    k_pe: np.ndarray          # uint16 [T, 64]
    positions: np.ndarray     # int32 [T]
    cos_sin: np.ndarray       # float32 [P, 64]
    slot_mapping: np.ndarray  # int64 [T]
    cache: np.ndarray         # uint16 [S, 576] (bf16) or uint8 [S, 576] (fp8)


def _bf16_bits(x: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def make_insert_case(*, num_tokens, num_heads, kv_dtype, num_slots=None, rope_positions=4096, neox=False,
                     pad_every=0, seed=0) -> InsertCase:
    T, H = int(num_tokens), int(num_heads)
    S = int(num_slots) if num_slots is not None else max(2 * T, 16)
    rng = lambda part: np.random.default_rng([seed, 20 + part])
    ql_nope = _bf16_bits(rng(0).standard_normal((T, H, 512), dtype=np.float32))
    q_pe = _bf16_bits(rng(1).standard_normal((T, H, 64), dtype=np.float32))
    kv_c_f = rng(2).standard_normal((T, 512), dtype=np.float32)
    k_pe_f = rng(3).standard_normal((T, 64), dtype=np.float32)
    kv_c, k_pe = _bf16_bits(kv_c_f), _bf16_bits(k_pe_f)
    freqs = 10000.0 ** (-np.arange(32, dtype=np.float64) / 32)
    ang = np.outer(np.arange(rope_positions, dtype=np.float64), freqs)
    cos_sin = np.concatenate([np.cos(ang), np.sin(ang)], axis=1).astype(np.float32)
    positions = rng(4).integers(0, rope_positions, T).astype(np.int32)
    slot_mapping = rng(5).permutation(S)[:T].astype(np.int64)
    if pad_every:
        slot_mapping[::pad_every] = -1
    if kv_dtype == "bf16":
        cache = rng(6).integers(0, 1 << 16, (S, 576), dtype=np.uint16)
        kv_scale = 1.0
    else:
        cache = rng(6).integers(0, 1 << 8, (S, 576), dtype=np.uint8)
        amax = float(max(np.abs(kv_c_f).max(initial=0.0), np.abs(k_pe_f).max(initial=0.0)))
        kv_scale = float(np.float32(amax / FP8_MAX)) if amax > 0 else 1.0
    return InsertCase(T, H, kv_dtype, kv_scale, S, int(rope_positions), bool(neox), ql_nope, q_pe, kv_c, k_pe,
                      positions, cos_sin, slot_mapping, cache)


# Epilogue workloads: the pages' dispatch boundary sits at 64 tokens; 8 local heads
# give the (token, head + 1) = 9 rows per token of the pages' concurrency-1 case.
INSERT_WORKLOADS = {
    "insert_t1_h8_fp8": dict(num_tokens=1, num_heads=8, kv_dtype="fp8_e4m3fn", seed=60),
    "insert_t64_h8_fp8": dict(num_tokens=64, num_heads=8, kv_dtype="fp8_e4m3fn", seed=61),
    "insert_t65_h8_fp8": dict(num_tokens=65, num_heads=8, kv_dtype="fp8_e4m3fn", seed=62),
    "insert_t256_h128_fp8": dict(num_tokens=256, num_heads=128, kv_dtype="fp8_e4m3fn", seed=63),
}
