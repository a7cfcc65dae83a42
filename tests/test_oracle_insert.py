"""Pins of the epilogue oracle (query concat + latent-cache insert), CPU only.

The encoders are checked against torch's own casts and hand-derived codes, rope
against closed forms and a float64 complex product, the insert against its
structure (copies, skipped slots, status bits)."""

import numpy as np
import pytest
import torch

from oracle.fp8 import E4M3FN_VALUES
from oracle.insert import (bf16_bits_to_f32, f32_to_bf16_rne, f32_to_e4m3fn, qcat_cache_insert_reference,
                           rope_f32)


# ------------------------------------------------------------------ encoders

def test_e4m3fn_codes_round_trip():
    codes = np.array([c for c in range(256) if not np.isnan(E4M3FN_VALUES[c])], dtype=np.uint8)
    vals = E4M3FN_VALUES[codes].astype(np.float32)
    assert np.array_equal(f32_to_e4m3fn(vals), codes)  # -0.0 included (0x80)


@pytest.mark.parametrize("x,code", [
    (1.0, 0x38), (1.0625, 0x38), (1.1875, 0x3A), (-1.1875, 0xBA), (448.0, 0x7E), (464.0, 0x7E),
    (1e6, 0x7E), (-1e6, 0xFE), (float("inf"), 0x7E), (0.0, 0x00), (-0.0, 0x80), (2.0 ** -9, 0x01),
    (2.0 ** -10, 0x00), (3 * 2.0 ** -10, 0x02), (2.0 ** -6, 0x08), (0.0146484375, 0x08),
    (float("nan"), 0x7F),
])
def test_e4m3fn_hand_codes(x, code):
    # ties: 1.0625 lies halfway between 1.0 (0x38) and 1.125 (0x39) -> even 0x38;
    # 1.1875 halfway between 0x39 and 1.25 (0x3a) -> 0x3a; 2^-10 halfway between 0 and
    # 2^-9 -> 0; 3 * 2^-10 halfway between 2^-9 (0x01) and 2^-8 (0x02) -> 0x02;
    # 0.0146484375 = 2^-6 - 2^-10 halfway between 7 * 2^-9 (0x07) and 2^-6 (0x08) -> 0x08
    assert int(f32_to_e4m3fn(np.float32(x))) == code


def test_e4m3fn_matches_torch_in_range():
    rng = np.random.default_rng(5)
    x = np.concatenate([rng.standard_normal(20000) * 40, rng.uniform(-448, 448, 20000),
                        (E4M3FN_VALUES[:0x7E] + E4M3FN_VALUES[1:0x7F]) / 2,  # every midpoint (ties)
                        -(E4M3FN_VALUES[:0x7E] + E4M3FN_VALUES[1:0x7F]) / 2]).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(f32_to_e4m3fn(x), ref)


def test_bf16_rne_matches_torch():
    rng = np.random.default_rng(6)
    u = rng.integers(0, 2 ** 32, 50000, dtype=np.uint64).astype(np.uint32)
    x = u.view(np.float32)
    x = x[np.isfinite(x)]
    ties = ((rng.integers(0, 2 ** 16, 5000, dtype=np.uint32) << 16) | 0x8000).view(np.float32)
    x = np.concatenate([x, ties[np.isfinite(ties)], rng.standard_normal(20000).astype(np.float32)])
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(f32_to_bf16_rne(x), ref)


# ------------------------------------------------------------------ rope

def _rand_row(rng, n=64):
    return rng.standard_normal(n).astype(np.float32)


@pytest.mark.parametrize("neox", [False, True])
def test_rope_identity_and_quarter_turn(neox):
    rng = np.random.default_rng(7)
    x = _rand_row(rng)
    one, zero = np.ones(32, np.float32), np.zeros(32, np.float32)
    assert np.array_equal(rope_f32(x, one, zero, neox), x)
    y = rope_f32(x, zero, one, neox)  # (a, b) -> (-b, a) exactly
    if neox:
        assert np.array_equal(y[:32], -x[32:]) and np.array_equal(y[32:], x[:32])
    else:
        assert np.array_equal(y[0::2], -x[1::2]) and np.array_equal(y[1::2], x[0::2])


def test_rope_styles_differ_by_a_fixed_permutation():
    rng = np.random.default_rng(8)
    x = _rand_row(rng)
    ang = rng.uniform(0, 2 * np.pi, 32)
    c, s = np.cos(ang).astype(np.float32), np.sin(ang).astype(np.float32)
    perm = np.empty(64, dtype=int)  # interleaved position 2i <- halves position i, 2i+1 <- i + 32
    perm[0::2], perm[1::2] = np.arange(32), np.arange(32) + 32
    assert np.array_equal(rope_f32(x[perm], c, s, neox=False), rope_f32(x, c, s, neox=True)[perm])


@pytest.mark.parametrize("neox", [False, True])
def test_rope_close_to_the_complex_product(neox):
    rng = np.random.default_rng(9)
    for _ in range(50):
        x = _rand_row(rng)
        ang = rng.uniform(0, 2 * np.pi, 32)
        c, s = np.cos(ang).astype(np.float32), np.sin(ang).astype(np.float32)
        y = rope_f32(x, c, s, neox).astype(np.float64)
        first, second = (x[:32], x[32:]) if neox else (x[0::2], x[1::2])
        z = (first.astype(np.float64) + 1j * second.astype(np.float64)) * (c.astype(np.float64) + 1j * s)
        yr, yi = (y[:32], y[32:]) if neox else (y[0::2], y[1::2])
        bound = 4 * 2.0 ** -24 * (np.abs(first) + np.abs(second))  # two rounded products and a rounded sum
        assert np.all(np.abs(yr - z.real) <= bound) and np.all(np.abs(yi - z.imag) <= bound)


# ------------------------------------------------------------------ the insert

def _case(rng, T=5, H=3, slots=16, P=40):
    bits = lambda *shape: (rng.standard_normal(shape).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    ang = np.outer(np.arange(P), 10000.0 ** (-np.arange(32) / 32))
    cos_sin = np.concatenate([np.cos(ang), np.sin(ang)], axis=1).astype(np.float32)
    return dict(ql_nope=bits(T, H, 512), q_pe=bits(T, H, 64), kv_c=bits(T, 512), k_pe=bits(T, 64),
                positions=rng.integers(0, P, T), cos_sin=cos_sin, slot_mapping=rng.permutation(slots)[:T])


@pytest.mark.parametrize("kv_dtype", ["bf16", "fp8_e4m3fn"])
def test_insert_structure(kv_dtype):
    rng = np.random.default_rng(10)
    c = _case(rng)
    c["slot_mapping"][1] = -1
    dt = np.uint16 if kv_dtype == "bf16" else np.uint8
    cache = rng.integers(0, 2 ** (16 if dt == np.uint16 else 8), (16, 576)).astype(dt)
    q, out, status = qcat_cache_insert_reference(cache=cache, kv_dtype=kv_dtype, kv_scale=0.02, neox=False, **c)
    assert status == 0
    assert np.array_equal(q[..., :512], c["ql_nope"]) and np.array_equal(q[..., 512:], c["q_pe"])
    written = {int(s) for s in c["slot_mapping"] if s >= 0}
    untouched = [s for s in range(16) if s not in written]
    assert np.array_equal(out[untouched], cache[untouched])
    for t, slot in enumerate(c["slot_mapping"]):
        if slot < 0:
            continue
        latent = bf16_bits_to_f32(c["kv_c"][t]).astype(np.float64)
        pos = c["positions"][t]
        rot = rope_f32(bf16_bits_to_f32(c["k_pe"][t]), c["cos_sin"][pos, :32], c["cos_sin"][pos, 32:], False)
        if kv_dtype == "bf16":
            assert np.array_equal(out[slot, :512], c["kv_c"][t])
            assert np.all(np.abs(bf16_bits_to_f32(out[slot, 512:]) - rot) <= 2.0 ** -8 * np.abs(rot))
        else:
            back = E4M3FN_VALUES[out[slot]] * 0.02
            # e4m3fn keeps 4 significant bits: relative error <= 2^-4 above 2^-6 * scale
            ref = np.concatenate([latent, rot.astype(np.float64)])
            assert np.all(np.abs(back - ref) <= 2.0 ** -4 * np.abs(ref) + 2.0 ** -10 * 0.02)


def test_insert_flags_bad_slots_and_positions():
    rng = np.random.default_rng(11)
    c = _case(rng, T=3)
    c["slot_mapping"] = np.array([2, 99, 5])
    c["positions"] = np.array([0, 1, 40])
    cache = np.zeros((16, 576), np.uint8)
    _, out, status = qcat_cache_insert_reference(cache=cache, kv_dtype="fp8_e4m3fn", kv_scale=1.0, neox=True, **c)
    assert status == 3
    assert out[2].any() and not out[5].any()
