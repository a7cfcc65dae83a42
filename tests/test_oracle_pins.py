"""Pins of the fp64 oracle to things other than itself (CPU only).

The pages print no worked example with values, so the oracle is pinned by brute
force on tiny inputs (pure Python and 50-digit mpmath), by torch's float64 SDPA,
by closed forms and by invariants of attention. ``test_planted_mistakes`` plants
plausible slips in a copy of the oracle and checks that these pins catch them.
"""

import math

import numpy as np
import pytest
import torch

import oracle
from oracle import attention as oatt
from mla_synth import make_case
from _brute import brute_decode, e4m3fn_value, bf16_value


def run(case, **kw):
    return oracle.mla_decode_reference(case.q_bits, case.cache_raw, case.kv_dtype, case.kv_scale,
                                       case.kv_indptr, case.kv_page_indices, case.context_lens,
                                       case.page_size, case.softmax_scale, case.causal, **kw)


def tiny(seed, kv_dtype="bf16", causal=False, S=1, H=3, ctx=(5, 9), P=2, pool_pages=None):
    return make_case(batch=len(ctx), seqlen_qo=S, num_heads=H, ctx=list(ctx), page_size=P,
                     kv_dtype=kv_dtype, causal=causal, seed=seed, pool_pages=pool_pages)


# ---------------------------------------------------------------- element formats

def test_fp8_table_matches_torch_on_all_256_bytes():
    raw = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = raw.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = oracle.decode_e4m3fn(np.arange(256))
    assert np.array_equal(np.isnan(ref), np.isnan(got))
    ok = ~np.isnan(ref)
    assert np.array_equal(ref[ok], got[ok])
    assert np.isnan(got[0x7F]) and np.isnan(got[0xFF]) and got[0x7E] == 448.0
    assert got[1] == 2.0 ** -9  # smallest subnormal


def test_fp8_table_matches_bit_formula_loop():
    for b in range(256):
        a, c = oracle.E4M3FN_VALUES[b], e4m3fn_value(b)
        assert (math.isnan(a) and math.isnan(c)) or a == c


def test_bf16_widening_is_exact():
    bits = np.random.default_rng(0).integers(0, 1 << 16, size=4096, dtype=np.uint16)
    bits = bits[((bits >> 7) & 0xFF) != 0xFF]  # finite only
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(oracle.bf16_bits_to_f64(bits), ref)
    assert all(bf16_value(int(x)) == y for x, y in zip(bits[:64], ref[:64]))


# ---------------------------------------------------------------- brute force

BRUTE_CASES = [
    dict(seed=11, kv_dtype="bf16", causal=False, S=1, H=3, ctx=(5, 9), P=2),
    dict(seed=12, kv_dtype="fp8_e4m3fn", causal=False, S=2, H=2, ctx=(3, 7, 4), P=3),
    dict(seed=13, kv_dtype="fp8_e4m3fn", causal=True, S=4, H=2, ctx=(4, 9), P=1),
    dict(seed=14, kv_dtype="bf16", causal=True, S=3, H=4, ctx=(8, 3), P=2, pool_pages=11),
]


@pytest.mark.parametrize("spec", BRUTE_CASES)
def test_oracle_matches_pure_python_brute_force(spec):
    case = tiny(**spec)
    out, lse = run(case)
    bout, blse = brute_decode(case)
    for (b, s, h), v in bout.items():
        assert np.max(np.abs(out[b, s, h] - np.array(v))) <= 1e-12
        assert abs(lse[b, s, h] - blse[(b, s, h)]) <= 1e-12


def test_oracle_matches_mpmath_brute_force():
    case = tiny(seed=15, kv_dtype="fp8_e4m3fn", causal=True, S=2, H=2, ctx=(4, 6), P=2)
    out, lse = run(case)
    bout, blse = brute_decode(case, use_mpmath=True)
    for (b, s, h), v in bout.items():
        assert np.max(np.abs(out[b, s, h] - np.array([float(x) for x in v]))) <= 1e-13
        assert abs(lse[b, s, h] - float(blse[(b, s, h)])) <= 1e-13


# ---------------------------------------------------------------- library routine

@pytest.mark.parametrize("kv_dtype", ["bf16", "fp8_e4m3fn"])
def test_oracle_matches_torch_float64_sdpa(kv_dtype):
    case = make_case(batch=3, seqlen_qo=1, num_heads=16, ctx=[300, 17, 129], page_size=16,
                     kv_dtype=kv_dtype, seed=21)
    out, lse = run(case)
    for b in range(case.batch):
        ctx = int(case.context_lens[b])
        plist = case.kv_page_indices[case.kv_indptr[b]:case.kv_indptr[b + 1]]
        slots = [int(p) * case.page_size + o for p in plist for o in range(case.page_size)][:ctx]
        raw = torch.from_numpy(case.cache_raw[slots].astype(np.int64))
        if kv_dtype == "bf16":
            k = raw.to(torch.int16).view(torch.bfloat16).to(torch.float64)
        else:
            k = raw.to(torch.uint8).view(torch.float8_e4m3fn).to(torch.float64) * case.kv_scale
        q = torch.from_numpy(case.q_bits[b, 0].view(np.int16)).view(torch.bfloat16).to(torch.float64)
        ref = torch.nn.functional.scaled_dot_product_attention(
            q[None, :, None, :], k[None, None].expand(1, 16, ctx, 576),
            k[None, None, :, :512].expand(1, 16, ctx, 512), scale=case.softmax_scale)[0, :, 0]
        assert np.max(np.abs(out[b, 0] - ref.numpy())) <= 1e-12
        z = case.softmax_scale * (q @ k.T)
        assert np.max(np.abs(lse[b, 0] - torch.logsumexp(z, dim=1).numpy())) <= 1e-12


# ---------------------------------------------------------------- closed forms

def test_single_row_returns_that_rows_value_exactly():
    case = tiny(seed=31, kv_dtype="fp8_e4m3fn", S=1, H=4, ctx=(1, 1), P=1, pool_pages=8)
    out, lse = run(case)
    for b in range(2):
        slot = case.kv_page_indices[case.kv_indptr[b]]
        v = oracle.decode_e4m3fn(case.cache_raw[slot]) * case.kv_scale
        assert np.array_equal(out[b, 0], np.broadcast_to(v[:512], (4, 512)))
        q = oracle.bf16_bits_to_f64(case.q_bits[b, 0])
        np.testing.assert_allclose(lse[b, 0], case.softmax_scale * (q @ v), rtol=0, atol=1e-12)


def test_constant_value_rows_return_the_constant():
    case = tiny(seed=32, S=2, H=3, ctx=(6, 11), P=3)
    const = case.cache_raw[0, :512].copy()
    case.cache_raw[:, :512] = const
    out, _ = run(case)
    np.testing.assert_allclose(out, np.broadcast_to(oracle.bf16_bits_to_f64(const), out.shape),
                               rtol=1e-14, atol=0)


def test_zero_query_returns_mean_of_visible_rows():
    case = tiny(seed=33, kv_dtype="fp8_e4m3fn", causal=True, S=3, H=2, ctx=(7, 5), P=2)
    case.q_bits[:] = 0
    out, lse = run(case)
    for b in range(2):
        ctx = int(case.context_lens[b])
        slots = oracle.row_slots(case.kv_indptr, case.kv_page_indices, b, ctx, case.page_size)
        v = oracle.decode_e4m3fn(case.cache_raw[slots][:, :512]) * case.kv_scale
        for s in range(3):
            n = ctx - 3 + 1 + s
            np.testing.assert_allclose(out[b, s], np.broadcast_to(v[:n].mean(axis=0), (2, 512)),
                                       rtol=0, atol=1e-14)
            np.testing.assert_allclose(lse[b, s], math.log(n), rtol=0, atol=1e-14)


def test_two_rows_weights_are_logistic():
    case = tiny(seed=34, S=1, H=2, ctx=(2,), P=1, pool_pages=4)
    out, _ = run(case)
    slots = oracle.row_slots(case.kv_indptr, case.kv_page_indices, 0, 2, 1)
    k = oracle.bf16_bits_to_f64(case.cache_raw[slots])
    q = oracle.bf16_bits_to_f64(case.q_bits[0, 0])
    z = case.softmax_scale * (q @ k.T)
    w0 = 1.0 / (1.0 + np.exp(z[:, 1] - z[:, 0]))
    expect = w0[:, None] * k[0, :512] + (1 - w0)[:, None] * k[1, :512]
    np.testing.assert_allclose(out[0, 0], expect, rtol=0, atol=1e-14)


# ---------------------------------------------------------------- invariants

def test_permuting_physical_pages_changes_nothing():
    case = tiny(seed=41, kv_dtype="fp8_e4m3fn", causal=True, S=2, H=3, ctx=(9, 4, 7), P=3, pool_pages=9)
    out, lse = run(case)
    P = case.page_size
    pi = np.random.default_rng(5).permutation(case.num_slots // P)
    new_cache = np.empty_like(case.cache_raw)
    for p in range(case.num_slots // P):
        new_cache[pi[p] * P:(pi[p] + 1) * P] = case.cache_raw[p * P:(p + 1) * P]
    case.cache_raw = new_cache
    case.kv_page_indices = pi[case.kv_page_indices].astype(np.int32)
    out2, lse2 = run(case)
    assert np.array_equal(out, out2) and np.array_equal(lse, lse2)


def test_causal_token_equals_truncated_context():
    S = 4
    case = tiny(seed=42, kv_dtype="fp8_e4m3fn", causal=True, S=S, H=2, ctx=(9, 6), P=2)
    out, lse = run(case)
    for i in range(S):
        ctx_i = [int(c) - S + 1 + i for c in case.context_lens]
        sub = make_case(batch=2, seqlen_qo=1, num_heads=2, ctx=ctx_i, page_size=2,
                        kv_dtype="fp8_e4m3fn", seed=42)
        # same pool and pages; only the query token and the context length differ
        o1, l1 = oracle.mla_decode_reference(case.q_bits[:, i:i + 1], case.cache_raw, case.kv_dtype,
                                             case.kv_scale, case.kv_indptr, case.kv_page_indices,
                                             np.array(ctx_i), case.page_size, case.softmax_scale, False)
        assert np.array_equal(o1[:, 0], out[:, i]) and np.array_equal(l1[:, 0], lse[:, i])
        del sub


def test_split_and_lse_merge_equals_unsplit():
    case = make_case(batch=1, seqlen_qo=1, num_heads=8, ctx=[700], page_size=1,
                     kv_dtype="fp8_e4m3fn", seed=43)
    slots = oracle.row_slots(case.kv_indptr, case.kv_page_indices, 0, 700, 1)
    k = oracle.dequantize_rows(case.cache_raw[slots], case.kv_dtype, case.kv_scale)
    q = oracle.bf16_bits_to_f64(case.q_bits[0, 0])
    full_o, full_l = oracle.attend(q, k, k[:, :512], case.softmax_scale)
    for cuts in ([0, 64, 700], [0, 1, 2, 650, 700], [0, 256, 512, 700, 700]):
        parts = [oracle.attend(q, k[a:b], k[a:b, :512], case.softmax_scale) for a, b in zip(cuts, cuts[1:])]
        mo, ml = oracle.merge_partials([p[0] for p in parts], [p[1] for p in parts])
        np.testing.assert_allclose(mo, full_o, rtol=0, atol=1e-12)
        np.testing.assert_allclose(ml, full_l, rtol=0, atol=1e-12)
    # all pieces empty -> zeros and -inf
    eo, el = oracle.merge_partials(np.zeros((2, 3, 512)), np.full((2, 3), -np.inf))
    assert np.all(eo == 0) and np.all(np.isneginf(el))


def test_duplicating_rows_keeps_output_and_adds_log2():
    case = tiny(seed=44, S=1, H=3, ctx=(5,), P=1, pool_pages=10)
    out, lse = run(case)
    dup = tiny(seed=44, S=1, H=3, ctx=(10,), P=1, pool_pages=10)
    dup.q_bits = case.q_bits
    dup.cache_raw = case.cache_raw
    pages = case.kv_page_indices[:5]
    dup.kv_page_indices = np.concatenate([pages, pages]).astype(np.int32)
    out2, lse2 = run(dup)
    np.testing.assert_allclose(out2, out, rtol=0, atol=1e-14)
    np.testing.assert_allclose(lse2, lse + math.log(2.0), rtol=0, atol=1e-13)


def test_permuting_heads_permutes_output():
    case = tiny(seed=45, kv_dtype="fp8_e4m3fn", S=2, H=5, ctx=(6, 3), P=2)
    out, lse = run(case)
    perm = np.array([3, 0, 4, 1, 2])
    case.q_bits = case.q_bits[:, :, perm].copy()
    out2, lse2 = run(case)
    assert np.array_equal(out2, out[:, :, perm]) and np.array_equal(lse2, lse[:, :, perm])


def test_affine_map_of_value_columns_with_rope_only_scores():
    # With the latent half of q zeroed, scores depend only on the 64 rope columns,
    # so an affine map of the 512 value columns passes straight through.
    case = tiny(seed=46, S=1, H=3, ctx=(7, 4), P=1)
    case.q_bits[..., :512] = 0
    out, _ = run(case)
    k = oracle.bf16_bits_to_f64(case.cache_raw)
    k2 = k.copy()
    k2[:, :512] = 2.0 * k[:, :512] + 0.5  # exact in bf16 for these magnitudes? widen via fp32 bits
    bits = torch.from_numpy(k2.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(oracle.bf16_bits_to_f64(bits)[:, 512:], k[:, 512:])
    k2 = oracle.bf16_bits_to_f64(bits)
    case.cache_raw = bits
    out2, _ = run(case)
    # compare against the same affine map applied to the exact (re-rounded) values
    expect = np.zeros_like(out)
    for b in range(2):
        ctx = int(case.context_lens[b])
        slots = oracle.row_slots(case.kv_indptr, case.kv_page_indices, b, ctx, 1)
        q = oracle.bf16_bits_to_f64(case.q_bits[b, 0])
        z = case.softmax_scale * (q @ k[slots].T)
        w = np.exp(z - z.max(axis=1, keepdims=True))
        w /= w.sum(axis=1, keepdims=True)
        expect[b, 0] = w @ k2[slots, :512]
    np.testing.assert_allclose(out2, expect, rtol=0, atol=1e-13)
    np.testing.assert_allclose(out2, 2.0 * out + 0.5, rtol=0, atol=2e-2)  # bf16 re-rounding of 2k+0.5


# ---------------------------------------------------------------- planted mistakes

@pytest.mark.parametrize("mutant", ["slot_offset", "page_stride", "value_is_last_512", "no_scale",
                                    "causal_off_by_one", "fp8_scale_dropped", "lse_log2"])
def test_planted_mistakes_are_caught(monkeypatch, mutant):
    orig_row_slots, orig_attend, orig_deq, orig_vis = oatt.row_slots, oatt.attend, oatt.dequantize_rows, oatt.visible_rows
    if mutant == "slot_offset":
        monkeypatch.setattr(oatt, "row_slots", lambda ip, pi, b, n, P: orig_row_slots(ip, pi, b, n, P) + 1)
    elif mutant == "page_stride":
        def rs(ip, pi, b, n, P):
            r = np.arange(n)
            return np.asarray(pi, np.int64)[ip[b] + r // P] + r % P  # forgot * page_size
        monkeypatch.setattr(oatt, "row_slots", rs)
    elif mutant == "value_is_last_512":
        def att(q, k, v, sc):
            return orig_attend(q, k, k[:, 64:], sc)
        monkeypatch.setattr(oatt, "attend", att)
    elif mutant == "no_scale":
        monkeypatch.setattr(oatt, "attend", lambda q, k, v, sc: orig_attend(q, k, v, 1.0))
    elif mutant == "causal_off_by_one":
        monkeypatch.setattr(oatt, "visible_rows", lambda ctx, S, s, c: orig_vis(ctx, S, s, c) - (1 if c else 0))
    elif mutant == "fp8_scale_dropped":
        monkeypatch.setattr(oatt, "dequantize_rows", lambda raw, dt, sc: orig_deq(raw, dt, 1.0))
    elif mutant == "lse_log2":
        def att(q, k, v, sc):
            o, l = orig_attend(q, k, v, sc)
            return o, l / math.log(2.0)
        monkeypatch.setattr(oatt, "attend", att)
    caught = False
    for spec in BRUTE_CASES:
        case = tiny(**spec)
        try:
            out, lse = run(case)
        except (IndexError, ValueError):
            caught = True
            break
        bout, blse = brute_decode(case)
        for (b, s, h), v in bout.items():
            if not (np.max(np.abs(out[b, s, h] - np.array(v))) <= 1e-12 and abs(lse[b, s, h] - blse[(b, s, h)]) <= 1e-12):
                caught = True
                break
        if caught:
            break
    assert caught, f"planted mistake {mutant} was not caught by the brute-force pin"
