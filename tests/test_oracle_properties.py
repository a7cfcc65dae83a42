"""The oracle's invariants as hypothesis properties over random small shapes
(CPU only): physical page permutation, one-row context, constant values,
causal masking = truncated context, split + log-sum-exp merge = unsplit."""

import numpy as np
from hypothesis import given, settings, strategies as st

import oracle
from mla_synth import make_case

SETTINGS = settings(max_examples=25, deadline=None, derandomize=True)

shapes = st.fixed_dictionaries({
    "batch": st.integers(1, 3),
    "seqlen_qo": st.integers(1, 4),
    "num_heads": st.integers(1, 5),
    "page_size": st.sampled_from([1, 2, 3, 16]),
    "kv_dtype": st.sampled_from(["bf16", "fp8_e4m3fn"]),
    "seed": st.integers(0, 10_000),
    "extra": st.lists(st.integers(0, 40), min_size=3, max_size=3),
})


def _case(d, causal=False, spare_pages=0):
    S = d["seqlen_qo"]
    ctx = [S + e for e in d["extra"][:d["batch"]]]
    pages = sum(-(-c // d["page_size"]) for c in ctx) + spare_pages
    return make_case(batch=d["batch"], seqlen_qo=S, num_heads=d["num_heads"], ctx=ctx, page_size=d["page_size"],
                     kv_dtype=d["kv_dtype"], causal=causal, seed=d["seed"], pool_pages=pages)


def _run(c, **kw):
    return oracle.mla_decode_reference(c.q_bits, c.cache_raw, c.kv_dtype, c.kv_scale, c.kv_indptr,
                                       c.kv_page_indices, c.context_lens, c.page_size, c.softmax_scale, c.causal,
                                       **kw)


@SETTINGS
@given(shapes, st.booleans(), st.integers(0, 2 ** 31))
def test_page_permutation_changes_nothing(d, causal, perm_seed):
    c = _case(d, causal, spare_pages=3)
    out, lse = _run(c)
    P = c.page_size
    n_pages = c.num_slots // P
    pi = np.random.default_rng(perm_seed).permutation(n_pages)
    moved = np.empty_like(c.cache_raw)
    for p in range(n_pages):
        moved[pi[p] * P:(pi[p] + 1) * P] = c.cache_raw[p * P:(p + 1) * P]
    c.cache_raw = moved
    c.kv_page_indices = pi[c.kv_page_indices].astype(np.int32)
    out2, lse2 = _run(c)
    assert np.array_equal(out, out2) and np.array_equal(lse, lse2)


@SETTINGS
@given(shapes)
def test_one_row_context_returns_that_rows_value(d):
    d = dict(d, seqlen_qo=1, extra=[0, 0, 0])
    c = _case(d)
    out, _ = _run(c)
    for b in range(c.batch):
        slot = oracle.row_slots(c.kv_indptr, c.kv_page_indices, b, 1, c.page_size)
        v = oracle.dequantize_rows(c.cache_raw[slot], c.kv_dtype, c.kv_scale)[0, :512]
        np.testing.assert_allclose(out[b], np.broadcast_to(v, out[b].shape), rtol=1e-15, atol=0)


@SETTINGS
@given(shapes, st.floats(-3.0, 3.0))
def test_constant_values_return_the_constant(d, value):
    c = _case(d)
    if c.kv_dtype == "bf16":
        bits = np.float32(value).view(np.uint32) >> 16
        c.cache_raw[:, :512] = bits
        expect = float((np.uint32(bits) << 16).view(np.float32))
    else:
        code = int(oracle.f32_to_e4m3fn(np.float32(value / c.kv_scale)))
        c.cache_raw[:, :512] = code
        expect = oracle.E4M3FN_VALUES[code] * c.kv_scale
    out, _ = _run(c)
    np.testing.assert_allclose(out, expect, rtol=1e-12, atol=1e-300)


@SETTINGS
@given(shapes)
def test_causal_token_equals_its_truncated_context(d):
    c = _case(d, causal=True)
    out, lse = _run(c)
    S = c.seqlen_qo
    for i in range(S):
        ctx_i = c.context_lens - S + 1 + i
        o1, l1 = oracle.mla_decode_reference(c.q_bits[:, i:i + 1], c.cache_raw, c.kv_dtype, c.kv_scale, c.kv_indptr,
                                             c.kv_page_indices, ctx_i, c.page_size, c.softmax_scale, False)
        assert np.array_equal(o1[:, 0], out[:, i]) and np.array_equal(l1[:, 0], lse[:, i])


@SETTINGS
@given(shapes, st.lists(st.integers(1, 60), min_size=1, max_size=4))
def test_split_merge_equals_unsplit(d, cut_points):
    d = dict(d, batch=1, seqlen_qo=1, extra=[60, 0, 0])
    c = _case(d)
    n = int(c.context_lens[0])
    slots = oracle.row_slots(c.kv_indptr, c.kv_page_indices, 0, n, c.page_size)
    k = oracle.dequantize_rows(c.cache_raw[slots], c.kv_dtype, c.kv_scale)
    q = oracle.bf16_bits_to_f64(c.q_bits[0, 0])
    full_o, full_l = oracle.attend(q, k, k[:, :512], c.softmax_scale)
    cuts = [0] + sorted(min(p, n) for p in cut_points) + [n]
    parts = [oracle.attend(q, k[a:b], k[a:b, :512], c.softmax_scale) for a, b in zip(cuts, cuts[1:])]
    mo, ml = oracle.merge_partials([p[0] for p in parts], [p[1] for p in parts])
    np.testing.assert_allclose(mo, full_o, rtol=0, atol=1e-12)
    np.testing.assert_allclose(ml, full_l, rtol=0, atol=1e-12)
