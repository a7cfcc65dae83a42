"""Pins of the cached-prefix expansion oracle (gather_kv_b_proj), CPU only.

What fixes the answer independently of the oracle's own code: selection
matrices turn the projection into a known permutation of latent columns (read
through a gather written differently, page list by page list), a pure-Python
brute force on tiny inputs, head independence, page-permutation invariance, the
fp8 scale as an exact power-of-two factor, and the rope part against torch's own
float8 and bfloat16 casts."""

import numpy as np
import pytest
import torch

from mla_synth import make_kvb_case
from oracle.fp8 import E4M3FN_VALUES, bf16_bits_to_f64
from oracle.kv_b_proj import gather_kv_b_proj_reference, output_rows


def _bits(x):
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _latent_by_pages(c):
    """Every sequence's cached rows, gathered page by page (not row by row)."""
    P = c.page_size
    seqs = []
    for b in range(c.batch):
        pages = c.kv_page_indices[c.kv_indptr[b]:c.kv_indptr[b + 1]]
        rows = np.concatenate([c.cache_raw[p * P:(p + 1) * P] for p in pages]) if len(pages) else c.cache_raw[:0]
        seqs.append(rows[:c.context_lens[b]])
    return seqs


def _deq(raw, c):
    return bf16_bits_to_f64(raw) if c.kv_dtype == "bf16" else E4M3FN_VALUES[raw] * c.kv_scale


def _ref(c, w_bits=None, **kw):
    return gather_kv_b_proj_reference(c.cache_raw, c.kv_dtype, c.kv_scale, c.kv_indptr, c.kv_page_indices,
                                      c.cu_ctx, c.page_size, c.w_bits if w_bits is None else w_bits, **kw)


@pytest.mark.parametrize("kv_dtype,P", [("bf16", 4), ("fp8_e4m3fn", 1), ("fp8_e4m3fn", 16)])
def test_selection_weights_give_latent_columns(kv_dtype, P):
    c = make_kvb_case(batch=3, num_heads=3, ctx=[5, 0, 37], page_size=P, kv_dtype=kv_dtype, seed=1, pool_pages=64)
    H = c.num_heads
    sel = np.array([[(3 * n + 37 * h) % 512 for n in range(256)] for h in range(H)])  # distinct per head
    w = np.zeros((H, 256, 512), np.float32)
    for h in range(H):
        w[h, np.arange(256), sel[h]] = 1.0
    k, k_rope, v = _ref(c, w_bits=_bits(w))
    seqs = _latent_by_pages(c)
    assert k.shape[0] == sum(len(s) for s in seqs) == c.cu_ctx[-1]
    for b, r, row in output_rows(c.cu_ctx):
        lat = _deq(seqs[b][r], c)
        for h in range(H):
            assert np.array_equal(k[row, h], lat[sel[h, :128]])
            assert np.array_equal(v[row, h], lat[sel[h, 128:]])


def test_brute_force_tiny():
    c = make_kvb_case(batch=2, num_heads=2, ctx=[2, 3], page_size=2, kv_dtype="fp8_e4m3fn", seed=2, pool_pages=8)
    k, _, v = _ref(c)
    seqs = _latent_by_pages(c)
    w = bf16_bits_to_f64(c.w_bits)
    for b, r, row in output_rows(c.cu_ctx):
        lat = [float(E4M3FN_VALUES[x]) * c.kv_scale for x in seqs[b][r][:512]]
        for h in range(2):
            for n in (0, 5, 127, 128, 200, 255):
                acc = 0.0
                for j in range(512):
                    acc += float(w[h, n, j]) * lat[j]
                got = k[row, h, n] if n < 128 else v[row, h, n - 128]
                assert abs(got - acc) <= 1e-12 * (1 + abs(acc))


def test_heads_are_independent():
    c = make_kvb_case(batch=2, num_heads=4, ctx=[10, 20], page_size=1, kv_dtype="bf16", seed=3)
    k0, _, v0 = _ref(c)
    w = c.w_bits.copy()
    w[2] = _bits(np.random.default_rng(4).standard_normal((256, 512)))
    k1, _, v1 = _ref(c, w_bits=w)
    others = [0, 1, 3]
    assert np.array_equal(k0[:, others], k1[:, others]) and np.array_equal(v0[:, others], v1[:, others])
    assert not np.allclose(k0[:, 2], k1[:, 2]) and not np.allclose(v0[:, 2], v1[:, 2])


def test_page_permutation_invariance():
    c = make_kvb_case(batch=3, num_heads=2, ctx=[17, 1, 40], page_size=8, kv_dtype="fp8_e4m3fn", seed=5, pool_pages=20)
    k0, r0, v0 = _ref(c)
    perm = np.random.default_rng(6).permutation(20)  # page p moves to perm[p]
    cache = np.empty_like(c.cache_raw)
    for p in range(20):
        cache[perm[p] * 8:(perm[p] + 1) * 8] = c.cache_raw[p * 8:(p + 1) * 8]
    k1, r1, v1 = gather_kv_b_proj_reference(cache, c.kv_dtype, c.kv_scale, c.kv_indptr, perm[c.kv_page_indices],
                                            c.cu_ctx, 8, c.w_bits)
    assert np.array_equal(k0, k1) and np.array_equal(v0, v1) and np.array_equal(r0, r1)


def test_fp8_scale_is_a_factor():
    c = make_kvb_case(batch=1, num_heads=2, ctx=[9], page_size=1, kv_dtype="fp8_e4m3fn", seed=7)
    k1, _, v1 = gather_kv_b_proj_reference(c.cache_raw, c.kv_dtype, 1.0, c.kv_indptr, c.kv_page_indices, c.cu_ctx,
                                           1, c.w_bits)
    k4, _, v4 = gather_kv_b_proj_reference(c.cache_raw, c.kv_dtype, 0.25, c.kv_indptr, c.kv_page_indices, c.cu_ctx,
                                           1, c.w_bits)
    assert np.array_equal(k4, 0.25 * k1) and np.array_equal(v4, 0.25 * v1)


@pytest.mark.parametrize("kv_dtype", ["bf16", "fp8_e4m3fn"])
def test_rope_part_against_torch_casts(kv_dtype):
    c = make_kvb_case(batch=2, num_heads=3, ctx=[7, 30], page_size=4, kv_dtype=kv_dtype, seed=8, pool_pages=16)
    _, k_rope, _ = _ref(c)
    seqs = _latent_by_pages(c)
    for b, r, row in output_rows(c.cu_ctx):
        raw = seqs[b][r][512:]
        if kv_dtype == "bf16":
            want = raw
        else:
            f = torch.from_numpy(raw.copy()).view(torch.float8_e4m3fn).to(torch.float32) * torch.tensor(
                c.kv_scale, dtype=torch.float32)
            want = f.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
        for h in range(3):
            assert np.array_equal(k_rope[row, h], want)


def test_row_subset_matches_full_and_rejects_bad_rows():
    c = make_kvb_case(batch=3, num_heads=2, ctx=[4, 0, 6], page_size=2, kv_dtype="bf16", seed=9, pool_pages=8)
    k, kr, v = _ref(c)
    pick = [(2, 5), (0, 0), (2, 0)]
    ks, krs, vs = _ref(c, rows=pick)
    idx = [int(c.cu_ctx[b]) + r for b, r in pick]
    assert np.array_equal(ks, k[idx]) and np.array_equal(krs, kr[idx]) and np.array_equal(vs, v[idx])
    with pytest.raises(ValueError):
        _ref(c, rows=[(1, 0)])  # sequence 1 has no cached rows
    empty = make_kvb_case(batch=2, num_heads=2, ctx=[0, 0], page_size=1, kv_dtype="bf16", seed=10, pool_pages=4)
    k, kr, v = _ref(empty)
    assert k.shape == (0, 2, 128) and kr.shape == (0, 2, 64) and v.shape == (0, 2, 128)
