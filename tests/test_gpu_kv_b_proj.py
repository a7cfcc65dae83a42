"""Parity of the cached-prefix expansion (mla_gather_kv_b_proj, through the C ABI)
with the fp64 oracle on MI355X.

K-nope and V: |gpu - oracle| <= 1e-2 + 1e-2 |oracle| element by element (bf16
output rounding is 2^-9 relative; the float32 accumulation of 512 products adds
far less). K's rope part: bit for bit. Output rows that belong to no sequence,
and rows the status word says were skipped, must keep their prior contents."""

import numpy as np
import pytest
import torch

import oracle
from mla_synth import KVB_WORKLOADS, make_kvb_case

pytestmark = pytest.mark.gpu

ATOL, RTOL = 1e-2, 1e-2
POISON = -21555  # 0xabcd as int16


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    import mla_paged_latent_02_amd  # noqa: F401  (fails loudly if the library is missing)
    yield


def _dev(a):
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).to("cuda")


def _bf16(bits):
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def run(c, *, extra_rows=0, max_context_len=None, kv_indptr=None, kv_page_indices=None, cu_ctx=None,
        num_out_rows=None):
    import mla_paged_latent_02_amd as mla
    cu = c.cu_ctx if cu_ctx is None else cu_ctx
    rows = int(c.cu_ctx[-1]) + extra_rows if num_out_rows is None else num_out_rows
    H = c.num_heads
    k = torch.full((max(rows, 1), H, 192), POISON, dtype=torch.int16, device="cuda")
    v = torch.full((max(rows, 1), H, 128), POISON, dtype=torch.int16, device="cuda")
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    p = mla.make_kv_b_proj_params(batch=c.batch, num_heads=H, page_size=c.page_size, kv_dtype=c.kv_dtype,
                                  kv_scale=c.kv_scale,
                                  max_context_len=c.max_context_len if max_context_len is None else max_context_len,
                                  num_slots=c.num_slots, num_out_rows=rows)
    mla.gather_kv_b_proj(p, _dev(c.cache_raw), _dev(c.kv_indptr if kv_indptr is None else kv_indptr),
                         _dev(c.kv_page_indices if kv_page_indices is None else kv_page_indices), _dev(cu),
                         _dev(c.w_bits), k, v, status)
    torch.cuda.synchronize()
    return (k.cpu().numpy().view(np.uint16)[:rows], v.cpu().numpy().view(np.uint16)[:rows], int(status.item()))


def compare(c, k, v, rows=None, label=""):
    rk, rrope, rv = oracle.gather_kv_b_proj_reference(c.cache_raw, c.kv_dtype, c.kv_scale, c.kv_indptr,
                                                      c.kv_page_indices, c.cu_ctx, c.page_size, c.w_bits, rows=rows)
    idx = (np.arange(int(c.cu_ctx[-1])) if rows is None else np.array([int(c.cu_ctx[b]) + r for b, r in rows],
                                                                         dtype=np.int64))
    gk, gv = _bf16(k[idx, :, :128]), _bf16(v[idx])
    for name, g, r in (("k_nope", gk, rk), ("v", gv, rv)):
        err = np.abs(g - r)
        bad = np.argwhere(~(err <= ATOL + RTOL * np.abs(r)))
        assert bad.size == 0, f"{label} {name}: {len(bad)} elements off, first {bad[:3]}, max err {err.max()}"
    assert np.array_equal(k[idx, :, 128:], rrope), f"{label}: rope part differs"


def untouched(a, rows):
    return np.all(a[rows].view(np.int16) == POISON)


SMALL = [  # (batch, heads, ctx list, page size, kv dtype)
    (1, 1, [1], 1, "bf16"), (1, 12, [128], 1, "fp8_e4m3fn"), (1, 12, [129], 1, "fp8_e4m3fn"),
    (2, 4, [255, 513], 16, "bf16"), (3, 12, [0, 77, 300], 64, "fp8_e4m3fn"), (4, 3, [5, 0, 0, 1000], 7, "bf16"),
    (2, 16, [640, 384], 128, "fp8_e4m3fn"), (1, 12, [4096], 1, "fp8_e4m3fn"), (5, 2, [1, 2, 3, 127, 128], 1, "bf16"),
]


@pytest.mark.parametrize("B,H,ctx,P,kv", SMALL)
def test_small_cases_full_output(B, H, ctx, P, kv):
    pool = sum(-(-x // P) for x in ctx) + 3
    c = make_kvb_case(batch=B, num_heads=H, ctx=ctx, page_size=P, kv_dtype=kv, seed=100 + B + H, pool_pages=pool)
    k, v, status = run(c, extra_rows=5)
    assert status == 0
    compare(c, k, v, label=f"B{B} H{H} ctx{ctx} P{P} {kv}")
    n = int(c.cu_ctx[-1])
    assert untouched(k, slice(n, n + 5)) and untouched(v, slice(n, n + 5))


@pytest.mark.parametrize("name", ["kvb_ragged_b5_h12_fp8_p16", "kvb_ragged_b3_h8_bf16_p64"])
def test_ragged_workloads(name):
    c = make_kvb_case(name=name, **KVB_WORKLOADS[name])
    k, v, status = run(c)
    assert status == 0
    compare(c, k, v, label=name)


def test_many_empty_programs_per_workgroup():
    # One long sequence sizes the chunk axis (300 chunks of 256 rows) for 64 sequences of one head:
    # 19200 programs, about 75 per persistent workgroup, most of them past their sequence's end, so
    # each workgroup's walk crosses its 64-program windows of sequence bounds while skipping.
    rng = np.random.default_rng(2024)
    ctx = [int(x) for x in rng.integers(1, 3000, size=64)]
    ctx[37] = 300 * 256
    pool = sum(-(-x // 16) for x in ctx) + 8
    c = make_kvb_case(batch=64, num_heads=1, ctx=ctx, page_size=16, kv_dtype="fp8_e4m3fn", seed=77, pool_pages=pool)
    k, v, status = run(c)
    assert status == 0
    rows = [(b, r) for b in (0, 1, 36, 38, 63) for r in range(ctx[b])]
    rows += [(37, int(r)) for r in rng.choice(ctx[37], size=1500, replace=False)]
    rows += [(37, r) for r in (0, 255, 256, ctx[37] - 1)]
    compare(c, k, v, rows=rows, label="many empty programs")


@pytest.mark.parametrize("name", ["kvb_b1_h12_ctx109440_fp8", "kvb_b1_h12_ctx65536_fp8", "kvb_b1_h12_ctx32000_fp8",
                                  "kvb_b1_h12_ctx4096_fp8"])
def test_full_size_every_row(name):
    # every cached row of the pages' context lengths, against the fp64 oracle (one dgemm per call)
    c = make_kvb_case(name=name, **KVB_WORKLOADS[name])
    k, v, status = run(c)
    assert status == 0
    compare(c, k, v, label=name)
    # every row of the full-size output was written: none still holds the poison pattern
    assert not np.any(np.all(k.view(np.int16) == POISON, axis=2))
    assert not np.any(np.all(v.view(np.int16) == POISON, axis=2))


def test_repeated_calls_are_bitwise_equal():
    c = make_kvb_case(name="r", **KVB_WORKLOADS["kvb_ragged_b5_h12_fp8_p16"])
    k1, v1, _ = run(c)
    k2, v2, _ = run(c)
    assert np.array_equal(k1, k2) and np.array_equal(v1, v2)


def test_status_too_few_pages_and_bad_slot():
    c = make_kvb_case(batch=3, num_heads=2, ctx=[40, 40, 40], page_size=16, kv_dtype="fp8_e4m3fn", seed=9,
                      pool_pages=12)
    # sequence 1 loses its last page (rows 32..39); sequence 2's second page id points past the cache
    indptr = c.kv_indptr.copy()
    pages = c.kv_page_indices.copy()
    pages[int(indptr[2]) + 1] = 10 ** 6
    short = np.concatenate([pages[:indptr[2] - 1], pages[indptr[2]:]]).astype(np.int32)
    indptr_short = indptr.copy()
    indptr_short[2:] -= 1
    k, v, status = run(c, kv_indptr=indptr_short, kv_page_indices=short)
    assert status == 1 | 2
    zero_rows = [40 + r for r in range(32, 40)] + [80 + r for r in range(16, 32)]
    assert np.all(k[zero_rows] == 0) and np.all(v[zero_rows] == 0)
    good = [(0, r) for r in range(40)] + [(1, r) for r in range(32)] + [(2, r) for r in range(16)] + \
           [(2, r) for r in range(32, 40)]
    ck = make_kvb_case(batch=3, num_heads=2, ctx=[40, 40, 40], page_size=16, kv_dtype="fp8_e4m3fn", seed=9,
                       pool_pages=12)
    compare(ck, k, v, rows=good, label="status case, good rows")


def test_status_ctx_too_long_and_rows_out_of_range():
    c = make_kvb_case(batch=2, num_heads=3, ctx=[300, 100], page_size=1, kv_dtype="bf16", seed=11)
    k, v, status = run(c, max_context_len=200)  # rows 200.. of sequence 0 are not written
    assert status == 8
    compare(c, k, v, rows=[(0, r) for r in range(200)] + [(1, r) for r in range(100)], label="ctx too long")
    assert untouched(k, slice(200, 300)) and untouched(v, slice(200, 300))
    cu = c.cu_ctx.copy()
    k, v, status = run(c, cu_ctx=cu, num_out_rows=350)  # sequence 1 (rows 300..399) does not fit
    assert status == 4
    compare(c, k, v, rows=[(0, r) for r in range(300)], label="rows out of range")
    assert untouched(k, slice(300, 350)) and untouched(v, slice(300, 350))
