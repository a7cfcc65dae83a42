"""Parity of the HIP path (through the C ABI) with the fp64 oracle, on MI355X.

Tolerance (from the accuracy target of this path: bf16 output, fp32 accumulate):
|gpu - oracle| <= 1e-2 + 1e-2 |oracle| elementwise, for the output and the lse.
Plan metadata must match the reference planner bit for bit. Output and
workspace buffers are poisoned with NaN before every call, so any element the
kernels fail to write fails the comparison.
"""

import math

import numpy as np
import pytest
import torch

import oracle
from mla_synth import WORKLOADS, make_case

pytestmark = pytest.mark.gpu

ATOL = 1e-2
RTOL = 1e-2


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    import mla_paged_latent_02_amd  # noqa: F401  (fails loudly if the library is missing)
    yield


def upload(case):
    from mla_paged_latent_02_amd.device import DeviceInputs
    return DeviceInputs.from_host(
        q_bits=case.q_bits, cache_raw=case.cache_raw, kv_indptr=case.kv_indptr,
        kv_page_indices=case.kv_page_indices, context_lens=case.context_lens, batch=case.batch,
        seqlen_qo=case.seqlen_qo, num_heads=case.num_heads, page_size=case.page_size,
        max_context_len=case.max_context_len, causal=case.causal, kv_dtype=case.kv_dtype,
        softmax_scale=case.softmax_scale, kv_scale=case.kv_scale, num_slots=case.num_slots,
        q_dtype=case.q_dtype, q_scale=case.q_scale)


def run(case, options=None, inputs=None, num_cu=0):
    from mla_paged_latent_02_amd.device import Decoder
    inp = inputs or upload(case)
    dec = Decoder(inp, options, num_cu=num_cu, poison=True)
    out, lse = dec()
    torch.cuda.synchronize()
    return dec, out.float().cpu().numpy(), lse.cpu().numpy()


def reference(case, batches=None):
    return oracle.mla_decode_reference(case.q_bits, case.cache_raw, case.kv_dtype, case.kv_scale, case.kv_indptr,
                                       case.kv_page_indices, case.context_lens, case.page_size,
                                       case.softmax_scale, case.causal, batches=batches, q_scale=case.q_scale)


def assert_close(case, out, lse, batches=None, label=""):
    ref_out, ref_lse = reference(case, batches)
    bs = range(case.batch) if batches is None else batches
    for b in bs:
        err = np.abs(out[b] - ref_out[b])
        bound = ATOL + RTOL * np.abs(ref_out[b])
        bad = ~(err <= bound)
        assert not bad.any(), (f"{label} b={b}: {int(bad.sum())} output elements out of tolerance, "
                               f"max err {np.nanmax(err):.3g}, first at {np.argwhere(bad)[0]}")
        lerr = np.abs(lse[b] - ref_lse[b])
        assert np.all(lerr <= ATOL + RTOL * np.abs(ref_lse[b])), f"{label} b={b}: lse max err {np.nanmax(lerr):.3g}"


def check_plan_arrays(case, dec):
    """Plan fields, per-sequence arrays, status words and the work list equal the oracle planner's,
    bit for bit, after the decode call too: the task counter is back at its start. Returns the
    status bits."""
    import mla_paged_latent_02_amd as mla
    n, base, status = mla.read_plan_arrays(dec.plan, dec.workspace)
    ref = oracle.reference_plan(case.batch, case.seqlen_qo, case.num_heads, case.max_context_len,
                                dec.plan.num_cu, _ref_options(dec.plan), kv_dtype=case.kv_dtype)
    assert mla.plan_to_dict(dec.plan) == {k: ref[k] for k in mla.plan_to_dict(dec.plan)}
    rn, rbase, rbits = oracle.device_plan_arrays(ref, case.seqlen_qo, case.max_context_len, case.page_size,
                                                 case.context_lens, case.kv_indptr)
    items = oracle.work_list(ref, rn, case.context_lens)
    assert n == rn and base == rbase
    assert status == oracle.status_words(ref, rbits, len(items))
    # each item: the (sequence, chunk) of the list, then its sequence's planned fields
    want = [(b, c, int(case.context_lens[b]), int(case.kv_indptr[b]), rn[b], rbase[b], 0, 0) for b, c in items]
    assert mla.read_work_list(dec.plan, dec.workspace) == want
    return status[0]


def _ref_options(plan):
    o = plan.options
    return oracle.PlanOptions(list(o.wg_per_cu), list(o.chunk_min), list(o.chunk_max), o.force_chunk)


def options(force_chunk=0):
    import mla_paged_latent_02_amd as mla
    return mla.make_options(force_chunk=force_chunk)


# (forced chunk length, num_cu) of the grid tests: the default plan on the device's CUs; a
# forced chunk length on the device's CUs; the forced length on three CUs, so that a few
# persistent workgroups each take many tasks from the counter.
SPLITS = [(0, 0), (128, 0), (128, 3)]


# ------------------------------------------------------------------ small cases, full comparison

def test_tiny_workload_default_plan():
    case = make_case(**WORKLOADS["tiny_b2_h16"])
    dec, out, lse = run(case)
    assert check_plan_arrays(case, dec) == 0
    assert dec.plan.max_chunks == 1
    assert_close(case, out, lse, label="tiny")


def test_tiny_workload_forced_split_exercises_the_combine():
    case = make_case(**WORKLOADS["tiny_b2_h16"])
    dec, out, lse = run(case, options(force_chunk=64))
    check_plan_arrays(case, dec)
    n, _, status = __import__("mla_paged_latent_02_amd").read_plan_arrays(dec.plan, dec.workspace)
    assert n == [1, 2] and status[1] == 3
    assert_close(case, out, lse, label="tiny split")


GRID = []
for kv_dtype in ("bf16", "fp8_e4m3fn"):
    for (S, H, causal) in ((1, 12, False), (1, 16, False), (4, 16, True), (2, 32, False), (1, 128, False),
                           (4, 32, True), (3, 5, True), (1, 40, False), (2, 16, True), (1, 20, False),
                           (2, 128, False), (3, 64, True)):
        for P in (1, 16, 64):
            GRID.append((kv_dtype, S, H, causal, P))


@pytest.mark.parametrize("kv_dtype,S,H,causal,P", GRID)
def test_boundary_grid(kv_dtype, S, H, causal, P):
    C = 128
    ctx = [max(S, c) for c in (1, 63, 64, 65, C - 1, C, C + 1, 2 * C + 1)]
    seed = 1000 + GRID.index((kv_dtype, S, H, causal, P))
    case = make_case(batch=len(ctx), seqlen_qo=S, num_heads=H, ctx=ctx, page_size=P, kv_dtype=kv_dtype,
                     causal=causal, seed=seed, pool_pages=sum(-(-c // P) for c in ctx) + 3)
    for force, num_cu in SPLITS:
        dec, out, lse = run(case, options(force_chunk=force), num_cu=num_cu)
        check_plan_arrays(case, dec)
        assert_close(case, out, lse, label=f"grid force={force} num_cu={num_cu}")


# fp8 query x fp8 cache: every tile class, page size and causal shape of the grid above
GRID_Q8 = [(S, H, causal, P) for (kv, S, H, causal, P) in GRID if kv == "fp8_e4m3fn"]


@pytest.mark.parametrize("S,H,causal,P", GRID_Q8)
def test_boundary_grid_fp8_query(S, H, causal, P):
    C = 128
    ctx = [max(S, c) for c in (1, 63, 64, 65, C - 1, C, C + 1, 2 * C + 1)]
    seed = 3000 + GRID_Q8.index((S, H, causal, P))
    case = make_case(batch=len(ctx), seqlen_qo=S, num_heads=H, ctx=ctx, page_size=P, kv_dtype="fp8_e4m3fn",
                     causal=causal, seed=seed, pool_pages=sum(-(-c // P) for c in ctx) + 3, q_dtype="fp8_e4m3fn")
    assert case.q_bits.dtype == np.uint8
    for force, num_cu in SPLITS:
        dec, out, lse = run(case, options(force_chunk=force), num_cu=num_cu)
        check_plan_arrays(case, dec)
        assert_close(case, out, lse, label=f"fp8 query grid force={force} num_cu={num_cu}")


# shapes the grid does not reach: the largest seqlen_qo (8), one head, 256 heads (two head
# groups of 128), odd page sizes, a causal context of exactly S rows, lengths just past a chunk
EDGE = [  # (S, H, causal, P, ctx list)
    (8, 16, True, 3, [8, 9, 200, 1000]),
    (8, 1, True, 5, [8, 77, 640]),
    (1, 1, False, 1, [1, 2, 129, 700]),
    (1, 256, False, 16, [1, 65, 300]),
    (5, 24, True, 2, [5, 6, 127, 513]),
    (2, 200, True, 7, [2, 3, 64, 450]),
]


@pytest.mark.parametrize("q_dtype,kv_dtype", [("bf16", "bf16"), ("bf16", "fp8_e4m3fn"), ("fp8_e4m3fn", "fp8_e4m3fn")])
@pytest.mark.parametrize("S,H,causal,P,ctx", EDGE)
def test_edge_shapes(q_dtype, kv_dtype, S, H, causal, P, ctx):
    seed = 5000 + EDGE.index((S, H, causal, P, ctx)) * 3 + ["bf16", "fp8_e4m3fn"].index(kv_dtype) + \
        (2 if q_dtype != "bf16" else 0)
    case = make_case(batch=len(ctx), seqlen_qo=S, num_heads=H, ctx=ctx, page_size=P, kv_dtype=kv_dtype,
                     causal=causal, seed=seed, pool_pages=sum(-(-c // P) for c in ctx) + 2, q_dtype=q_dtype)
    for force, num_cu in ((0, 0), (64, 0), (64, 2)):
        dec, out, lse = run(case, options(force_chunk=force), num_cu=num_cu)
        check_plan_arrays(case, dec)
        assert_close(case, out, lse, label=f"edge S={S} H={H} P={P} force={force} num_cu={num_cu}")


# merge paths: at most 16 chunks -> one wave per row; more -> column blocks of 16, 128 or 512
# (by how many rows the batch has). Each case forces 64-row chunks so the merge sees many partials.
@pytest.mark.parametrize("batch,heads,ctx,expect_many", [
    (2, 128, [300, 64], False),                 # 5 chunks
    (2, 128, [1000, 64], False),                # 16 chunks, one wave per row
    (2, 12, [1100, 700], True),                 # 18 chunks, 24 rows
    (3, 128, [1100, 700, 64], True),            # 18 chunks, 384 rows
    (9, 128, [1100, 64, 700, 1, 900, 130, 1000, 65, 1024], True),  # 18 chunks, 1152 rows
])
def test_merge_paths(batch, heads, ctx, expect_many):
    case = make_case(batch=batch, seqlen_qo=1, num_heads=heads, ctx=ctx, page_size=16, kv_dtype="fp8_e4m3fn",
                     seed=90 + batch, pool_pages=sum(-(-c // 16) for c in ctx) + 2)
    dec, out, lse = run(case, options(force_chunk=64))
    check_plan_arrays(case, dec)
    assert (dec.plan.max_chunks > 16) == expect_many
    assert_close(case, out, lse, label=f"merge B={batch} H={heads}")


def test_planner_walks_a_batch_of_several_tiles():
    # 600 sequences: the device planner takes them in three tiles of 256, carrying the
    # partial-record scan, the full-chunk count and every length class's rank from tile to
    # tile; lengths (1..320, some exact multiples of the 64-row chunk) put sequences of
    # every class and of one to five chunks in each tile
    rng = np.random.default_rng(91)
    ctx = rng.integers(1, 321, size=600)
    ctx[::37] = 64 * rng.integers(1, 6, size=len(ctx[::37]))
    case = make_case(batch=600, seqlen_qo=1, num_heads=16, ctx=[int(c) for c in ctx], page_size=16,
                     kv_dtype="fp8_e4m3fn", seed=91, pool_pages=int(sum(-(-int(c) // 16) for c in ctx)) + 2)
    dec, out, lse = run(case, options(force_chunk=64))
    check_plan_arrays(case, dec)
    assert_close(case, out, lse, label="600 sequences")


def test_one_cu_runs_the_whole_batch():
    # num_cu = 1: the two persistent workgroups of one CU (64-row tiles at occupancy 2) take
    # all of the batch's 43 tasks (chunks of 64 rows) from the counter in turn
    case = make_case(batch=6, seqlen_qo=4, num_heads=16, ctx=[4, 700, 65, 1300, 17, 400], page_size=16,
                     kv_dtype="fp8_e4m3fn", causal=True, seed=84)
    dec, out, lse = run(case, options(force_chunk=64), num_cu=1)
    assert dec.plan.num_workgroups == 2
    check_plan_arrays(case, dec)
    assert_close(case, out, lse, label="one CU")


def test_counters_are_reset_after_every_call():
    # the last workgroup to finish sets the task counter back, so that call after call (on
    # one plan, on the same workspace) starts from the same state
    import mla_paged_latent_02_amd as mla
    case = make_case(batch=9, seqlen_qo=1, num_heads=128, ctx=[1100, 64, 700, 1, 900, 130, 1000, 65, 1024],
                     page_size=16, kv_dtype="bf16", seed=86)
    dec, out, lse = run(case, options(force_chunk=64), num_cu=5)
    bits = check_plan_arrays(case, dec)
    for _ in range(3):
        o2, l2 = dec()
        torch.cuda.synchronize()
        _, _, status = mla.read_plan_arrays(dec.plan, dec.workspace)
        assert status[0] == bits and status[2:] == [dec.plan.num_workgroups, 0]
        assert np.array_equal(o2.float().cpu().numpy().view(np.uint32), out.view(np.uint32))


def test_stale_plan_is_flagged():
    # planned for one set of lengths, decoded with one sequence a row longer (a decode step
    # without re-planning): the status bit is set and the call computes with the planned
    # lengths, bit for bit what it gave before; re-planned, the bit is clear again
    import mla_paged_latent_02_amd as mla
    case = make_case(batch=3, seqlen_qo=1, num_heads=16, ctx=[300, 128, 500], page_size=16, kv_dtype="bf16",
                     seed=85, pool_pages=64)
    dec, out, lse = run(case, options(force_chunk=128))
    assert check_plan_arrays(case, dec) == 0
    inp = dec.inputs
    inp.context_lens[0] += 1  # 301 rows: its 19 pages of 16 hold them
    dec.out.fill_(float("nan"))
    out2, _ = dec()
    torch.cuda.synchronize()
    assert mla.read_plan_arrays(dec.plan, dec.workspace)[2][0] == mla.DEV_STALE_PLAN
    assert np.array_equal(out2.float().cpu().numpy().view(np.uint32), out.view(np.uint32))
    dec.plan = mla.decode_plan(inp.params, inp.context_lens, inp.kv_indptr, dec.workspace, options(force_chunk=128))
    dec()
    torch.cuda.synchronize()
    assert mla.read_plan_arrays(dec.plan, dec.workspace)[2][0] == 0


def test_run_to_run_bitwise_determinism():
    case = make_case(batch=3, seqlen_qo=4, num_heads=16, ctx=[700, 5, 1300], page_size=16, kv_dtype="fp8_e4m3fn",
                     causal=True, seed=77)
    inp = upload(case)
    _, o1, l1 = run(case, options(force_chunk=256), inputs=inp)
    _, o2, l2 = run(case, options(force_chunk=256), inputs=inp)
    assert np.array_equal(o1.view(np.uint32), o2.view(np.uint32))
    assert np.array_equal(l1.view(np.uint32), l2.view(np.uint32))


def test_repeated_calls_on_one_workspace():
    # one plan and workspace, three decode + combine calls: identical bits every time
    from mla_paged_latent_02_amd.device import Decoder
    case = make_case(batch=5, seqlen_qo=2, num_heads=32, ctx=[900, 2, 640, 1025, 333], page_size=16,
                     kv_dtype="bf16", causal=True, seed=81)
    dec = Decoder(upload(case), options(force_chunk=256), poison=True)
    first = None
    for _ in range(3):
        dec.out.fill_(float("nan"))
        dec.lse.fill_(float("nan"))
        out, lse = dec()
        torch.cuda.synchronize()
        o, l = out.float().cpu().numpy(), lse.cpu().numpy()
        if first is None:
            first = (o, l)
            assert_close(case, o, l, label="repeated calls")
        else:
            assert np.array_equal(o.view(np.uint32), first[0].view(np.uint32))
            assert np.array_equal(l.view(np.uint32), first[1].view(np.uint32))


def test_invalid_sequences_get_nan_rows_and_status_bits():
    import mla_paged_latent_02_amd as mla
    case = make_case(batch=4, seqlen_qo=2, num_heads=16, ctx=[40, 1, 90, 33], page_size=16, kv_dtype="bf16",
                     seed=78, max_context_len=80)
    dec, out, lse = run(case, options(force_chunk=64))
    check_plan_arrays(case, dec)
    n, _, status = mla.read_plan_arrays(dec.plan, dec.workspace)
    assert status[0] == (mla.DEV_CTX_TOO_SHORT | mla.DEV_CTX_TOO_LONG)
    assert n[1] == 0 and n[2] == 0
    assert np.isnan(out[1]).all() and np.isnan(out[2]).all()
    assert np.isnan(lse[1]).all() and np.isnan(lse[2]).all()
    assert_close(case, out, lse, batches=[0, 3], label="valid rows next to invalid ones")


def test_short_page_list_and_bad_page_ids_are_flagged_not_read():
    import mla_paged_latent_02_amd as mla
    case = make_case(batch=3, seqlen_qo=1, num_heads=16, ctx=[50, 70, 20], page_size=16, kv_dtype="fp8_e4m3fn",
                     seed=79)
    # sequence 1: a page id past the pool (the kernel must clamp it and raise a flag)
    good = case.kv_page_indices.copy()
    case.kv_page_indices[case.kv_indptr[1]] = case.num_slots // 16 + 5
    dec, out, lse = run(case)
    _, _, status = mla.read_plan_arrays(dec.plan, dec.workspace)
    assert status[0] & mla.DEV_PAGE_OUT_OF_RANGE
    case.kv_page_indices = good
    assert_close(case, out, lse, batches=[0, 2], label="bad page id in another sequence")
    # sequence 2: a page list one page short of its context length
    case2 = make_case(batch=2, seqlen_qo=1, num_heads=16, ctx=[50, 40], page_size=16, kv_dtype="fp8_e4m3fn", seed=80)
    case2.kv_indptr = case2.kv_indptr.copy()
    case2.kv_indptr[2] -= 1
    dec, out, lse = run(case2)
    n, _, status = mla.read_plan_arrays(dec.plan, dec.workspace)
    assert status[0] == mla.DEV_TOO_FEW_PAGES and n[1] == 0 and np.isnan(out[1]).all()
    assert_close(case2, out, lse, batches=[0], label="short page list next door")


@pytest.mark.gpu
@pytest.mark.parametrize("kv_dtype,heads", [("bf16", 128), ("fp8_e4m3fn", 32)])
def test_page_id_bounds_at_one_row_per_page(kv_dtype, heads):
    # one row per page on ring-gather kernels (128-row bf16, 32-row fp8): the pool's last slot is a
    # valid page and is read; one past it and -1 are flagged, clamped to page 0, and leave the
    # other sequence exact
    import mla_paged_latent_02_amd as mla
    case = make_case(batch=2, seqlen_qo=1, num_heads=heads, ctx=[90, 70], page_size=1, kv_dtype=kv_dtype,
                     seed=81)
    case.kv_page_indices[case.kv_indptr[0] + 5] = case.num_slots - 1
    dec, out, lse = run(case)
    _, _, status = mla.read_plan_arrays(dec.plan, dec.workspace)
    assert not status[0] & mla.DEV_PAGE_OUT_OF_RANGE
    assert_close(case, out, lse, label="last slot of the pool")
    good = case.kv_page_indices.copy()
    for bad in (case.num_slots, -1):
        case.kv_page_indices = good.copy()
        case.kv_page_indices[case.kv_indptr[1] + 3] = bad
        dec, out, lse = run(case)
        _, _, status = mla.read_plan_arrays(dec.plan, dec.workspace)
        assert status[0] & mla.DEV_PAGE_OUT_OF_RANGE, bad
        case.kv_page_indices = good
        assert_close(case, out, lse, batches=[0], label=f"page id {bad} in the other sequence")


# ------------------------------------------------------------------ full-size workloads, every sequence
# The oracle computes each sequence exactly (numpy fp64 on the host cores): every output row of
# every benchmark workload is compared, not a sample.

def _full(name):
    case = make_case(**WORKLOADS[name])
    dec, out, lse = run(case)
    check_plan_arrays(case, dec)
    assert_close(case, out, lse, label=name)


def test_dense_b64_h128_ctx8192_bf16_full():
    _full("dense_b64_h128_ctx8192_bf16")


def test_dense_b64_h128_ctx8192_fp8_full():
    _full("dense_b64_h128_ctx8192_fp8")


def test_dense_b64_h128_ctx8192_fp8q_full():
    _full("dense_b64_h128_ctx8192_fp8q")


def test_ragged_b256_h128_fp8_p64_full():
    _full("ragged_b256_h128_fp8_p64")


@pytest.mark.parametrize("b", [1, 2, 3, 4, 5])
def test_longctx_h12_ctx109440_fp8(b):
    _full(f"longctx_b{b}_h12_ctx109440_fp8")


def test_causal_mtp4_b128_h16_ctx5200_fp8_p16_full():
    _full("causal_mtp4_b128_h16_ctx5200_fp8_p16")


@pytest.mark.parametrize("b", [1, 5, 16])
def test_small_batch_h128_ctx8192_fp8q_full(b):
    _full(f"small_b{b}_h128_ctx8192_fp8q")
