"""Bitwise parity of the decode epilogue (mla_qcat_cache_insert, through the C ABI)
with the oracle, on MI355X: the query, every cache row (written or not) and the
status word must match exactly."""

import numpy as np
import pytest
import torch

import oracle
from mla_synth import INSERT_WORKLOADS, make_insert_case

pytestmark = pytest.mark.gpu


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


def run_insert(c):
    import mla_paged_latent_02_amd as mla
    q = torch.full((c.num_tokens, c.num_heads, 576), -1, dtype=torch.int16, device="cuda")  # poison
    cache = _dev(c.cache)
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    p = mla.make_insert_params(num_tokens=c.num_tokens, num_heads=c.num_heads, kv_dtype=c.kv_dtype,
                               kv_scale=c.kv_scale, num_slots=c.num_slots, rope_positions=c.rope_positions,
                               rope_neox=c.neox)
    mla.qcat_cache_insert(p, _dev(c.ql_nope), _dev(c.q_pe), _dev(c.kv_c), _dev(c.k_pe), _dev(c.positions),
                          _dev(c.cos_sin), _dev(c.slot_mapping), q, cache, status)
    torch.cuda.synchronize()
    out_cache = cache.cpu().numpy()
    if c.kv_dtype == "bf16":
        out_cache = out_cache.view(np.uint16)
    return q.cpu().numpy().view(np.uint16), out_cache, int(status.item())


def check(c, label=""):
    q, cache, status = run_insert(c)
    rq, rcache, rstatus = oracle.qcat_cache_insert_reference(
        c.ql_nope, c.q_pe, c.kv_c, c.k_pe, c.positions, c.cos_sin, c.slot_mapping, c.cache, c.kv_dtype, c.kv_scale,
        c.neox)
    assert np.array_equal(q, rq), f"{label}: query differs at {np.argwhere(q != rq)[:3]}"
    bad = np.argwhere(cache != rcache)
    assert bad.size == 0, f"{label}: {len(bad)} cache elements differ, first {bad[:3]}"
    assert status == rstatus
    return status


GRID = [(T, H, kv, neox, pad) for T in (1, 3, 64, 65, 200) for H in (1, 8, 12, 128) if not (T > 65 and H == 128)
        for kv in ("bf16", "fp8_e4m3fn") for neox in (False, True) for pad in (0, 4)]


@pytest.mark.parametrize("T,H,kv,neox,pad", GRID)
def test_insert_grid(T, H, kv, neox, pad):
    c = make_insert_case(num_tokens=T, num_heads=H, kv_dtype=kv, neox=neox, pad_every=pad, rope_positions=512,
                         seed=GRID.index((T, H, kv, neox, pad)))
    check(c, f"T={T} H={H} {kv} neox={neox} pad={pad}")


@pytest.mark.parametrize("name", sorted(INSERT_WORKLOADS))
def test_insert_workloads(name):
    check(make_insert_case(**INSERT_WORKLOADS[name]), name)


def test_insert_bad_slot_and_position_are_flagged_and_skipped():
    import mla_paged_latent_02_amd as mla
    c = make_insert_case(num_tokens=6, num_heads=4, kv_dtype="fp8_e4m3fn", rope_positions=64, seed=70)
    c.slot_mapping[1] = c.num_slots + 3
    c.positions[4] = 64
    assert check(c, "bad slot and position") == mla.INSERT_SLOT_OUT_OF_RANGE | mla.INSERT_POSITION_OUT_OF_RANGE


def test_insert_saturation_nan_and_signed_zero_in_fp8():
    c = make_insert_case(num_tokens=4, num_heads=2, kv_dtype="fp8_e4m3fn", seed=71)
    bits = lambda v: np.float32(v).view(np.uint32) >> 16
    c.kv_c[0, :6] = [bits(np.inf), bits(-np.inf), bits(np.nan), bits(-0.0), bits(1e30), bits(-1e30)]
    check(c, "special values")


def test_insert_zero_tokens_is_a_no_op():
    import mla_paged_latent_02_amd as mla
    p = mla.make_insert_params(num_tokens=0, num_heads=8, kv_dtype="bf16", kv_scale=1.0, num_slots=4,
                               rope_positions=4, rope_neox=False)
    assert mla.lib().mla_qcat_cache_insert(p, None, None, None, None, None, None, None, None, None, None, None) == 0
