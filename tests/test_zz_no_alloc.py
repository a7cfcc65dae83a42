"""mla_decode_scratch, the entry point that allocates nothing (its workspace is the
library's static device array), against the workspace entry points on MI355X.

Two calls in a row, the second with a smaller input, each compared bit for bit
with mla_decode_plan + mla_decode + mla_split_combine on a fresh workspace (the
same kernels and plan: identical bits), and with the fp64 oracle at the path's
tolerance (|gpu - oracle| <= 1e-2 + 1e-2 |oracle|). A call that needs more than
the static array is rejected before any device work.
"""

import numpy as np
import pytest
import torch

import oracle
from mla_synth import make_case

pytestmark = pytest.mark.gpu

ATOL = 1e-2
RTOL = 1e-2


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    import mla_paged_latent_02_amd  # noqa: F401  (fails loudly if the library is missing)
    yield


def _upload(case):
    from mla_paged_latent_02_amd.device import DeviceInputs
    return DeviceInputs.from_host(
        q_bits=case.q_bits, cache_raw=case.cache_raw, kv_indptr=case.kv_indptr,
        kv_page_indices=case.kv_page_indices, context_lens=case.context_lens, batch=case.batch,
        seqlen_qo=case.seqlen_qo, num_heads=case.num_heads, page_size=case.page_size,
        max_context_len=case.max_context_len, causal=case.causal, kv_dtype=case.kv_dtype,
        softmax_scale=case.softmax_scale, kv_scale=case.kv_scale, num_slots=case.num_slots,
        q_dtype=case.q_dtype, q_scale=case.q_scale)


def _scratch_call(inp):
    import mla_paged_latent_02_amd as mla
    p = inp.params
    out = torch.full((p.batch, p.seqlen_qo, p.num_heads, 512), float("nan"), dtype=torch.bfloat16, device="cuda")
    lse = torch.full((p.batch, p.seqlen_qo, p.num_heads), float("nan"), dtype=torch.float32, device="cuda")
    plan = mla.decode_scratch(p, inp.q, inp.cache, inp.kv_indptr, inp.kv_page_indices, inp.context_lens, out, lse)
    torch.cuda.synchronize()
    return plan, out.float().cpu().numpy(), lse.cpu().numpy()


def _check_against_oracle(case, out, lse):
    ref_out, ref_lse = oracle.mla_decode_reference(case.q_bits, case.cache_raw, case.kv_dtype, case.kv_scale,
                                                   case.kv_indptr, case.kv_page_indices, case.context_lens,
                                                   case.page_size, case.softmax_scale, case.causal,
                                                   q_scale=case.q_scale)
    assert np.all(np.abs(out - ref_out) <= ATOL + RTOL * np.abs(ref_out))
    assert np.all(np.abs(lse - ref_lse) <= ATOL + RTOL * np.abs(ref_lse))


def test_scratch_entry_point_matches_the_workspace_path_on_two_calls():
    import mla_paged_latent_02_amd as mla
    from mla_paged_latent_02_amd.device import Decoder
    # first a batch whose sequences are split (128 heads, bf16, a workspace of ~67 MB), then a
    # smaller one (16 heads x 4 causal tokens, fp8 cache, ~2 MB): the second call reuses the
    # array the first one left full
    cases = [
        make_case(batch=16, seqlen_qo=1, num_heads=128, ctx=("uniform", 40, 3000), page_size=16,
                  kv_dtype="bf16", seed=700),
        make_case(batch=3, seqlen_qo=4, num_heads=16, ctx=[5, 600, 1300], page_size=16, kv_dtype="fp8_e4m3fn",
                  causal=True, seed=701),
    ]
    sizes = []
    for case in cases:
        inp = _upload(case)
        sizes.append(mla.workspace_size(inp.params))
        assert sizes[-1] <= mla.SCRATCH_BYTES
        plan, out_s, lse_s = _scratch_call(inp)
        dec = Decoder(inp, None, poison=True)
        out_w, lse_w = dec()
        torch.cuda.synchronize()
        assert mla.plan_to_dict(plan) == mla.plan_to_dict(dec.plan)
        assert plan.max_chunks > 1  # the merge ran
        assert np.array_equal(out_s.view(np.uint32), out_w.float().cpu().numpy().view(np.uint32))
        assert np.array_equal(lse_s.view(np.uint32), lse_w.cpu().numpy().view(np.uint32))
        _check_against_oracle(case, out_s, lse_s)
    assert sizes[1] < sizes[0]


def test_scratch_entry_point_rejects_calls_larger_than_its_array():
    import math
    import mla_paged_latent_02_amd as mla
    # the ragged 256 x 128-head shape needs ~270 MB of partials, more than the static array: the
    # host half rejects it before any device work, so the buffers are never read (small stand-ins)
    p = mla.make_params(batch=256, seqlen_qo=1, num_heads=128, page_size=64, max_context_len=23333, causal=False,
                        kv_dtype="fp8_e4m3fn", softmax_scale=1 / math.sqrt(192), kv_scale=0.01,
                        num_slots=64 * 47000)
    assert mla.workspace_size(p) > mla.SCRATCH_BYTES
    small = torch.zeros(16, dtype=torch.int32, device="cuda")
    out = torch.full((4,), float("nan"), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(mla.MlaError) as e:
        mla.decode_scratch(p, small, small, small, small, small, out, None)
    assert e.value.status == 6  # MLA_ERR_SCRATCH_TOO_SMALL
    torch.cuda.synchronize()
    assert torch.isnan(out.float()).all()  # untouched
