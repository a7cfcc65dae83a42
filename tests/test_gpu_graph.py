"""HIP-graph capture of one decode call (mla_decode + mla_split_combine through the C ABI).

A serving loop replays the call from a captured graph: the two launches allocate
nothing and record no memset, so the graph is the eager call. The graph is replayed
several times with eager work (NaN fills of the outputs) and synchronisations in
between, and every replay must reproduce the eager result bit for bit."""

import numpy as np
import pytest
import torch

from mla_synth import make_case

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    import mla_paged_latent_02_amd  # noqa: F401  (fails loudly if the library is missing)
    yield


@pytest.mark.parametrize("kv_dtype,q_dtype,force", [("bf16", "bf16", 256), ("fp8_e4m3fn", "bf16", 64),
                                                    ("fp8_e4m3fn", "fp8_e4m3fn", 0)])
def test_graph_replays_match_the_eager_call(kv_dtype, q_dtype, force):
    import mla_paged_latent_02_amd as mla
    from mla_paged_latent_02_amd.device import Decoder, DeviceInputs
    case = make_case(batch=3, seqlen_qo=2, num_heads=32, ctx=[700, 5, 1300], page_size=16, kv_dtype=kv_dtype,
                     causal=True, seed=83, q_dtype=q_dtype)
    inp = DeviceInputs.from_host(
        q_bits=case.q_bits, cache_raw=case.cache_raw, kv_indptr=case.kv_indptr,
        kv_page_indices=case.kv_page_indices, context_lens=case.context_lens, batch=case.batch,
        seqlen_qo=case.seqlen_qo, num_heads=case.num_heads, page_size=case.page_size,
        max_context_len=case.max_context_len, causal=case.causal, kv_dtype=case.kv_dtype,
        softmax_scale=case.softmax_scale, kv_scale=case.kv_scale, num_slots=case.num_slots,
        q_dtype=case.q_dtype, q_scale=case.q_scale)
    dec = Decoder(inp, mla.make_options(force_chunk=force))
    out, lse = dec()
    torch.cuda.synchronize()
    ref_o = out.float().cpu().numpy().view(np.uint32).copy()
    ref_l = lse.cpu().numpy().view(np.uint32).copy()

    def call(stream):
        mla.decode(dec.plan, inp.q, inp.cache, inp.kv_indptr, inp.kv_page_indices, inp.context_lens, dec.out,
                   dec.lse, dec.workspace, stream)
        mla.split_combine(dec.plan, dec.workspace, dec.out, dec.lse, stream)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call(side)  # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=side):
        call(torch.cuda.current_stream())
    for _ in range(3):
        dec.out.fill_(float("nan"))
        dec.lse.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert np.array_equal(dec.out.float().cpu().numpy().view(np.uint32), ref_o)
        assert np.array_equal(dec.lse.cpu().numpy().view(np.uint32), ref_l)
