"""Pins of the oracle's fp8-query path (CPU only): the query is e4m3fn bytes times one
per-tensor q_scale, the fp8-query x fp8-cache setting of the fp8_fp8 kernels in the
file table of "HK MLA: MI35x m16x8 retune, new m16x4 kernel, page_size + mask support".

* brute force: the pure-Python loops (their own e4m3fn decoder from the bit formula)
  on tiny cases, including the causal mask and several page sizes;
* reduction to the bf16-query path: when q_scale is a power of two, every query
  value is a bf16 value, so widening the bytes with torch's own fp8 cast and running
  the (separately pinned) bf16-query oracle must give the same result bit for bit;
* the scale is a factor of every score: q_scale moves into softmax_scale;
* a planted slip (q_scale dropped) fails the brute-force pin.
"""

import numpy as np
import pytest
import torch

import oracle
from oracle import attention as oatt
from mla_synth import make_case
from _brute import brute_decode


def tiny_fp8q(seed, causal=False, S=1, H=3, ctx=(5, 9), P=2):
    return make_case(batch=len(ctx), seqlen_qo=S, num_heads=H, ctx=list(ctx), page_size=P,
                     kv_dtype="fp8_e4m3fn", causal=causal, seed=seed, q_dtype="fp8_e4m3fn")


def run(case, q_bits=None, q_scale=None, softmax_scale=None):
    return oracle.mla_decode_reference(case.q_bits if q_bits is None else q_bits, case.cache_raw, case.kv_dtype,
                                       case.kv_scale, case.kv_indptr, case.kv_page_indices, case.context_lens,
                                       case.page_size, case.softmax_scale if softmax_scale is None else softmax_scale,
                                       case.causal, q_scale=case.q_scale if q_scale is None else q_scale)


def brute_arrays(case):
    bout, blse = brute_decode(case)
    B, S, H = case.batch, case.seqlen_qo, case.num_heads
    out = np.array([[[bout[(b, s, h)] for h in range(H)] for s in range(S)] for b in range(B)], dtype=np.float64)
    lse = np.array([[[blse[(b, s, h)] for h in range(H)] for s in range(S)] for b in range(B)], dtype=np.float64)
    return out, lse


CASES = [dict(seed=1), dict(seed=2, S=2, causal=True, ctx=(4, 7), P=3), dict(seed=3, H=2, ctx=(1, 6), P=1),
         dict(seed=4, S=3, causal=True, ctx=(3, 8), P=2)]


@pytest.mark.parametrize("kw", CASES)
def test_fp8_query_against_brute_force(kw):
    case = tiny_fp8q(**kw)
    assert case.q_bits.dtype == np.uint8 and case.q_scale > 0
    out, lse = run(case)
    bout, blse = brute_arrays(case)
    assert np.max(np.abs(out - bout)) <= 1e-12 * max(1.0, np.max(np.abs(bout)))
    assert np.max(np.abs(lse - blse)) <= 1e-12 * max(1.0, np.max(np.abs(blse)))


def test_fp8_query_reduces_to_bf16_query_with_torch_casts():
    case = tiny_fp8q(seed=7, S=2, causal=True, H=4, ctx=(6, 11), P=4)
    q_scale = 0.125  # a power of two: every e4m3fn value times it is a bf16 value
    q = torch.from_numpy(case.q_bits.copy()).view(torch.float8_e4m3fn).to(torch.float32) * q_scale
    q_bf16 = q.to(torch.bfloat16)
    assert torch.equal(q_bf16.to(torch.float32), q)  # exact
    q_bits_bf16 = q_bf16.view(torch.int16).numpy().view(np.uint16)
    out8, lse8 = run(case, q_scale=q_scale)
    out16, lse16 = run(case, q_bits=q_bits_bf16, q_scale=1.0)
    assert np.array_equal(out8, out16) and np.array_equal(lse8, lse16)


def test_q_scale_is_a_factor_of_every_score():
    case = tiny_fp8q(seed=8, H=3, ctx=(9, 4), P=2)
    s = 0.37
    out_a, lse_a = run(case, q_scale=s, softmax_scale=case.softmax_scale)
    out_b, lse_b = run(case, q_scale=1.0, softmax_scale=case.softmax_scale * np.float64(np.float32(s)))
    assert np.max(np.abs(out_a - out_b)) <= 1e-12 and np.max(np.abs(lse_a - lse_b)) <= 1e-12


def test_dropped_q_scale_is_caught(monkeypatch):
    case = tiny_fp8q(seed=9, H=2, ctx=(7, 5), P=2)
    bout, _ = brute_arrays(case)
    orig = oatt.query_values
    monkeypatch.setattr(oatt, "query_values", lambda rows, sc=1.0: orig(rows, 1.0))
    out, _ = run(case)
    assert np.max(np.abs(out - bout)) > 1e-6
