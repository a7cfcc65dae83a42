"""Writes oracle_tiny_fingerprint.json: a regression fingerprint of the oracle.

The pages print no worked example with output values, so nothing here comes from
them. This script calls only the oracle and the seeded input generator; the
fixture guards the oracle against accidental change (any change to its
arithmetic must come with a regenerated file and a reason).
Run from the repository root: python tests/golden/make_golden.py
"""
import json
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
from mla_synth import make_case  # noqa: E402

CASES = {
    "tiny_bf16": dict(batch=2, seqlen_qo=1, num_heads=16, ctx=[37, 100], page_size=1, kv_dtype="bf16",
                      pool_pages=256, seed=1),
    "causal_fp8": dict(batch=2, seqlen_qo=3, num_heads=4, ctx=[9, 70], page_size=16,
                       kv_dtype="fp8_e4m3fn", causal=True, seed=7),
}


def fingerprint(spec):
    c = make_case(**spec)
    out, lse = oracle.mla_decode_reference(c.q_bits, c.cache_raw, c.kv_dtype, c.kv_scale, c.kv_indptr,
                                           c.kv_page_indices, c.context_lens, c.page_size,
                                           c.softmax_scale, c.causal)
    return {
        "spec": spec,
        "row_sums": [float(x) for x in out.sum(axis=-1).ravel()],
        "samples": [float(out.reshape(-1, 512)[i % out.reshape(-1, 512).shape[0], (37 * i) % 512])
                    for i in range(16)],
        "lse": [float(x) for x in lse.ravel()],
    }


if __name__ == "__main__":
    data = {k: fingerprint(v) for k, v in CASES.items()}
    with open(os.path.join(os.path.dirname(os.path.abspath(__file__)), "oracle_tiny_fingerprint.json"), "w") as f:
        json.dump(data, f, indent=1)
