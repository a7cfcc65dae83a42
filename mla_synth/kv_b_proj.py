"""Seeded inputs for the cached-prefix expansion (gather_kv_b_proj).

Recipe (deterministic for a given seed):

* the paged latent cache, page table and context lengths come from the decode
  generator (``make_case``): pool rows ~ N(0, 1) rounded to bf16, or quantised to
  e4m3fn with the per-tensor scale ``amax / 448``; pages dealt from a seeded
  permutation of the pool;
* ``cu_ctx [B + 1]``: the exclusive prefix sum of the context lengths (output row
  of each sequence's first cached row);
* the projection ``w [H, 256, 512]`` ~ N(0, 1/512) in float32 rounded to bf16, from
  its own stream ``default_rng([seed, 30])``, so a K or V element is of the same
  size as a latent element.

The workloads are the shapes the pages time this kernel on: 12 local heads
(Kimi-K3 at TP8), an fp8 cache with page size 1, one sequence of 4096, 32000,
65536 or 109440 cached rows ("perf(mla): chunk the non-FP4 gather_kv_b_proj over
KV", ctx table).
"""

from dataclasses import dataclass

import numpy as np
import torch

from .gen import make_case


@dataclass
class KvbCase:
    name: str
    batch: int
    num_heads: int
    page_size: int
    kv_dtype: str
    kv_scale: float
    num_slots: int
    max_context_len: int
    cache_raw: np.ndarray        # uint16 [num_slots, 576] (bf16) or uint8 (fp8)
    kv_indptr: np.ndarray        # int32 [B + 1]
    kv_page_indices: np.ndarray  # int32 [total pages]
    context_lens: np.ndarray     # int32 [B]
    cu_ctx: np.ndarray           # int32 [B + 1]
    w_bits: np.ndarray           # uint16 [H, 256, 512]

    @property
    def total_rows(self) -> int:
        return int(self.cu_ctx[-1])


def make_kvb_case(*, batch, num_heads, ctx, page_size, kv_dtype, seed=0, pool_pages=None,
                  name="kvb_case") -> KvbCase:
    base = make_case(batch=batch, seqlen_qo=1, num_heads=1, ctx=ctx, page_size=page_size, kv_dtype=kv_dtype,
                     seed=seed, pool_pages=pool_pages, name=name)
    H = int(num_heads)
    w = np.random.default_rng([seed, 30]).standard_normal((H, 256, 512), dtype=np.float32) / np.float32(np.sqrt(512.0))
    w_bits = torch.from_numpy(w).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    lens = base.context_lens.astype(np.int64)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    return KvbCase(name=name, batch=base.batch, num_heads=H, page_size=base.page_size, kv_dtype=kv_dtype,
                   kv_scale=base.kv_scale, num_slots=base.num_slots, max_context_len=base.max_context_len,
                   cache_raw=base.cache_raw, kv_indptr=base.kv_indptr, kv_page_indices=base.kv_page_indices,
                   context_lens=base.context_lens, cu_ctx=cu, w_bits=w_bits)


KVB_WORKLOADS = {
    f"kvb_b1_h12_ctx{c}_fp8": dict(batch=1, num_heads=12, ctx=c, page_size=1, kv_dtype="fp8_e4m3fn", seed=60 + i)
    for i, c in enumerate((4096, 32000, 65536, 109440))
}
# a ragged batch with an empty sequence and lengths that are not multiples of 128
KVB_WORKLOADS["kvb_ragged_b5_h12_fp8_p16"] = dict(batch=5, num_heads=12, ctx=[0, 1, 127, 300, 2049], page_size=16,
                                                  kv_dtype="fp8_e4m3fn", seed=70, pool_pages=300)
KVB_WORKLOADS["kvb_ragged_b3_h8_bf16_p64"] = dict(batch=3, num_heads=8, ctx=[129, 640, 1000], page_size=64,
                                                  kv_dtype="bf16", seed=71, pool_pages=40)
