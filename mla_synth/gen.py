"""Seeded generator of MLA decode inputs (queries, paged latent cache, page table).

Recipe (deterministic for a given seed):

* query rows ``q[B, S, H, 576]`` ~ N(0, 1) in float32, rounded to bf16 (RNE);
* a cache pool of ``num_pages * page_size`` rows of 576 values ~ N(0, 1) in
  float32, generated in fixed blocks of rows so memory stays bounded;
  - bf16 pool: rounded to bf16 (RNE);
  - fp8 pool: per-tensor ``kv_scale = float32(amax / 448)`` over the whole pool
    (1 if amax is 0), then ``x / kv_scale`` clipped to [-448, 448] and rounded to
    e4m3fn (RNE) by torch;
* pages: ``ceil(ctx_b / page_size)`` pages per sequence, dealt in batch order from
  a seeded permutation of all pool pages (the pool may hold spare pages);
* context lengths: given, or drawn uniformly from an inclusive range.

Each part draws from its own stream ``default_rng([seed, part, ...])`` so that a
part can be regenerated without the others.
"""

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass
from typing import Optional

import numpy as np
import torch

ROW = 576  # width of a cache row and of a query row (512 latent + 64 rope)
FP8_MAX = 448.0  # largest finite e4m3fn value
_GEN_ROWS = 1 << 16  # pool rows generated per block


@dataclass
class MlaCase:
    name: str
    batch: int
    seqlen_qo: int
    num_heads: int
    page_size: int
    causal: bool
    kv_dtype: str  # "bf16" or "fp8_e4m3fn"
    softmax_scale: float
    kv_scale: float
    max_context_len: int
    num_slots: int
    q_bits: np.ndarray  # [B, S, H, 576]: uint16 (bf16) or uint8 (fp8 e4m3fn bytes)
    cache_raw: np.ndarray  # uint16 [num_slots, 576] (bf16) or uint8 (fp8)
    kv_indptr: np.ndarray  # int32 [B + 1]
    kv_page_indices: np.ndarray  # int32 [total pages]
    context_lens: np.ndarray  # int32 [B]
    q_dtype: str = "bf16"  # or "fp8_e4m3fn": query value = byte * q_scale
    q_scale: float = 1.0

    @property
    def kv_bytes_per_elem(self) -> int:
        return 2 if self.kv_dtype == "bf16" else 1


def _to_bf16_bits(x: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def _to_fp8_bytes(x: np.ndarray, scale: np.float32) -> np.ndarray:
    y = np.clip(x / scale, -FP8_MAX, FP8_MAX).astype(np.float32)
    t = torch.from_numpy(y).to(torch.float8_e4m3fn)
    return t.view(torch.uint8).numpy()


def _pool_block(seed: int, block: int, rows: int) -> np.ndarray:
    return np.random.default_rng([seed, 1, block]).standard_normal((rows, ROW), dtype=np.float32)


def make_case(*, batch, seqlen_qo, num_heads, ctx, page_size, kv_dtype, causal=False, seed=0,
              pool_pages: Optional[int] = None, softmax_scale: float = 1.0 / np.sqrt(192.0),
              name: str = "case", max_context_len: Optional[int] = None, q_dtype: str = "bf16") -> MlaCase:
    """Build one seeded case. ``ctx`` is an int, a list of ints, or ("uniform", lo, hi)."""
    B, S, H, P = int(batch), int(seqlen_qo), int(num_heads), int(page_size)
    if isinstance(ctx, tuple) and ctx and ctx[0] == "uniform":
        lens = np.random.default_rng([seed, 3]).integers(ctx[1], ctx[2], size=B, endpoint=True)
    elif np.ndim(ctx) == 0:
        lens = np.full(B, int(ctx))
    else:
        lens = np.asarray(ctx)
    lens = lens.astype(np.int64)
    if lens.shape != (B,):
        raise ValueError("need one context length per sequence")
    pages_b = -(-lens // P)
    total_pages = int(pages_b.sum())
    num_pages = max(total_pages, int(pool_pages or 0))
    perm = np.random.default_rng([seed, 2]).permutation(num_pages)
    kv_page_indices = perm[:total_pages].astype(np.int32)
    kv_indptr = np.concatenate([[0], np.cumsum(pages_b)]).astype(np.int32)
    num_slots = num_pages * P

    q = np.random.default_rng([seed, 0]).standard_normal((B, S, H, ROW), dtype=np.float32)
    if q_dtype == "bf16":
        q_bits, q_scale = _to_bf16_bits(q), 1.0
    elif q_dtype == "fp8_e4m3fn":  # the same per-tensor recipe as the cache: scale = amax / 448
        amax = float(np.abs(q).max())
        q_scale = np.float32(amax / FP8_MAX) if amax > 0 else np.float32(1.0)
        q_bits, q_scale = _to_fp8_bytes(q, q_scale), float(q_scale)
    else:
        raise ValueError(f"unknown query dtype {q_dtype!r}")

    # The pool is drawn in blocks of _GEN_ROWS rows, each from its own seeded stream, so the
    # blocks can be drawn on several threads (numpy and torch fill without the GIL) and the
    # bytes do not depend on the thread count.
    n_blocks = -(-num_slots // _GEN_ROWS)
    rows_of = lambda k: min(_GEN_ROWS, num_slots - k * _GEN_ROWS)
    workers = max(1, min(8, len(os.sched_getaffinity(0)), n_blocks))

    def each_block(fn):
        with ThreadPoolExecutor(max_workers=workers) as ex:
            return list(ex.map(fn, range(n_blocks)))

    if kv_dtype == "bf16":
        cache = np.empty((num_slots, ROW), np.uint16)

        def fill_bf16(k):
            cache[k * _GEN_ROWS:k * _GEN_ROWS + rows_of(k)] = _to_bf16_bits(_pool_block(seed, k, rows_of(k)))
        each_block(fill_bf16)
        kv_scale = 1.0
    elif kv_dtype == "fp8_e4m3fn":
        amax = max([0.0] + each_block(lambda k: float(np.abs(_pool_block(seed, k, rows_of(k))).max())))
        scale = np.float32(amax / FP8_MAX) if amax > 0 else np.float32(1.0)
        cache = np.empty((num_slots, ROW), np.uint8)

        def fill_fp8(k):
            cache[k * _GEN_ROWS:k * _GEN_ROWS + rows_of(k)] = _to_fp8_bytes(_pool_block(seed, k, rows_of(k)), scale)
        each_block(fill_fp8)
        kv_scale = float(scale)
    else:
        raise ValueError(f"unknown kv dtype {kv_dtype!r}")

    return MlaCase(
        name=name, batch=B, seqlen_qo=S, num_heads=H, page_size=P, causal=bool(causal),
        kv_dtype=kv_dtype, softmax_scale=float(np.float32(softmax_scale)), kv_scale=kv_scale,
        max_context_len=int(max_context_len if max_context_len is not None else lens.max()),
        num_slots=num_slots, q_bits=q_bits, cache_raw=cache, kv_indptr=kv_indptr,
        kv_page_indices=kv_page_indices, context_lens=lens.astype(np.int32), q_dtype=q_dtype, q_scale=q_scale)


# The workloads, named by what they are. Sizes follow the decode shapes the pages
# measure: 128 heads x seqlen_qo 1 with ctx up to 23333 ("HK MLA ... page_size +
# mask support", results table), 12 local heads at ctx up to 109440 with an fp8
# page-size-1 cache ("perf(mla): chunk the non-FP4 gather_kv_b_proj over KV",
# ctx table), and 16 heads x 4 draft tokens under the causal mask (the m16x4 /
# nh16+mtp shapes of the HK page's Summary).
WORKLOADS = {
    "tiny_b2_h16": dict(batch=2, seqlen_qo=1, num_heads=16, ctx=[37, 100], page_size=1,
                        kv_dtype="bf16", pool_pages=256, seed=1),
    "dense_b64_h128_ctx8192_bf16": dict(batch=64, seqlen_qo=1, num_heads=128, ctx=8192, page_size=1,
                                        kv_dtype="bf16", seed=2),
    "ragged_b256_h128_fp8_p64": dict(batch=256, seqlen_qo=1, num_heads=128, ctx=("uniform", 21, 23333),
                                     page_size=64, kv_dtype="fp8_e4m3fn", seed=3),
    "causal_mtp4_b128_h16_ctx5200_fp8_p16": dict(batch=128, seqlen_qo=4, num_heads=16, ctx=5200,
                                                 page_size=16, kv_dtype="fp8_e4m3fn", causal=True, seed=5),
    # the dense shape with an fp8 cache: the shape and precision of the pages' MI355 table row
    # (batch 64, ctx 8192, 128 heads, fp8 kernels), for comparison only
    "dense_b64_h128_ctx8192_fp8": dict(batch=64, seqlen_qo=1, num_heads=128, ctx=8192, page_size=1,
                                       kv_dtype="fp8_e4m3fn", seed=6),
    # the same shape with an fp8 query as well: the fp8_fp8 kernels of the HK page's file table
    "dense_b64_h128_ctx8192_fp8q": dict(batch=64, seqlen_qo=1, num_heads=128, ctx=8192, page_size=1,
                                        kv_dtype="fp8_e4m3fn", q_dtype="fp8_e4m3fn", seed=7),
}
# small batches of the same 128-head shape, fp8 query x fp8 cache as in the HK page's
# results table (its batch sweep at ctx 8192)
for _b, _seed in ((1, 8), (5, 9), (16, 10)):
    WORKLOADS[f"small_b{_b}_h128_ctx8192_fp8q"] = dict(batch=_b, seqlen_qo=1, num_heads=128, ctx=8192,
                                                       page_size=1, kv_dtype="fp8_e4m3fn",
                                                       q_dtype="fp8_e4m3fn", seed=_seed)
for _b in range(1, 6):
    WORKLOADS[f"longctx_b{_b}_h12_ctx109440_fp8"] = dict(batch=_b, seqlen_qo=1, num_heads=12, ctx=109440,
                                                          page_size=1, kv_dtype="fp8_e4m3fn", seed=40 + _b)


def workload_params(name: str) -> dict:
    return dict(WORKLOADS[name])
