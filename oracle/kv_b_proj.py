"""Reference for the cached-prefix expansion of the paged latent cache into
per-head K and V, the "gather_kv_b_proj" (TEST INFRASTRUCTURE: only the tests,
the smoke check and the benchmark's CPU-baseline leg use it).

Page "perf(mla): chunk the non-FP4 gather_kv_b_proj over KV" (description): once
per MLA layer, the cached prefix is expanded from the paged latent into full
per-head K and V over the whole cached context, one program per (batch, head,
KV chunk), chunks past a sequence's end exiting at once. The page prints no
formula; the plainest reading (the standard MLA up-projection, ``kv_b_proj``
applied to the cached latent) is taken:

* Sequence b has ``ctx_b = cu_ctx[b + 1] - cu_ctx[b]`` cached rows; its row r is
  cache slot ``kv_page_indices[kv_indptr[b] + r // P] * P + r % P`` (the same
  page-list form as the decode), whose first 512 columns are the latent c and
  last 64 the rope part k_pe (already rotated when the row was inserted).
* The projection is one bf16 matrix per head, ``W[h]`` of 256 x 512: rows 0..127
  give the head's K "nope" part, rows 128..255 its V (the kv_b_proj weight laid
  out as [H * 256, 512]).
* Output row ``cu_ctx[b] + r``: ``k[row, h] = (W[h][0:128] c, k_pe)`` (192 wide)
  and ``v[row, h] = W[h][128:256] c``.
* fp8 cache: c is the e4m3fn values times the per-tensor kv_scale. The
  projection is the exact fp64 product here. The copied rope part is
  ``bf16(float32(e4m3fn value) * float32(kv_scale))`` (one float32 product, round
  to nearest even) for an fp8 cache and a bit copy for a bf16 cache, so it is
  compared bit for bit.

Pins: ``tests/test_oracle_kv_b_proj.py`` (selection weights that turn the product
into a known permutation of latent columns, head independence, page
permutation, the fp8 scale, the rope part against torch's own casts, a
pure-Python brute force on tiny inputs).
"""

import numpy as np

from .attention import dequantize_rows, row_slots
from .fp8 import bf16_bits_to_f64, decode_e4m3fn
from .insert import f32_to_bf16_rne

NOPE_DIM = 128  # K "nope" part of a head
V_DIM = 128  # V of a head
W_ROWS = NOPE_DIM + V_DIM  # rows of one head's projection matrix
LATENT = 512
ROPE = 64


def rope_bits(raw_rows, kv_dtype: str, kv_scale: float) -> np.ndarray:
    """The rope part of cache rows as bf16 bits: a copy (bf16) or bf16(f32(e4m3fn) * f32(scale))."""
    raw = np.asarray(raw_rows)[:, LATENT:]
    if kv_dtype == "bf16":
        return raw.astype(np.uint16)
    vals = decode_e4m3fn(raw).astype(np.float32) * np.float32(kv_scale)  # exact widening, one f32 product
    return f32_to_bf16_rne(vals)


def output_rows(cu_ctx) -> list:
    """[(b, r, out_row)] for every cached row, in output-row order."""
    cu = np.asarray(cu_ctx, dtype=np.int64)
    return [(b, r, int(cu[b]) + r) for b in range(len(cu) - 1) for r in range(int(cu[b + 1] - cu[b]))]


def gather_kv_b_proj_reference(cache_raw, kv_dtype, kv_scale, kv_indptr, kv_page_indices, cu_ctx, page_size,
                               w_bits, rows=None):
    """K and V of the cached prefix, in float64 (K's rope part as bf16 bits).

    w_bits: bf16 bits [H, 256, 512]. rows: optional list of (b, r) pairs to compute
    (default: every cached row, in output-row order).
    Returns (k_nope [N, H, 128] f64, k_rope [N, H, 64] uint16, v [N, H, 128] f64),
    row i belonging to ``rows[i]`` (or to output row i by default).
    """
    cu = np.asarray(cu_ctx, dtype=np.int64)
    if rows is None:
        rows = [(b, r) for b, r, _ in output_rows(cu)]
    w = bf16_bits_to_f64(np.asarray(w_bits, dtype=np.uint16))  # [H, 256, 512]
    H = w.shape[0]
    if not rows:
        return np.zeros((0, H, NOPE_DIM)), np.zeros((0, H, ROPE), np.uint16), np.zeros((0, H, V_DIM))
    slots = np.empty(len(rows), np.int64)
    seq_slots = {}  # the slots of every cached row of a sequence, gathered once per sequence
    for i, (b, r) in enumerate(rows):
        if not 0 <= r < cu[b + 1] - cu[b]:
            raise ValueError(f"row {r} is not a cached row of sequence {b}")
        if b not in seq_slots:
            seq_slots[b] = row_slots(kv_indptr, kv_page_indices, b, int(cu[b + 1] - cu[b]), page_size)
        slots[i] = seq_slots[b][r]
    raw = np.asarray(cache_raw)[slots]
    latent = dequantize_rows(raw, kv_dtype, kv_scale)[:, :LATENT]  # [N, 512]
    proj = (latent @ w.reshape(H * W_ROWS, LATENT).T).reshape(len(rows), H, W_ROWS)  # dgemm
    k_rope = np.repeat(rope_bits(raw, kv_dtype, kv_scale)[:, None, :], H, axis=1)
    return proj[:, :, :NOPE_DIM], k_rope, proj[:, :, NOPE_DIM:]
