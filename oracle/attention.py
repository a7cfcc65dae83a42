"""fp64 reference of MLA decode over a paged latent cache (test infrastructure).

Every step is written out as its plain definition; numpy's dgemm is the only
library primitive used for the dot products. See the package docstring for the
reading of the pages this follows.
"""

import numpy as np

from .fp8 import bf16_bits_to_f64, decode_e4m3fn

LATENT_DIM = 512  # the V slice: latent part of the row, first in the row
ROPE_DIM = 64  # the rope part of the row, after the latent part
ROW_DIM = LATENT_DIM + ROPE_DIM  # 576-wide cache row and query row


def row_slots(kv_indptr, kv_page_indices, b, n_rows, page_size) -> np.ndarray:
    """Physical cache slot of each logical row ``r < n_rows`` of sequence ``b``.

    The page list of sequence ``b`` is ``kv_page_indices[kv_indptr[b]:kv_indptr[b+1]]``;
    row ``r`` lives in page ``r // page_size`` of that list, at offset
    ``r % page_size`` inside the page ("HK MLA ... page_size + mask support",
    Summary: variable page size; the page list form follows aiter's kv_indices
    named in that page's file table).
    """
    r = np.arange(int(n_rows), dtype=np.int64)
    first = int(kv_indptr[b])
    pages = np.asarray(kv_page_indices, dtype=np.int64)[first + r // page_size]
    return pages * int(page_size) + r % page_size


def dequantize_rows(raw_rows, kv_dtype: str, kv_scale: float) -> np.ndarray:
    """Cache rows to float64: bf16 exactly, fp8 e4m3fn exactly times the per-tensor scale."""
    if kv_dtype == "bf16":
        return bf16_bits_to_f64(raw_rows)
    if kv_dtype == "fp8_e4m3fn":
        return decode_e4m3fn(raw_rows) * np.float64(kv_scale)
    raise ValueError(f"unknown kv dtype {kv_dtype!r}")


def attend(q, keys, values, softmax_scale):
    """Softmax attention of query rows over key/value rows, in float64.

    q [R, 576], keys [n, 576], values [n, 512]. Returns (out [R, 512], lse [R]).
    With no rows (n == 0) the softmax is empty: out is 0 and lse is -inf, the
    value that gives such a piece weight 0 in ``merge_partials``.
    """
    q = np.asarray(q, dtype=np.float64)
    R = q.shape[0]
    n = keys.shape[0]
    if n == 0:
        return np.zeros((R, values.shape[1]), np.float64), np.full(R, -np.inf)
    z = np.float64(softmax_scale) * (q @ keys.T)  # [R, n]
    mu = z.max(axis=1)
    w = np.exp(z - mu[:, None])
    denom = w.sum(axis=1)
    out = (w @ values) / denom[:, None]
    lse = mu + np.log(denom)
    return out, lse


def merge_partials(outs, lses):
    """Merge softmax results computed on disjoint pieces of the same row set.

    outs [J, ..., 512], lses [J, ...] (natural-log lse of each piece). With
    M = max_j lse_j and w_j = exp(lse_j - M):  out = sum_j w_j out_j / sum_j w_j,
    lse = M + ln(sum_j w_j). Pieces with lse = -inf (no rows) weigh 0; if every
    piece is empty the result is out = 0, lse = -inf. The pages describe no merge;
    this is the standard identity for splitting a softmax sum, and it is pinned by
    the split/merge invariant test.
    """
    outs = np.asarray(outs, dtype=np.float64)
    lses = np.asarray(lses, dtype=np.float64)
    M = lses.max(axis=0)
    empty = np.isneginf(M)
    M_safe = np.where(empty, 0.0, M)
    w = np.exp(lses - M_safe[None])  # exp(-inf) = 0 for empty pieces
    total = w.sum(axis=0)
    total_safe = np.where(empty, 1.0, total)
    out = (w[..., None] * outs).sum(axis=0) / total_safe[..., None]
    out = np.where(empty[..., None], 0.0, out)
    lse = np.where(empty, -np.inf, M_safe + np.log(total_safe))
    return out, lse


def visible_rows(ctx, seqlen_qo, s, causal) -> int:
    """Rows that query token ``s`` of a sequence with ``ctx`` cached rows sees.

    Without the mask every token sees all ``ctx`` rows. With it, the ``seqlen_qo``
    draft tokens are the last ``seqlen_qo`` rows of the context, so token ``s``
    sees ``ctx - seqlen_qo + 1 + s`` rows ("HK MLA ... page_size + mask support",
    Summary: causal mask for the nh/mtp shapes).
    """
    return int(ctx) - int(seqlen_qo) + 1 + int(s) if causal else int(ctx)


def query_values(q_rows, q_scale=1.0) -> np.ndarray:
    """Query rows in float64: bf16 bits (uint16) exactly, or e4m3fn bytes (uint8) times the
    per-tensor q_scale, the fp8-query x fp8-cache setting of the HK page's fp8_fp8 kernels."""
    q_rows = np.asarray(q_rows)
    if q_rows.dtype == np.uint8:
        return decode_e4m3fn(q_rows) * np.float64(np.float32(q_scale))
    return bf16_bits_to_f64(q_rows)


def mla_decode_reference_one(q_bits, cache_raw, kv_dtype, kv_scale, kv_indptr, kv_page_indices,
                             context_lens, page_size, softmax_scale, causal, b, q_scale=1.0):
    """Reference output of one sequence ``b``: (out [S, H, 512], lse [S, H]) in float64."""
    q_bits = np.asarray(q_bits)
    S, H = q_bits.shape[1], q_bits.shape[2]
    ctx = int(context_lens[b])
    slots = row_slots(kv_indptr, kv_page_indices, b, ctx, page_size)
    keys = dequantize_rows(np.asarray(cache_raw)[slots], kv_dtype, kv_scale)  # [ctx, 576]
    values = keys[:, :LATENT_DIM]
    out = np.zeros((S, H, LATENT_DIM), np.float64)
    lse = np.zeros((S, H), np.float64)
    for s in range(S):
        n = visible_rows(ctx, S, s, causal)
        q = query_values(q_bits[b, s], q_scale)  # [H, 576]
        out[s], lse[s] = attend(q, keys[:n], values[:n], softmax_scale)
    return out, lse


def mla_decode_reference(q_bits, cache_raw, kv_dtype, kv_scale, kv_indptr, kv_page_indices,
                         context_lens, page_size, softmax_scale, causal, batches=None, q_scale=1.0):
    """Reference MLA decode over the whole batch (or the listed ``batches``).

    q_bits [B, S, H, 576] uint16 (bf16 bits), or uint8 (fp8 e4m3fn bytes, each times q_scale);
    cache_raw [num_slots, 576] uint16 (bf16)
    or uint8 (fp8 e4m3fn); kv_indptr [B+1], kv_page_indices, context_lens [B] int.
    Returns (out [B, S, H, 512], lse [B, S, H]) float64; rows of batches not listed
    are left NaN.
    """
    q_bits = np.asarray(q_bits)
    B, S, H, D = q_bits.shape
    if D != ROW_DIM:
        raise ValueError("query rows must be 576 wide")
    out = np.full((B, S, H, LATENT_DIM), np.nan)
    lse = np.full((B, S, H), np.nan)
    for b in (range(B) if batches is None else batches):
        out[b], lse[b] = mla_decode_reference_one(q_bits, cache_raw, kv_dtype, kv_scale, kv_indptr,
                                                  kv_page_indices, context_lens, page_size,
                                                  softmax_scale, causal, b, q_scale)
    return out, lse
