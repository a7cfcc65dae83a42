"""CPU oracle for multi-head latent attention (MLA) decode over a paged latent KV cache.

TEST INFRASTRUCTURE. This package is the slow, plainly written fp64 reference that
the HIP library is checked against. Only the tests, the smoke check and the
benchmark's CPU-baseline leg may import it; the library and its binding never do,
and nothing here imports them. It shares no code, constants or helpers with the
HIP path: the two meet only in the seeded input generator (``mla_synth``), which
holds none of the method's arithmetic.

What it computes, and where it comes from
-----------------------------------------
The pages never print the attention formula. The plainest reading that everything
on them supports, taken here:

* "HK MLA: MI35x m16x8 retune, new m16x4 kernel, page_size + mask support"
  (Summary): decode attention runs over a *paged* latent cache with a variable
  page size, and multi-token (MTP) queries under a causal mask.
* "[Perf][Kimi-K3] Cut MLA decode concat/cache epilogue latency" (Purpose): the
  decode FMHA consumes the absorbed query (``ql_nope`` joined with ``q_pe``) and a
  576-wide latent cache row per token.
* "perf(mla): chunk the non-FP4 gather_kv_b_proj over KV" (description): the cache
  is fp8 with page size 1 in the deployed shape.

So for each query token and head, attention is scaled-dot-product attention in
absorbed form: the 576-wide latent row (512 latent + 64 rope) is the key, its first
512 columns are the value, scores are ``softmax_scale * q . k``, softmax is over the
visible rows, and ``lse`` is the natural log of the softmax denominator plus the
max. A per-tensor fp8 scale multiplies every dequantised element.

Pins (all in ``tests/test_oracle_pins.py``, CPU only): brute force in pure Python
and in 50-digit mpmath on tiny inputs, torch's float64 SDPA on gathered rows,
closed forms (one row, constant V, zero query, two rows), invariants (page
permutation, causal = truncation, split + LSE merge = unsplit, row duplication,
head permutation, affine V), the fp8 decoder against torch on all 256 bytes, and
the planner's structural invariants; the same invariants also run as hypothesis
properties over random small shapes (``tests/test_oracle_properties.py``). The decode epilogue that produces the
path's inputs (query concat and latent-cache insert, ``insert.py``) is pinned in
``tests/test_oracle_insert.py``: encoders against torch's casts and hand-derived
codes, rope against closed forms and a float64 complex product. The cached-prefix
expansion of the latent into per-head K and V (``kv_b_proj.py``) is pinned in
``tests/test_oracle_kv_b_proj.py``: selection matrices, brute force, head and page
invariants, the fp8 scale and the rope part against torch's casts. No function here
is "parity unpinned".
"""

from .fp8 import E4M3FN_VALUES, decode_e4m3fn, bf16_bits_to_f64
from .attention import (
    LATENT_DIM,
    ROPE_DIM,
    ROW_DIM,
    row_slots,
    dequantize_rows,
    query_values,
    attend,
    merge_partials,
    mla_decode_reference,
    mla_decode_reference_one,
)
from .planner import PlanOptions, reference_plan, device_plan_arrays, work_list, status_words, first_task
from .insert import bf16_bits_to_f32, f32_to_bf16_rne, f32_to_e4m3fn, rope_f32, qcat_cache_insert_reference
from .kv_b_proj import gather_kv_b_proj_reference, output_rows, rope_bits

__all__ = [
    "E4M3FN_VALUES",
    "decode_e4m3fn",
    "bf16_bits_to_f64",
    "LATENT_DIM",
    "ROPE_DIM",
    "ROW_DIM",
    "row_slots",
    "dequantize_rows",
    "query_values",
    "attend",
    "merge_partials",
    "mla_decode_reference",
    "mla_decode_reference_one",
    "PlanOptions",
    "reference_plan",
    "device_plan_arrays",
    "work_list",
    "status_words",
    "first_task",
    "bf16_bits_to_f32",
    "f32_to_bf16_rne",
    "f32_to_e4m3fn",
    "rope_f32",
    "qcat_cache_insert_reference",
    "gather_kv_b_proj_reference",
    "output_rows",
    "rope_bits",
]
