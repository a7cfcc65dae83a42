"""Reference work planner for split-KV MLA decode (test infrastructure).

An independent Python statement of the plan rule, used to check the library's
host planner (plan fields) and device planner (per-sequence arrays, status
words and the work list) bit for bit. It shares no code with the library;
nothing in the library imports it.

Where the rule comes from:

* "perf(mla): chunk the non-FP4 gather_kv_b_proj over KV" (description): the
  serial walk over the context becomes a set of KV chunks sized from the
  longest sequence; no program works past its own sequence's end, so ragged
  batches stay correct. Too few programs starve HBM (12 workgroups on a 256-CU
  part).
* "HK MLA: MI35x m16x8 retune, new m16x4 kernel, page_size + mask support"
  (Summary and file table): the decode kernel is persistent; device-built
  metadata sizes its grid for ``num_cu`` clusters, or twice that when the
  64-row kernel runs at occupancy 2; heads times query tokens are stacked into
  one tile of rows (64 or 128).

The rule (all integer arithmetic):

    hpg  = min(H, 128 // S)            heads per group (rows = hpg * S <= 128)
    G    = ceil(H / hpg)               head groups
    rows = hpg * S                     valid rows of a tile
    TR   = 16 | 32 | 64 | 128          smallest of these >= rows; class = log2(TR/16)
    occ  = min(wg_per_cu[cls], fit[kv_dtype][cls])
           (fit: workgroups of that class's decode kernel one CU holds)
    W    = num_cu * occ                persistent workgroups: the decode grid
    C    = force_chunk if set, else
           clamp(roundup(ceil(Lmax / want), 64), chunk_min[cls], chunk_max[cls])
           with want = max(1, floor(W / (B * G)))
    max_chunks = ceil(Lmax / C)
    work_capacity = B * max_chunks     entries of the work list

Per sequence (device half): a sequence is valid when ``S <= ctx_b <= Lmax`` and
its page list holds at least ``ceil(ctx_b / P)`` pages; then
``n_b = ceil(ctx_b / C)``, else ``n_b = 0`` and a status bit is set.
``part_base_b`` is the exclusive prefix sum over ``b`` of
``(n_b if n_b > 1 else 0) * G``: partial records of sequence b, group g, chunk c
sit at record ``part_base_b + g * n_b + c``.

Work list (a design choice of this library, not from the pages): items
(sequence, chunk), longest work first so that the last tasks a workgroup takes
are short. Every full chunk (exactly C rows) in (sequence, chunk) order; then
each sequence's partial last chunk (length r = ctx - (n - 1) * C < C), by length
class floor(16 * r / C) from the longest class down, ties by sequence; then one
item (sequence, -1) per invalid sequence, whose rows are filled with NaN.

Tasks and workgroups: task t is item t // G for head group t % G. Workgroup x
of the persistent grid first runs task first_task(x, W) (consecutive tasks on
one XCD: the hardware deals workgroups to the 8 XCDs in turn, so the groups
and chunks of one sequence share an L2), then takes the next untaken task from
a counter, in list order, as each task's last block starts, until none is
left: so a workgroup takes more work when it is about to be free, in
longest-first order, whatever the order in which the hardware starts
workgroups. Status words after the plan (and after every decode call): (OR of
the status bits, item count, W = the counter's start, 0).
"""

from dataclasses import dataclass, field
from typing import List

BLOCK_ROWS = 64  # chunk lengths are multiples of this many cache rows
MAX_TILE_ROWS = 128
TILE_CLASSES = (16, 32, 64, 128)

STATUS_CTX_TOO_SHORT = 1  # context_lens[b] < seqlen_qo
STATUS_CTX_TOO_LONG = 2  # context_lens[b] > max_context_len
STATUS_TOO_FEW_PAGES = 4  # page list shorter than ceil(ctx / page_size)
LENGTH_CLASSES = 16  # partial last chunks are dispatched by length class, longest first


def _cdiv(a: int, b: int) -> int:
    return -(-a // b)


# workgroups per CU that the decode kernel of each cache type and tile class fits
# (its LDS footprint); the target wg_per_cu is capped at it
KERNEL_WG_PER_CU = {"bf16": [1, 1, 1, 1], "fp8_e4m3fn": [1, 1, 2, 1]}
NUM_XCD = 8


@dataclass
class PlanOptions:
    wg_per_cu: List[int] = field(default_factory=lambda: [1, 1, 2, 1])
    chunk_min: List[int] = field(default_factory=lambda: [256, 256, 256, 64])
    chunk_max: List[int] = field(default_factory=lambda: [8192, 8192, 4096, 6144])
    force_chunk: int = 0


def reference_plan(batch, seqlen_qo, num_heads, max_context_len, num_cu, options=None, *, kv_dtype):
    """Plan fields for one call shape and cache type ("bf16" or "fp8_e4m3fn"). Returns a dict;
    see the module docstring."""
    o = options or PlanOptions()
    B, S, H, L = int(batch), int(seqlen_qo), int(num_heads), int(max_context_len)
    hpg = min(H, MAX_TILE_ROWS // S)
    G = _cdiv(H, hpg)
    rows = hpg * S
    TR = next(t for t in TILE_CLASSES if t >= rows)
    cls = TILE_CLASSES.index(TR)
    occ = min(o.wg_per_cu[cls], KERNEL_WG_PER_CU[kv_dtype][cls])
    W = int(num_cu) * occ
    if o.force_chunk:
        C = int(o.force_chunk)
    else:
        want = max(1, W // (B * G))
        C = _cdiv(_cdiv(L, want), BLOCK_ROWS) * BLOCK_ROWS
        C = min(max(C, o.chunk_min[cls]), o.chunk_max[cls])
    max_chunks = _cdiv(L, C)
    return {
        "work_capacity": B * max_chunks,
        "heads_per_group": hpg,
        "num_groups": G,
        "rows_per_group": rows,
        "tile_rows": TR,
        "tile_class": cls,
        "chunk_len": C,
        "max_chunks": max_chunks,
        "wg_per_cu": occ,
        "num_workgroups": W,
        "grid": (W, 1, 1),
        "partial_capacity_records": B * G * max_chunks,
    }


def device_plan_arrays(plan, seqlen_qo, max_context_len, page_size, context_lens, kv_indptr):
    """Per-sequence chunk counts, partial bases and the status bits (device half)."""
    S, L, P = int(seqlen_qo), int(max_context_len), int(page_size)
    C, G = plan["chunk_len"], plan["num_groups"]
    n_chunks, part_base = [], []
    status = 0
    running = 0
    for b, ctx in enumerate(context_lens):
        ctx = int(ctx)
        pages = int(kv_indptr[b + 1]) - int(kv_indptr[b])
        bad = 0
        if ctx < S:
            bad |= STATUS_CTX_TOO_SHORT
        if ctx > L:
            bad |= STATUS_CTX_TOO_LONG
        if not bad and pages < _cdiv(ctx, P):
            bad |= STATUS_TOO_FEW_PAGES
        status |= bad
        n = 0 if bad else _cdiv(ctx, C)
        n_chunks.append(n)
        part_base.append(running)
        running += (n if n > 1 else 0) * G
    return n_chunks, part_base, status


def work_list(plan, n_chunks, context_lens):
    """Work items (sequence, chunk) in dispatch order; chunk -1 marks an invalid sequence."""
    C = plan["chunk_len"]
    full, partial, invalid = [], [], []
    for b, (n, ctx) in enumerate(zip(n_chunks, context_lens)):
        n, ctx = int(n), int(ctx)
        if n == 0:
            invalid.append((b, -1))
            continue
        last = ctx - (n - 1) * C  # rows of the last chunk, 1..C
        n_full = n if last == C else n - 1
        full.extend((b, c) for c in range(n_full))
        if last < C:
            partial.append((LENGTH_CLASSES * last // C, b, n - 1))
    partial.sort(key=lambda t: (-t[0], t[1]))
    return full + [(b, c) for _, b, c in partial] + invalid


def status_words(plan, status_bits, n_items):
    """The four status words the planner writes (and every decode call leaves behind)."""
    return [int(status_bits), int(n_items), plan["num_workgroups"], 0]


def first_task(x, num_workgroups):
    """The task workgroup x of the persistent grid runs first (a permutation of [0, W))."""
    W = int(num_workgroups)
    if W % NUM_XCD:
        return x
    return (x % NUM_XCD) * (W // NUM_XCD) + x // NUM_XCD
