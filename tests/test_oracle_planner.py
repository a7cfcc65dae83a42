"""Structural pins of the reference planner (CPU only)."""

import numpy as np
import pytest

from oracle import PlanOptions, reference_plan, device_plan_arrays, work_list, first_task
from oracle.planner import STATUS_CTX_TOO_SHORT, STATUS_CTX_TOO_LONG, STATUS_TOO_FEW_PAGES


def _cdiv(a, b):
    return -(-a // b)


SHAPES = [
    # batch, S, H, Lmax
    (2, 1, 16, 100), (64, 1, 128, 8192), (256, 1, 128, 23333), (1, 1, 12, 109440),
    (5, 1, 12, 109440), (128, 4, 16, 5200), (3, 2, 128, 1000), (7, 8, 16, 64), (1, 3, 5, 3),
    (9, 1, 40, 777), (4, 4, 64, 4096), (1, 1, 1, 1),
]


@pytest.mark.parametrize("shape", SHAPES)
def test_plan_structure(shape):
    B, S, H, L = shape
    p = reference_plan(B, S, H, L, num_cu=256, kv_dtype="bf16")
    hpg, G, rows, TR, C = p["heads_per_group"], p["num_groups"], p["rows_per_group"], p["tile_rows"], p["chunk_len"]
    assert 1 <= hpg <= H and hpg * S <= 128 and rows == hpg * S
    assert G * hpg >= H and (G - 1) * hpg < H  # groups cover every head, no empty group
    assert TR in (16, 32, 64, 128) and TR >= rows and (TR == 16 or TR // 2 < rows)
    assert C % 64 == 0 and C >= 64
    assert p["max_chunks"] * C >= L and (p["max_chunks"] - 1) * C < L
    assert p["work_capacity"] == B * p["max_chunks"]
    assert p["num_workgroups"] == 256 * p["wg_per_cu"] and p["grid"] == (p["num_workgroups"], 1, 1)


def test_plan_values_for_the_benchmark_shapes():
    # Hand-derived from the rule with the default options and 256 CUs.
    p = reference_plan(64, 1, 128, 8192, 256, kv_dtype="bf16")
    assert (p["heads_per_group"], p["num_groups"], p["tile_rows"], p["chunk_len"], p["max_chunks"]) == (128, 1, 128, 2048, 4)
    # 16 heads x 4 tokens, 64-row tiles at two workgroups per CU: want = floor(256 * 2 / 128) = 4
    # -> ceil(5200 / 4) = 1300 -> 1344 rows, 4 chunks
    p = reference_plan(128, 4, 16, 5200, 256, kv_dtype="fp8_e4m3fn")
    assert (p["heads_per_group"], p["tile_rows"], p["chunk_len"], p["max_chunks"]) == (16, 64, 1344, 4)
    assert (p["wg_per_cu"], p["num_workgroups"]) == (2, 512)  # 512 chunks, one per persistent workgroup
    # the same shape with a bf16 cache: its 64-row kernel fits one workgroup per CU, so the target of 2
    # is capped at 1: want = 2 -> 2600 -> 2624 rows, 2 chunks
    p = reference_plan(128, 4, 16, 5200, 256, kv_dtype="bf16")
    assert (p["chunk_len"], p["max_chunks"], p["num_workgroups"]) == (2624, 2, 256)
    # small batches of 128 heads at ctx 8192: b = 1: want = 256 -> 32 -> 64 rows (chunk_min), 128 chunks;
    # b = 5: want = 51 -> 161 -> 192 rows, 43 chunks; b = 16: want = 16 -> 512 rows, 16 chunks
    for b, C, n in ((1, 64, 128), (5, 192, 43), (16, 512, 16)):
        p = reference_plan(b, 1, 128, 8192, 256, kv_dtype="fp8_e4m3fn")
        assert (p["tile_rows"], p["chunk_len"], p["max_chunks"]) == (128, C, n), b
    # 256 x 128 heads: want = 1 -> ceil(23333 / 1) rounds to 23360 -> capped at chunk_max = 6144, 4 chunks
    p = reference_plan(256, 1, 128, 23333, 256, kv_dtype="fp8_e4m3fn")
    assert (p["chunk_len"], p["max_chunks"]) == (6144, 4)
    # 12 heads, one sequence: want = 256 -> ceil(109440 / 256) = 428 -> 448 rows, 245 chunks
    p = reference_plan(1, 1, 12, 109440, 256, kv_dtype="fp8_e4m3fn")
    assert (p["tile_rows"], p["chunk_len"], p["max_chunks"]) == (16, 448, 245)
    # five sequences: want = floor(256 / 5) = 51 -> 2146 -> 2176 rows, 51 chunks, 255 workgroups
    # (a ceiling would give 52 -> 2112 rows -> 52 chunks, 260 workgroups on 256 CUs)
    p = reference_plan(5, 1, 12, 109440, 256, kv_dtype="fp8_e4m3fn")
    assert (p["chunk_len"], p["max_chunks"]) == (2176, 51)
    assert 5 * p["max_chunks"] <= 256
    p = reference_plan(2, 1, 16, 100, 256, PlanOptions(force_chunk=64), kv_dtype="bf16")
    assert (p["chunk_len"], p["max_chunks"]) == (64, 2)


@pytest.mark.parametrize("seed", range(5))
def test_device_arrays_tile_every_context_exactly(seed):
    rng = np.random.default_rng(seed)
    B, S, H, P = 37, int(rng.integers(1, 5)), int(rng.integers(1, 130)), int(rng.choice([1, 16, 64]))
    lens = rng.integers(S, 3000, size=B)
    L = int(lens.max())
    indptr = np.concatenate([[0], np.cumsum(_cdiv(lens, P))])
    p = reference_plan(B, S, H, L, 256, PlanOptions(force_chunk=int(rng.choice([0, 64, 192]))), kv_dtype="bf16")
    n, base, status = device_plan_arrays(p, S, L, P, lens, indptr)
    assert status == 0
    C, G = p["chunk_len"], p["num_groups"]
    used = set()
    for b in range(B):
        assert n[b] == _cdiv(int(lens[b]), C) >= 1 and n[b] <= p["max_chunks"]
        starts = [c * C for c in range(n[b])]
        ends = [min((c + 1) * C, int(lens[b])) for c in range(n[b])]
        assert starts[0] == 0 and ends[-1] == lens[b]
        assert all(e > s for s, e in zip(starts, ends)) and all(e == s2 for e, s2 in zip(ends, starts[1:]))
        if n[b] > 1:
            recs = {base[b] + g * n[b] + c for g in range(G) for c in range(n[b])}
            assert not (recs & used) and len(recs) == G * n[b]
            used |= recs
    assert max(used, default=-1) < p["partial_capacity_records"]


def test_device_status_bits():
    p = reference_plan(4, 2, 8, 100, 256, kv_dtype="bf16")
    lens = [1, 101, 50, 50]
    indptr = [0, 1, 102, 103, 153]  # seq 2 has 1 page of size 1 for 50 rows
    n, base, status = device_plan_arrays(p, 2, 100, 1, lens, indptr)
    assert status == STATUS_CTX_TOO_SHORT | STATUS_CTX_TOO_LONG | STATUS_TOO_FEW_PAGES
    assert n[:3] == [0, 0, 0] and n[3] == _cdiv(50, p["chunk_len"])


def test_work_list_hand_example():
    # C = 64: ctx 200 -> chunks of 64, 64, 64, 8 (last: class 16*8//64 = 2);
    # ctx 64 -> one full chunk; ctx 100 -> 64 + 36 (class 9); ctx 0 < S -> invalid;
    # ctx 120 -> 64 + 56 (class 14)
    plan = reference_plan(5, 1, 16, 200, 256, PlanOptions(force_chunk=64), kv_dtype="bf16")
    lens = [200, 64, 100, 0, 120]
    n, _, status = device_plan_arrays(plan, 1, 200, 1, lens, [0, 200, 264, 364, 364, 484])
    assert n == [4, 1, 2, 0, 2] and status == 1
    assert work_list(plan, n, lens) == [(0, 0), (0, 1), (0, 2), (1, 0), (2, 0), (4, 0),
                                        (4, 1), (2, 1), (0, 3), (3, -1)]


@pytest.mark.parametrize("seed", range(6))
def test_work_list_covers_every_chunk_once_longest_first(seed):
    rng = np.random.default_rng(100 + seed)
    B, S = int(rng.integers(1, 300)), int(rng.integers(1, 5))
    L = int(rng.integers(S, 6000))
    lens = rng.integers(0, L + 1, size=B)
    plan = reference_plan(B, S, 16, L, 256, PlanOptions(force_chunk=int(rng.choice([0, 64, 256, 1024]))), kv_dtype="bf16")
    C = plan["chunk_len"]
    indptr = np.concatenate([[0], np.cumsum(lens)])  # page size 1: one page per row
    n, _, _ = device_plan_arrays(plan, S, L, 1, lens, indptr)
    items = work_list(plan, n, lens)
    assert len(items) <= plan["work_capacity"]
    want = {(b, c) for b in range(B) for c in range(n[b])} | {(b, -1) for b in range(B) if n[b] == 0}
    assert len(items) == len(want) and set(items) == want
    # dispatch order: class (full chunk 16, partial floor(16 r / C), invalid -1) never rises,
    # and within a class the items follow (sequence, chunk) order
    keys = []
    for b, c in items:
        r = -1 if c < 0 else min(C, int(lens[b]) - c * C)
        keys.append((-1 if r < 0 else 16 * r // C, b, c))
    assert all(keys[i][0] >= keys[i + 1][0] for i in range(len(keys) - 1))
    assert all(keys[i][1:] < keys[i + 1][1:] for i in range(len(keys) - 1) if keys[i][0] == keys[i + 1][0])


def test_first_tasks_are_a_permutation_keeping_consecutive_tasks_on_one_xcd():
    for W in (256, 512, 24, 7, 1):
        ts = [first_task(x, W) for x in range(W)]
        assert sorted(ts) == list(range(W))
        if W % 8 == 0:
            # workgroups x and x + 8 run on one XCD (the hardware deals them out in turn)
            # and take consecutive tasks: the head groups and chunks of one sequence
            assert all(ts[x + 8] == ts[x] + 1 for x in range(W - 8))


def _simulate_counter(items_len, W, durations):
    """Tasks handed out as the library's persistent workgroups take them: workgroup x first
    runs first_task(x), then whichever workgroup frees up first takes the next task of the
    list. Returns each workgroup's busy time."""
    import heapq
    busy = [0.0] * W
    free = []
    for x in range(W):
        t = first_task(x, W)
        if t < items_len:
            busy[x] = durations[t]
            heapq.heappush(free, (busy[x], x))
    nxt = W
    while nxt < items_len and free:
        when, x = heapq.heappop(free)
        busy[x] = when + durations[nxt]
        heapq.heappush(free, (busy[x], x))
        nxt += 1
    return busy


def test_longest_first_hand_out_balances_the_ragged_batch():
    # the ragged 128-head batch (lengths as the benchmark draws them): with the list longest
    # first and tasks handed out as workgroups free up, the busiest workgroup does at most 5%
    # more rows than the mean
    rng = np.random.default_rng([3, 3])
    lens = rng.integers(21, 23333, size=256, endpoint=True)
    plan = reference_plan(256, 1, 128, int(lens.max()), 256, kv_dtype="fp8_e4m3fn")
    C = plan["chunk_len"]
    n, _, _ = device_plan_arrays(plan, 1, int(lens.max()), 64, lens, np.concatenate([[0], np.cumsum(-(-lens // 64))]))
    items = work_list(plan, n, lens)
    rows = [min(C, int(lens[b]) - c * C) for b, c in items]
    busy = _simulate_counter(len(items), plan["num_workgroups"], rows)
    assert max(busy) <= 1.05 * sum(rows) / plan["num_workgroups"]
