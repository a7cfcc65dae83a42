"""Benchmark: MLA decode over a paged latent cache on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]
    python bench.py --copy-probe     (a plain 1 GiB device copy, to scale the HBM byte counters)
    python bench.py --workload insert_t64_h8_fp8   (the decode epilogue: query concat + cache insert)
    python bench.py --workload kvb_b1_h12_ctx109440_fp8   (the cached-prefix gather_kv_b_proj)

One step = one call of the hot path (mla_decode + mla_split_combine) over the
whole batch, inputs resident in HBM. Between steps a 1 GiB buffer is read
(outside the timed events) so that neither L2 nor the 256 MB MALL holds the
previous call's cache rows, as in serving where other layers run in between.
The flush reads rather than writes: a write leaves ~256 MB of dirty lines whose
write-back would compete with the next call's reads. Prints one JSON line.

The default run (the dense batch-64 workload) also measures every other decode
workload of the suite the same way, with fewer calls each, and reports them in
the line's "configs" object: µs per call, decode and merge kernel times, the
device planner's time (event pair around one plan launch; the plan is made once
per batch composition and shared by every layer, so it is not part of a call),
the roofline bound and fraction per call and per decode launch, and the
counter-measured traffic over the algorithmic bytes where a current profile is
committed. --no-configs skips them.

Roofline accounting (per decode launch):
  algorithmic bytes = sum_b ctx_b * 576 * e (each cache row read once; e = 2 bf16, 1 fp8)
                      + B*S*H*576*eq (q; eq = 2 bf16, 1 fp8) + B*S*H*512*2 (out) + 4*(B+1) + 4*pages + 4*B (page table, lengths)
  algorithmic flops = 2 * H * (visible row visits) * (576 + 512)
against 8 TB/s HBM and 2.5 PFLOP/s dense bf16 MFMA. roofline.traffic is the HBM
rate implied by the rocprofv3 FETCH_SIZE + WRITE_SIZE counters of the decode
kernel recorded under profiles/ for this workload, taken only while the kernel
sources still hash to the value recorded with them (else null).
"""

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)
CSRC = os.path.join(ROOT, "mla_paged_latent_02_amd", "csrc")
PROFILES = os.path.join(ROOT, "profiles")

HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0
DEFAULT_WORKLOAD = "dense_b64_h128_ctx8192_bf16"
METRIC = "MLA decode µs/call + HBM TB/s & MFMA % peak, 128 heads ctx 8192 batch 64"


def algorithmic_counts(case):
    import numpy as np
    e = 2 if case.kv_dtype == "bf16" else 1
    eq = 2 if case.q_dtype == "bf16" else 1
    ctx = case.context_lens.astype(np.int64)
    B, S, H = case.batch, case.seqlen_qo, case.num_heads
    rows = int(ctx.sum())
    nbytes = rows * 576 * e + B * S * H * 576 * eq + B * S * H * 512 * 2 + 4 * (B + 1) + 4 * int(case.kv_indptr[-1]) + 4 * B
    if case.causal:
        visits = int(sum(int(c) - S + 1 + s for c in ctx for s in range(S)))
    else:
        visits = rows * S
    flops = 2 * H * visits * (576 + 512)
    return nbytes, flops


# The sources that make up the decode path (planner, decode and merge kernels, their launch code);
# the epilogue and the cached-prefix expansion live in files of their own and are not part of it.
DECODE_SOURCES = ("mla_api.cpp", "mla_internal.h", "mla_kernels.hip", "mla_plan.cpp")
KVB_SOURCES = ("mla_internal.h", "mla_kv_b_proj.hip")
INSERT_SOURCES = ("mla_internal.h", "mla_insert.hip")


def source_digest(names=DECODE_SOURCES):
    """First 16 hex digits of the sha256 over the named C/HIP sources of the library."""
    import hashlib
    h = hashlib.sha256()
    for path in [os.path.join(CSRC, n) for n in names]:
        h.update(os.path.basename(path).encode())
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def kernel_source_digest():
    """The decode path's source digest."""
    return source_digest(DECODE_SOURCES)


def recorded_fields(name, digest):
    """The "- key: value" fields of a committed profile summary, if it was taken at these sources."""
    import re
    path = os.path.join(PROFILES, name)
    if not os.path.exists(path):
        return None
    with open(path) as f:
        fields = dict(re.findall(r"^- (\w+): (\S+)\s*$", f.read(), flags=re.M))
    return fields if fields.get("kernel_source_sha256_16") == digest else None


def recorded_traffic(workload):
    """HBM bytes per decode launch from the committed counter summary, if it matches these sources."""
    f = recorded_fields(f"mla_decode_kernel_{workload}_hbm_traffic.md", kernel_source_digest())
    return None if f is None else float(f["hbm_bytes_per_launch"])


def recorded_mfma_busy(kernel, workload, digest):
    """MFMA-busy percentage (rocprofv3 MfmaUtil) from the committed counter summary, if current."""
    f = recorded_fields(f"{kernel}_{workload}_mfma_lds.md", digest)
    return None if f is None else float(f["mfma_busy_pct"])


def copy_probe(nbytes=1 << 30, reps=3):
    """A plain device-to-device copy of known size: FETCH_SIZE / WRITE_SIZE of this kernel scale the counters."""
    import torch
    src = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes": nbytes, "reps": reps}), flush=True)


def cpu_baseline(case, min_s=10.0, max_s=30.0):
    """The oracle as it stands, timed on a bounded sample: sequences of the batch in order, cycling
    through the batch again until at least min_s of oracle work (or max_s) has run; scaled by cache rows."""
    import numpy as np
    import oracle
    cores = len(os.sched_getaffinity(0))
    secs, rows_done, evals = 0.0, 0, 0
    while secs < min_s and (secs < max_s or evals == 0):
        b = evals % case.batch
        s0 = time.perf_counter()
        oracle.mla_decode_reference_one(case.q_bits, case.cache_raw, case.kv_dtype, case.kv_scale, case.kv_indptr,
                                        case.kv_page_indices, case.context_lens, case.page_size,
                                        case.softmax_scale, case.causal, b, q_scale=case.q_scale)
        secs += time.perf_counter() - s0
        rows_done += int(case.context_lens[b])
        evals += 1
    rows_all = int(case.context_lens.astype(np.int64).sum())
    per_call_us = secs * rows_all / rows_done * 1e6
    return {"value": per_call_us, "unit": "us", "cores": cores, "kind": "oracle",
            "sample": f"{evals} sequence evaluations over a batch of {case.batch} ({rows_done} cache rows, "
                      f"{secs:.1f} s), scaled by cache rows to one full call; float64 numpy, BLAS threads = {cores}"}


def insert_bench(args):
    """The decode epilogue (mla_qcat_cache_insert) on one workload: one call per step,
    inputs resident, the same read flush between steps. Algorithmic bytes per call:
    query parts read and written (T*H*576*2 each), latent rows read (T*576*2), one
    rope-table row, position and slot per token, cache rows written (576*e per token
    with a slot)."""
    import numpy as np
    import torch

    import mla_paged_latent_02_amd as mla
    import oracle
    from mla_synth import INSERT_WORKLOADS, make_insert_case

    c = make_insert_case(**INSERT_WORKLOADS[args.workload])
    torch.cuda.set_device(0)

    def dev(a):
        a = np.ascontiguousarray(a)
        return torch.from_numpy(a.view(np.int16) if a.dtype == np.uint16 else a).to("cuda")

    ins = [dev(x) for x in (c.ql_nope, c.q_pe, c.kv_c, c.k_pe, c.positions, c.cos_sin, c.slot_mapping)]
    q = torch.empty((c.num_tokens, c.num_heads, 576), dtype=torch.int16, device="cuda")
    cache = dev(c.cache)
    p = mla.make_insert_params(num_tokens=c.num_tokens, num_heads=c.num_heads, kv_dtype=c.kv_dtype,
                               kv_scale=c.kv_scale, num_slots=c.num_slots, rope_positions=c.rope_positions,
                               rope_neox=c.neox)
    stream = torch.cuda.current_stream()
    flush = None if args.no_flush else torch.ones(1 << 28, dtype=torch.float32, device="cuda")
    sink = torch.empty((), dtype=torch.float32, device="cuda")
    for _ in range(args.warmup):
        mla.qcat_cache_insert(p, *ins, q, cache, None, stream)
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
    for k in range(args.steps):
        if flush is not None:
            torch.sum(flush, dim=0, out=sink)
        ev[k][0].record(stream)
        mla.qcat_cache_insert(p, *ins, q, cache, None, stream)
        ev[k][1].record(stream)
    torch.cuda.synchronize()
    ms = np.array([e[0].elapsed_time(e[1]) for e in ev])
    T, H = c.num_tokens, c.num_heads
    e = 2 if c.kv_dtype == "bf16" else 1
    written = int((c.slot_mapping >= 0).sum())
    nbytes = 2 * T * H * 576 * 2 + T * 576 * 2 + T * (256 + 4 + 8) + written * 576 * e
    us = float(np.mean(ms) * 1e3)
    gbs = nbytes / (us * 1e-6) / 1e9
    tf = recorded_fields(f"mla_insert_kernel_{args.workload}_hbm_traffic.md", source_digest(INSERT_SOURCES))
    insert_traffic = None if tf is None else float(tf["hbm_bytes_per_launch"]) / (us * 1e-6) / 1e9
    cpu = None
    if not args.no_cpu_baseline:
        t0, n = time.perf_counter(), 0
        while time.perf_counter() - t0 < 10.0:
            oracle.qcat_cache_insert_reference(c.ql_nope, c.q_pe, c.kv_c, c.k_pe, c.positions, c.cos_sin,
                                               c.slot_mapping, c.cache, c.kv_dtype, c.kv_scale, c.neox)
            n += 1
        cpu = {"value": (time.perf_counter() - t0) / n * 1e6, "unit": "us", "cores": 1, "kind": "oracle",
               "sample": f"{n} full calls of the numpy oracle (one thread, per-token loop), mean"}
    print(json.dumps({
        "metric": "MLA decode epilogue (query concat + latent-cache insert) µs/call", "value": us, "unit": "us",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": us / 1e3,
        "higher_is_better": False, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16 query, " + ("bf16" if e == 2 else "fp8-e4m3fn") + " cache", "data": "synthetic",
        "config": {"workload": args.workload, "tokens": T, "heads": H, "kv_dtype": c.kv_dtype,
                   "rope_neox": c.neox, "tokens_with_slot": written},
        "call_us_p10_p50_p90": [float(np.percentile(ms, x) * 1e3) for x in (10, 50, 90)],
        "flush_between_steps": flush is not None,
        "roofline": {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": gbs / HBM_PEAK_GBS, "traffic": insert_traffic, "kernel": "mla_insert_kernel",
                     "kernel_source_sha256_16": source_digest(INSERT_SOURCES),
                     "alg_bytes": nbytes, "note": "event pair around one launch; includes the launch gap"},
        "cpu_baseline": cpu,
    }), flush=True)


# The pages' timings of this kernel on MI355X after the KV-chunk grid, in ms
# ("perf(mla): chunk the non-FP4 gather_kv_b_proj over KV", ctx table).
KVB_PAGE_MS = {4096: 0.038, 32000: 0.227, 65536: 0.442, 109440: 0.711}


def kvb_bench(args):
    """The cached-prefix expansion (mla_gather_kv_b_proj) on one workload: one call per
    step, inputs resident, the same read flush between steps. Per call, over N cached
    rows and H heads: algorithmic flops 2*N*H*256*512; algorithmic bytes N*576*e
    (latent rows read once) + N*H*(192 + 128)*2 (K and V written) + H*256*512*2 (W)
    + 4*(2B + 2 + pages) (page table and row offsets)."""
    import numpy as np
    import torch

    import mla_paged_latent_02_amd as mla
    import oracle
    from mla_synth import KVB_WORKLOADS, make_kvb_case

    c = make_kvb_case(name=args.workload, **KVB_WORKLOADS[args.workload])
    torch.cuda.set_device(0)

    def dev(a):
        a = np.ascontiguousarray(a)
        return torch.from_numpy(a.view(np.int16) if a.dtype == np.uint16 else a).to("cuda")

    N, H = c.total_rows, c.num_heads
    ins = [dev(x) for x in (c.cache_raw, c.kv_indptr, c.kv_page_indices, c.cu_ctx, c.w_bits)]
    k = torch.empty((N, H, 192), dtype=torch.int16, device="cuda")
    v = torch.empty((N, H, 128), dtype=torch.int16, device="cuda")
    p = mla.make_kv_b_proj_params(batch=c.batch, num_heads=H, page_size=c.page_size, kv_dtype=c.kv_dtype,
                                  kv_scale=c.kv_scale, max_context_len=c.max_context_len, num_slots=c.num_slots,
                                  num_out_rows=N)
    stream = torch.cuda.current_stream()
    flush = None if args.no_flush else torch.ones(1 << 28, dtype=torch.float32, device="cuda")
    sink = torch.empty((), dtype=torch.float32, device="cuda")
    for _ in range(args.warmup):
        mla.gather_kv_b_proj(p, *ins, k, v, None, stream)
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
    for s in range(args.steps):
        if flush is not None:
            torch.sum(flush, dim=0, out=sink)
        ev[s][0].record(stream)
        mla.gather_kv_b_proj(p, *ins, k, v, None, stream)
        ev[s][1].record(stream)
    torch.cuda.synchronize()
    ms = np.array([e[0].elapsed_time(e[1]) for e in ev])
    us = float(np.mean(ms) * 1e3)
    e = 2 if c.kv_dtype == "bf16" else 1
    flops = 2.0 * N * H * 256 * 512
    nbytes = N * 576 * e + N * H * (192 + 128) * 2 + H * 256 * 512 * 2 + 4 * (2 * c.batch + 2 + len(c.kv_page_indices))
    tf = flops / (us * 1e-6) / 1e12
    gbs = nbytes / (us * 1e-6) / 1e9
    t_mfma, t_hbm = flops / (MFMA_BF16_PEAK_TFLOPS * 1e12), nbytes / (HBM_PEAK_GBS * 1e9)
    if t_mfma >= t_hbm:
        roof = {"bound": "mfma", "achieved": tf, "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": tf / MFMA_BF16_PEAK_TFLOPS}
    else:
        roof = {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": gbs / HBM_PEAK_GBS}
    kd = source_digest(KVB_SOURCES)
    tf_fields = recorded_fields(f"mla_kv_b_proj_kernel_{args.workload}_hbm_traffic.md", kd)
    traffic = None if tf_fields is None else float(tf_fields["hbm_bytes_per_launch"]) / (us * 1e-6) / 1e9
    roof.update({"traffic": traffic, "kernel": "mla_kv_b_proj_kernel", "alg_bytes": nbytes, "alg_flops": flops,
                 "hbm_gbs": gbs, "kernel_source_sha256_16": kd,
                 "mfma_busy_pct_counter": recorded_mfma_busy("mla_kv_b_proj_kernel", args.workload, kd),
                 "note": "event pair around one launch; includes the launch gap"})
    cpu = None
    if not args.no_cpu_baseline:
        t0, done = time.perf_counter(), 0
        while time.perf_counter() - t0 < 10.0 and done < N:
            b0 = done
            n = min(8192, N - b0)
            rows = [r for r in oracle.output_rows(c.cu_ctx)[b0:b0 + n]]
            oracle.gather_kv_b_proj_reference(c.cache_raw, c.kv_dtype, c.kv_scale, c.kv_indptr, c.kv_page_indices,
                                              c.cu_ctx, c.page_size, c.w_bits, rows=[(b, r) for b, r, _ in rows])
            done += n
        el = time.perf_counter() - t0
        cpu = {"value": el / done * N * 1e6, "unit": "us", "cores": len(os.sched_getaffinity(0)), "kind": "oracle",
               "sample": f"first {done} of {N} cached rows through the numpy fp64 oracle (dgemm on all cores), "
                         "time scaled to the full call"}
    ctx = int(c.context_lens.max())
    page_ms = KVB_PAGE_MS.get(ctx) if c.batch == 1 and c.page_size == 1 and H == 12 else None
    print(json.dumps({
        "metric": "MLA cached-prefix gather_kv_b_proj µs/call", "value": us, "unit": "us",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": us / 1e3,
        "higher_is_better": False, "scaling": "weak",
        "vs_baseline": (us / (page_ms * 1e3)) if page_ms else None,
        "pages_us_mi355x": page_ms * 1e3 if page_ms else None,
        "dtype": ("bf16" if e == 2 else "fp8-e4m3fn") + " cache widened to bf16; bf16 MFMA, fp32 accumulation",
        "data": "synthetic",
        "config": {"workload": args.workload, "batch": c.batch, "heads": H, "cached_rows": N,
                   "page_size": c.page_size, "kv_dtype": c.kv_dtype},
        "call_us_p10_p50_p90": [float(np.percentile(ms, x) * 1e3) for x in (10, 50, 90)],
        "flush_between_steps": flush is not None,
        "roofline": roof,
        "cpu_baseline": cpu,
    }), flush=True)


# The workloads of the per-config lines (one each; the headline workload is the
# dense batch-64 one above): the tiny two-sequence case, the ragged 256-sequence
# fp8 batch, the long-context 12-head fp8 decode at batch 1 to 5, and the causal
# four-token decode.
CONFIG_WORKLOADS = ("tiny_b2_h16", "ragged_b256_h128_fp8_p64",
                    *[f"longctx_b{b}_h12_ctx109440_fp8" for b in range(1, 6)],
                    "causal_mtp4_b128_h16_ctx5200_fp8_p16")


def upload_case(case):
    from mla_paged_latent_02_amd.device import DeviceInputs
    return DeviceInputs.from_host(
        q_bits=case.q_bits, cache_raw=case.cache_raw, kv_indptr=case.kv_indptr,
        kv_page_indices=case.kv_page_indices, context_lens=case.context_lens, batch=case.batch,
        seqlen_qo=case.seqlen_qo, num_heads=case.num_heads, page_size=case.page_size,
        max_context_len=case.max_context_len, causal=case.causal, kv_dtype=case.kv_dtype,
        softmax_scale=case.softmax_scale, kv_scale=case.kv_scale, num_slots=case.num_slots,
        q_dtype=case.q_dtype, q_scale=case.q_scale)


def roofline_for(nbytes, flops, seconds):
    """The bound the workload's arithmetic intensity puts it under, and the fraction of that peak reached."""
    ridge = MFMA_BF16_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9)
    if flops / nbytes < ridge:
        gbs = nbytes / seconds / 1e9
        return {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": gbs / HBM_PEAK_GBS}
    tf = flops / seconds / 1e12
    return {"bound": "mfma", "achieved": tf, "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
            "frac": tf / MFMA_BF16_PEAK_TFLOPS}


def measure_decode(case, workload, steps, warmup, use_flush, plan_reps=20, warm_s=0.0):
    """Times one workload: plan (device launch, event pairs), then `steps` calls of decode + merge with a
    read flush before each. After the `warmup` calls, untimed calls continue until `warm_s` seconds have
    passed (the per-config lines follow an idle stretch of the GPU, whose clocks then take a while to
    come back up). Returns the raw measurements and derived rates as a dict."""
    import numpy as np
    import torch

    import mla_paged_latent_02_amd as mla
    from mla_paged_latent_02_amd.device import Decoder

    inp = upload_case(case)
    stream = torch.cuda.current_stream()
    t0 = time.perf_counter()
    dec = Decoder(inp, None, 0, stream)
    torch.cuda.synchronize()
    plan_wall_us = (time.perf_counter() - t0) * 1e6
    # the planner re-run on the same workspace writes the same arrays; each run is one device launch
    plan_ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(plan_reps)]
    for e in plan_ev:
        e[0].record(stream)
        mla.decode_plan(inp.params, inp.context_lens, inp.kv_indptr, dec.workspace, None, 0, stream)
        e[1].record(stream)
    torch.cuda.synchronize()
    plan_us = float(np.mean([e[0].elapsed_time(e[1]) for e in plan_ev]) * 1e3)

    flush = torch.ones(1 << 28, dtype=torch.float32, device="cuda") if use_flush else None
    sink = torch.empty((), dtype=torch.float32, device="cuda")

    def step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        mla.decode(dec.plan, inp.q, inp.cache, inp.kv_indptr, inp.kv_page_indices, inp.context_lens, dec.out,
                   dec.lse, dec.workspace, stream)
        if ev is not None:
            ev[1].record(stream)
        mla.split_combine(dec.plan, dec.workspace, dec.out, dec.lse, stream)
        if ev is not None:
            ev[2].record(stream)

    for _ in range(warmup):
        if flush is not None:
            torch.sum(flush, dim=0, out=sink)
        step()
    torch.cuda.synchronize()
    t_warm = time.perf_counter()
    while time.perf_counter() - t_warm < warm_s:
        for _ in range(5):
            if flush is not None:
                torch.sum(flush, dim=0, out=sink)
            step()
        torch.cuda.synchronize()
    # Timed loop 1 (the reported value): one event pair around each whole call, nothing in between.
    call_ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(steps)]
    wall0 = time.perf_counter()
    for k in range(steps):
        if flush is not None:
            torch.sum(flush, dim=0, out=sink)
        call_ev[k][0].record(stream)
        step()
        call_ev[k][1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    call_ms = np.array([e[0].elapsed_time(e[1]) for e in call_ev])
    # Timed loop 2 (the roofline): a third event between the decode and the merge, so that each
    # kernel has its own duration; the extra event adds a few µs of gap to each call.
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    for k in range(steps):
        if flush is not None:
            torch.sum(flush, dim=0, out=sink)
        step(events[k])
    torch.cuda.synchronize()
    dec_ms = np.array([e[0].elapsed_time(e[1]) for e in events])
    comb_ms = np.array([e[1].elapsed_time(e[2]) for e in events])
    del dec, inp, flush
    torch.cuda.empty_cache()

    nbytes, flops = algorithmic_counts(case)
    call_us = float(np.mean(call_ms) * 1e3)
    dec_us = float(np.mean(dec_ms) * 1e3)
    traffic_bytes = recorded_traffic(workload)
    return {
        "call_us": call_us, "call_ms_all": call_ms, "wall_s": wall,
        "decode_us": dec_us, "combine_us": float(np.mean(comb_ms) * 1e3),
        "call_us_p10_p50_p90": [float(np.percentile(call_ms, q) * 1e3) for q in (10, 50, 90)],
        "plan_us": plan_us, "plan_wall_us_first_call": plan_wall_us,
        "alg_bytes": nbytes, "alg_flops": flops,
        "per_call": roofline_for(nbytes, flops, call_us * 1e-6),
        "decode": roofline_for(nbytes, flops, dec_us * 1e-6),
        "traffic_bytes_per_launch": traffic_bytes,
        "traffic_over_alg_bytes": None if traffic_bytes is None else traffic_bytes / nbytes,
    }


def config_summary(case, m):
    """The compact per-config record of the default run."""
    pc, d = m["per_call"], m["decode"]
    return {
        "batch": case.batch, "heads": case.num_heads, "seqlen_qo": case.seqlen_qo,
        "max_ctx": case.max_context_len, "page_size": case.page_size, "kv_dtype": case.kv_dtype,
        "causal": case.causal, "us_per_call": m["call_us"], "call_us_p50": m["call_us_p10_p50_p90"][1],
        "decode_us": m["decode_us"], "combine_us": m["combine_us"], "plan_us": m["plan_us"],
        "bound": pc["bound"], "frac_per_call": pc["frac"], "frac_decode": d["frac"],
        "achieved_per_call": pc["achieved"], "unit": pc["unit"],
        "hbm_tb_per_s_per_call": m["alg_bytes"] / (m["call_us"] * 1e-6) / 1e12,
        "alg_bytes": m["alg_bytes"], "alg_flops": m["alg_flops"],
        "counter_traffic_over_alg_bytes": m["traffic_over_alg_bytes"],
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-flush", action="store_true")
    ap.add_argument("--no-configs", action="store_true", help="skip the per-config lines of the other workloads")
    ap.add_argument("--config-steps", type=int, default=30, help="timed calls per config of the per-config lines")
    ap.add_argument("--copy-probe", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only: this decode path has no multi-GPU mode (asked for --gpus {args.gpus})",
              file=sys.stderr)
        sys.exit(2)

    if args.copy_probe:
        copy_probe()
        return
    if args.workload.startswith("insert_"):
        insert_bench(args)
        return
    if args.workload.startswith("kvb_"):
        kvb_bench(args)
        return

    if not args.no_cpu_baseline:
        n = str(len(os.sched_getaffinity(0)))
        for var in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS"):
            os.environ[var] = n

    import torch

    from mla_synth import WORKLOADS, make_case

    torch.cuda.set_device(0)
    case = make_case(**WORKLOADS[args.workload])
    m = measure_decode(case, args.workload, args.steps, args.warmup, not args.no_flush)

    roof = dict(m["decode"])
    roof["traffic"] = (None if m["traffic_bytes_per_launch"] is None
                       else m["traffic_bytes_per_launch"] / (m["decode_us"] * 1e-6) / 1e9)
    roof["traffic_bytes_per_launch"] = m["traffic_bytes_per_launch"]
    roof["kernel_source_sha256_16"] = kernel_source_digest()
    roof["mfma_busy_pct_counter"] = recorded_mfma_busy("mla_decode_kernel", args.workload, kernel_source_digest())
    roof["kernel"] = "mla_decode_kernel"
    roof["kernel_avg_us"] = m["decode_us"]
    roof["alg_bytes"] = m["alg_bytes"]
    roof["alg_flops"] = m["alg_flops"]

    cpu = None if args.no_cpu_baseline else cpu_baseline(case)

    configs = None
    if not args.no_configs and args.workload == DEFAULT_WORKLOAD:
        configs = {}
        for name in CONFIG_WORKLOADS:
            del case
            case = make_case(**WORKLOADS[name])
            configs[name] = config_summary(case, measure_decode(case, name, args.config_steps,
                                                                min(args.warmup, 5), not args.no_flush,
                                                                warm_s=0.2))
            print(json.dumps({"config_done": name, "us_per_call": configs[name]["us_per_call"]}),
                  file=sys.stderr, flush=True)

    result = {
        "metric": METRIC,
        "value": m["call_us"],
        "unit": "us",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": m["call_us"] / 1e3,
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": ("bf16" if case_dtype_is_bf16(args.workload) else
                  "fp8-e4m3fn query and cache: QK^T on fp8 MFMA, PV on bf16 MFMA"
                  if WORKLOADS[args.workload].get("q_dtype", "bf16") != "bf16" else
                  "fp8-e4m3fn cache: QK^T on fp8 MFMA, PV on bf16 MFMA"),
        "data": "synthetic",
        "config": {"workload": args.workload, **{k: v for k, v in workload_shape(args.workload).items()}},
        "hbm_tb_per_s": m["alg_bytes"] / (m["call_us"] * 1e-6) / 1e12,
        "mfma_pct_of_bf16_peak": m["alg_flops"] / (m["call_us"] * 1e-6) / (MFMA_BF16_PEAK_TFLOPS * 1e12) * 100,
        "decode_us": m["decode_us"],
        "combine_us": m["combine_us"],
        "plan_us": m["plan_us"],
        "call_us_p10_p50_p90": m["call_us_p10_p50_p90"],
        "plan_wall_us_first_call": m["plan_wall_us_first_call"],
        "wall_s_timed_loop": m["wall_s"],
        "flush_between_steps": not args.no_flush,
        "roofline": roof,
        "cpu_baseline": cpu,
        "configs": configs,
    }
    print(json.dumps(result), flush=True)


def case_dtype_is_bf16(workload):
    from mla_synth import WORKLOADS
    return WORKLOADS[workload]["kv_dtype"] == "bf16"


def workload_shape(workload):
    """The shape fields of a workload, as the config object names them."""
    from mla_synth import WORKLOADS
    w = WORKLOADS[workload]
    ctx = w["ctx"]
    return {"batch": w["batch"], "heads": w["num_heads"], "seqlen_qo": w["seqlen_qo"],
            "max_ctx": (ctx[2] if isinstance(ctx, tuple) else max(ctx) if isinstance(ctx, list) else ctx),
            "page_size": w["page_size"], "kv_dtype": w["kv_dtype"], "causal": bool(w.get("causal", False))}


if __name__ == "__main__":
    main()
