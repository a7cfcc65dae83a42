"""Python binding of libmla_decode.so: MLA decode over a paged latent KV cache on MI355X.

Argument marshalling only: every step runs in the library's HIP kernels. The
functions mirror the C entry points in include/mla_decode.h and take torch
tensors for device buffers (torch supplies device memory and streams).
The library must have been built (``python mla_paged_latent_02_amd/build.py``);
importing this package without it raises ImportError.
"""

import ctypes
import os
from typing import Optional

# torch ships its own HIP runtime. Loaded first, it also serves this library
# (same soname, libamdhip64.so.7); loaded after the library, it would bring a
# second runtime into the process, and device pointers and the current device
# of one would mean nothing to the other.
try:
    import torch  # noqa: F401
except ImportError:  # C-only use: the library takes the system runtime
    pass

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmla_decode.so")

KV_BF16 = 0
KV_FP8_E4M3FN = 1
_KV_DTYPES = {"bf16": KV_BF16, "fp8_e4m3fn": KV_FP8_E4M3FN}
_Q_DTYPES = {"bf16": 0, "fp8_e4m3fn": 1}  # mla_q_dtype_t

MLA_OK = 0
STATUS_NAMES = {0: "MLA_OK", 1: "MLA_ERR_INVALID_ARG", 2: "MLA_ERR_UNSUPPORTED",
                3: "MLA_ERR_WORKSPACE_TOO_SMALL", 4: "MLA_ERR_HIP", 5: "MLA_ERR_BAD_PLAN",
                6: "MLA_ERR_SCRATCH_TOO_SMALL"}
SCRATCH_BYTES = 96 << 20  # MLA_SCRATCH_BYTES

DEV_CTX_TOO_SHORT = 1
DEV_CTX_TOO_LONG = 2
DEV_TOO_FEW_PAGES = 4
DEV_PAGE_OUT_OF_RANGE = 8
DEV_STALE_PLAN = 16

# Every function the header declares, in declaration order.
EXPORTED = ["mla_abi_version", "mla_status_string", "mla_plan_options_default", "mla_decode_plan_host",
            "mla_decode_workspace_size", "mla_decode_plan", "mla_decode", "mla_split_combine",
            "mla_debug_read_plan_arrays", "mla_debug_read_work_list", "mla_decode_scratch",
            "mla_qcat_cache_insert", "mla_gather_kv_b_proj"]

INSERT_SLOT_OUT_OF_RANGE = 1
INSERT_POSITION_OUT_OF_RANGE = 2

KVB_TOO_FEW_PAGES = 1
KVB_SLOT_OUT_OF_RANGE = 2
KVB_ROWS_OUT_OF_RANGE = 4
KVB_CTX_TOO_LONG = 8


class DecodeParams(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("seqlen_qo", ctypes.c_int32), ("num_heads", ctypes.c_int32),
                ("page_size", ctypes.c_int32), ("max_context_len", ctypes.c_int32), ("causal", ctypes.c_int32),
                ("kv_dtype", ctypes.c_int32), ("softmax_scale", ctypes.c_float), ("kv_scale", ctypes.c_float),
                ("num_slots", ctypes.c_int64), ("q_dtype", ctypes.c_int32), ("q_scale", ctypes.c_float)]


class PlanOptions(ctypes.Structure):
    _fields_ = [("wg_per_cu", ctypes.c_int32 * 4), ("chunk_min", ctypes.c_int32 * 4),
                ("chunk_max", ctypes.c_int32 * 4), ("force_chunk", ctypes.c_int32)]


class InsertParams(ctypes.Structure):
    _fields_ = [("num_tokens", ctypes.c_int32), ("num_heads", ctypes.c_int32), ("kv_dtype", ctypes.c_int32),
                ("kv_scale", ctypes.c_float), ("num_slots", ctypes.c_int64), ("rope_positions", ctypes.c_int32),
                ("rope_neox", ctypes.c_int32)]


class KvbParams(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("num_heads", ctypes.c_int32), ("page_size", ctypes.c_int32),
                ("kv_dtype", ctypes.c_int32), ("kv_scale", ctypes.c_float), ("max_context_len", ctypes.c_int32),
                ("num_slots", ctypes.c_int64), ("num_out_rows", ctypes.c_int64)]


class Plan(ctypes.Structure):
    _fields_ = [("magic", ctypes.c_uint32), ("num_cu", ctypes.c_int32), ("params", DecodeParams),
                ("options", PlanOptions), ("heads_per_group", ctypes.c_int32), ("num_groups", ctypes.c_int32),
                ("rows_per_group", ctypes.c_int32), ("tile_rows", ctypes.c_int32), ("tile_class", ctypes.c_int32),
                ("chunk_len", ctypes.c_int32), ("max_chunks", ctypes.c_int32), ("wg_per_cu", ctypes.c_int32),
                ("num_workgroups", ctypes.c_int32),
                ("partial_capacity_records", ctypes.c_int64), ("work_capacity", ctypes.c_int64),
                ("ws_status_offset", ctypes.c_uint64), ("ws_nchunks_offset", ctypes.c_uint64),
                ("ws_partbase_offset", ctypes.c_uint64), ("ws_part_out_offset", ctypes.c_uint64),
                ("ws_part_lse_offset", ctypes.c_uint64), ("ws_work_offset", ctypes.c_uint64),
                ("ws_bytes", ctypes.c_uint64)]


class MlaError(RuntimeError):
    def __init__(self, fn, status):
        self.status = status
        super().__init__(f"{fn} failed: {STATUS_NAMES.get(status, status)} ({_lib.mla_status_string(status).decode()})")


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with `python mla_paged_latent_02_amd/build.py`")
    lib = ctypes.CDLL(LIB_PATH)
    P, V = ctypes.POINTER, ctypes.c_void_p
    sig = {
        "mla_abi_version": ([], ctypes.c_int32),
        "mla_status_string": ([ctypes.c_int], ctypes.c_char_p),
        "mla_plan_options_default": ([P(PlanOptions)], None),
        "mla_decode_plan_host": ([P(DecodeParams), P(PlanOptions), ctypes.c_int32, P(Plan)], ctypes.c_int),
        "mla_decode_workspace_size": ([P(DecodeParams), P(PlanOptions), ctypes.c_int32], ctypes.c_size_t),
        "mla_decode_plan": ([P(DecodeParams), P(PlanOptions), ctypes.c_int32, V, V, V, ctypes.c_size_t, V, P(Plan)],
                            ctypes.c_int),
        "mla_decode": ([P(Plan), V, V, V, V, V, V, V, V, ctypes.c_size_t, V], ctypes.c_int),
        "mla_split_combine": ([P(Plan), V, ctypes.c_size_t, V, V, V], ctypes.c_int),
        "mla_debug_read_plan_arrays": ([P(Plan), V, V, V, V], ctypes.c_int),
        "mla_debug_read_work_list": ([P(Plan), V, V, V], ctypes.c_int),
        "mla_decode_scratch": ([P(DecodeParams), P(PlanOptions), ctypes.c_int32, V, V, V, V, V, V, V, V, P(Plan)],
                               ctypes.c_int),
        "mla_qcat_cache_insert": ([P(InsertParams), V, V, V, V, V, V, V, V, V, V, V], ctypes.c_int),
        "mla_gather_kv_b_proj": ([P(KvbParams), V, V, V, V, V, V, V, V, V], ctypes.c_int),
    }
    for name, (args, res) in sig.items():
        if not hasattr(lib, name):
            raise ImportError(f"{LIB_PATH} does not export {name}: it is older than this binding; "
                              "rebuild it with `python mla_paged_latent_02_amd/build.py`")
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = res
    return lib


_lib = _load()


def lib():
    return _lib


def abi_version() -> int:
    return _lib.mla_abi_version()


def make_params(*, batch, seqlen_qo, num_heads, page_size, max_context_len, causal, kv_dtype, softmax_scale,
                kv_scale, num_slots, q_dtype="bf16", q_scale=1.0) -> DecodeParams:
    if isinstance(kv_dtype, str):
        kv_dtype = _KV_DTYPES[kv_dtype]
    if isinstance(q_dtype, str):
        q_dtype = _Q_DTYPES[q_dtype]
    return DecodeParams(int(batch), int(seqlen_qo), int(num_heads), int(page_size), int(max_context_len),
                        int(causal), int(kv_dtype), float(softmax_scale), float(kv_scale), int(num_slots),
                        int(q_dtype), float(q_scale))


def default_options() -> PlanOptions:
    o = PlanOptions()
    _lib.mla_plan_options_default(ctypes.byref(o))
    return o


def make_options(force_chunk: int = 0, **over) -> PlanOptions:
    o = default_options()
    o.force_chunk = int(force_chunk)
    for k, v in over.items():
        arr = getattr(o, k)
        for i, x in enumerate(v):
            arr[i] = int(x)
    return o


def plan_host(params: DecodeParams, options: Optional[PlanOptions] = None, num_cu: int = 0) -> Plan:
    plan = Plan()
    st = _lib.mla_decode_plan_host(ctypes.byref(params), ctypes.byref(options) if options else None,
                                   int(num_cu), ctypes.byref(plan))
    if st != MLA_OK:
        raise MlaError("mla_decode_plan_host", st)
    return plan


def workspace_size(params: DecodeParams, options: Optional[PlanOptions] = None, num_cu: int = 0) -> int:
    return int(_lib.mla_decode_workspace_size(ctypes.byref(params), ctypes.byref(options) if options else None,
                                              int(num_cu)))


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        import torch
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    if hasattr(stream, "cuda_stream"):
        return ctypes.c_void_p(stream.cuda_stream)
    return ctypes.c_void_p(int(stream))


def decode_plan(params: DecodeParams, context_lens, kv_indptr, workspace, options: Optional[PlanOptions] = None,
                num_cu: int = 0, stream=None) -> Plan:
    plan = Plan()
    st = _lib.mla_decode_plan(ctypes.byref(params), ctypes.byref(options) if options else None, int(num_cu),
                              _ptr(context_lens), _ptr(kv_indptr), _ptr(workspace),
                              workspace.numel() * workspace.element_size(), _stream(stream), ctypes.byref(plan))
    if st != MLA_OK:
        raise MlaError("mla_decode_plan", st)
    return plan


def decode(plan: Plan, q, kv_cache, kv_indptr, kv_page_indices, context_lens, out, lse, workspace, stream=None):
    st = _lib.mla_decode(ctypes.byref(plan), _ptr(q), _ptr(kv_cache), _ptr(kv_indptr), _ptr(kv_page_indices),
                         _ptr(context_lens), _ptr(out), _ptr(lse), _ptr(workspace),
                         workspace.numel() * workspace.element_size(), _stream(stream))
    if st != MLA_OK:
        raise MlaError("mla_decode", st)


def decode_scratch(params: DecodeParams, q, kv_cache, kv_indptr, kv_page_indices, context_lens, out, lse,
                   options: Optional[PlanOptions] = None, num_cu: int = 0, stream=None) -> Plan:
    """mla_decode_scratch: plan, decode and merge with the library's static workspace (no allocation)."""
    plan = Plan()
    st = _lib.mla_decode_scratch(ctypes.byref(params), ctypes.byref(options) if options else None, int(num_cu),
                                 _ptr(q), _ptr(kv_cache), _ptr(kv_indptr), _ptr(kv_page_indices),
                                 _ptr(context_lens), _ptr(out), _ptr(lse), _stream(stream), ctypes.byref(plan))
    if st != MLA_OK:
        raise MlaError("mla_decode_scratch", st)
    return plan


def split_combine(plan: Plan, workspace, out, lse, stream=None):
    st = _lib.mla_split_combine(ctypes.byref(plan), _ptr(workspace), workspace.numel() * workspace.element_size(),
                                _ptr(out), _ptr(lse), _stream(stream))
    if st != MLA_OK:
        raise MlaError("mla_split_combine", st)


def make_insert_params(*, num_tokens, num_heads, kv_dtype, kv_scale, num_slots, rope_positions,
                       rope_neox) -> InsertParams:
    p = InsertParams()
    p.num_tokens, p.num_heads = int(num_tokens), int(num_heads)
    p.kv_dtype = _KV_DTYPES[kv_dtype] if isinstance(kv_dtype, str) else int(kv_dtype)
    p.kv_scale = float(kv_scale)
    p.num_slots, p.rope_positions, p.rope_neox = int(num_slots), int(rope_positions), int(bool(rope_neox))
    return p


def qcat_cache_insert(params: InsertParams, ql_nope, q_pe, kv_c, k_pe, positions, cos_sin, slot_mapping, q, cache,
                      status=None, stream=None):
    """mla_qcat_cache_insert on torch device tensors (contiguous; bf16 data passed as any 2-byte dtype)."""
    st = _lib.mla_qcat_cache_insert(ctypes.byref(params), _ptr(ql_nope), _ptr(q_pe), _ptr(kv_c), _ptr(k_pe),
                                    _ptr(positions), _ptr(cos_sin), _ptr(slot_mapping), _ptr(q), _ptr(cache),
                                    _ptr(status), _stream(stream))
    if st != MLA_OK:
        raise MlaError("mla_qcat_cache_insert", st)


def make_kv_b_proj_params(*, batch, num_heads, page_size, kv_dtype, kv_scale, max_context_len, num_slots,
                          num_out_rows) -> KvbParams:
    p = KvbParams()
    p.batch, p.num_heads, p.page_size = int(batch), int(num_heads), int(page_size)
    p.kv_dtype = _KV_DTYPES[kv_dtype] if isinstance(kv_dtype, str) else int(kv_dtype)
    p.kv_scale, p.max_context_len = float(kv_scale), int(max_context_len)
    p.num_slots, p.num_out_rows = int(num_slots), int(num_out_rows)
    return p


def gather_kv_b_proj(params: KvbParams, kv_cache, kv_indptr, kv_page_indices, cu_ctx, w_kv_b, k_out, v_out,
                     status=None, stream=None):
    """mla_gather_kv_b_proj on torch device tensors (contiguous; bf16 data passed as any 2-byte dtype)."""
    st = _lib.mla_gather_kv_b_proj(ctypes.byref(params), _ptr(kv_cache), _ptr(kv_indptr), _ptr(kv_page_indices),
                                   _ptr(cu_ctx), _ptr(w_kv_b), _ptr(k_out), _ptr(v_out), _ptr(status),
                                   _stream(stream))
    if st != MLA_OK:
        raise MlaError("mla_gather_kv_b_proj", st)


def read_plan_arrays(plan: Plan, workspace):
    """(n_chunks list, partial bases list, the four status words) copied synchronously to the host."""
    B = plan.params.batch
    n = (ctypes.c_int32 * B)()
    base = (ctypes.c_int32 * B)()
    status = (ctypes.c_uint32 * 4)()
    st = _lib.mla_debug_read_plan_arrays(ctypes.byref(plan), _ptr(workspace), ctypes.cast(n, ctypes.c_void_p),
                                         ctypes.cast(base, ctypes.c_void_p), ctypes.cast(status, ctypes.c_void_p))
    if st != MLA_OK:
        raise MlaError("mla_debug_read_plan_arrays", st)
    return list(n), list(base), list(status)


def read_work_list(plan: Plan, workspace):
    """The planner's work list in hand-out order, copied synchronously: one 8-tuple per item
    (sequence, chunk, planned ctx, page-list start, n_b, first partial record, 0, 0)."""
    count = ctypes.c_int32(0)
    items = (ctypes.c_int32 * (8 * max(1, plan.work_capacity)))()
    st = _lib.mla_debug_read_work_list(ctypes.byref(plan), _ptr(workspace), ctypes.cast(ctypes.byref(count), ctypes.c_void_p),
                                       ctypes.cast(items, ctypes.c_void_p))
    if st != MLA_OK:
        raise MlaError("mla_debug_read_work_list", st)
    return [tuple(items[8 * i:8 * i + 8]) for i in range(count.value)]


def plan_to_dict(plan: Plan) -> dict:
    return {
        "heads_per_group": plan.heads_per_group, "num_groups": plan.num_groups,
        "rows_per_group": plan.rows_per_group, "tile_rows": plan.tile_rows, "tile_class": plan.tile_class,
        "chunk_len": plan.chunk_len, "max_chunks": plan.max_chunks, "wg_per_cu": plan.wg_per_cu,
        "num_workgroups": plan.num_workgroups, "grid": (plan.num_workgroups, 1, 1),
        "partial_capacity_records": plan.partial_capacity_records, "work_capacity": plan.work_capacity,
    }
