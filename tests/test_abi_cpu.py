"""The C ABI loads and exports every declared symbol; host planning and argument
checks behave (CPU only: no call here touches a GPU)."""

import ctypes
import math
import os
import re
import subprocess

import pytest

import mla_paged_latent_02_amd as mla
from oracle import PlanOptions as RefOptions, reference_plan

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mla_decode.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return re.findall(r"\b(mla_[a-z0-9_]+)\s*\(", text)


def test_every_declared_symbol_is_exported():
    names = declared_functions()
    assert set(names) == set(mla.EXPORTED)
    for n in names:
        assert hasattr(mla.lib(), n), n


def test_struct_layouts_match_the_c_compiler(tmp_path):
    # sizeof/offsetof as gcc lays out the header, against the ctypes mirrors
    checks = [("mla_decode_params_t", mla.DecodeParams), ("mla_plan_options_t", mla.PlanOptions),
              ("mla_insert_params_t", mla.InsertParams),
              ("mla_kv_b_proj_params_t", mla.KvbParams),
              ("mla_plan_t", mla.Plan)]
    lines = ["#include <stdio.h>", "#include <stddef.h>", '#include "mla_decode.h"', "int main(void) {"]
    for cname, cls in checks:
        lines.append(f'printf("%zu\\n", sizeof({cname}));')
        for f, _ in cls._fields_:
            lines.append(f'printf("%zu\\n", offsetof({cname}, {f}));')
    lines.append("return 0; }")
    src = tmp_path / "layout.c"
    src.write_text("\n".join(lines))
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe)], check=True)
    got = [int(x) for x in subprocess.run([str(exe)], capture_output=True, text=True, check=True).stdout.split()]
    want = []
    for _, cls in checks:
        want.append(ctypes.sizeof(cls))
        want += [getattr(cls, f).offset for f, _ in cls._fields_]
    assert got == want


def test_abi_version_and_status_strings():
    declared = int(re.search(r"#define MLA_ABI_VERSION (\d+)", open(HEADER).read()).group(1))
    assert mla.abi_version() == declared
    for code in range(6):
        assert mla.lib().mla_status_string(code)
    assert mla.lib().mla_status_string(99) == b"unknown status"


def params(**kw):
    base = dict(batch=4, seqlen_qo=1, num_heads=16, page_size=16, max_context_len=1000, causal=False,
                kv_dtype="fp8_e4m3fn", softmax_scale=1 / math.sqrt(192), kv_scale=0.01, num_slots=4096)
    base.update(kw)
    return mla.make_params(**base)


SHAPES = [(2, 1, 16, 100), (64, 1, 128, 8192), (256, 1, 128, 23333), (1, 1, 12, 109440), (5, 1, 12, 109440),
          (128, 4, 16, 5200), (3, 2, 128, 1000), (7, 8, 16, 64), (1, 3, 5, 3), (9, 1, 40, 777), (4, 4, 64, 4096)]


@pytest.mark.parametrize("shape", SHAPES)
@pytest.mark.parametrize("force", [0, 64, 320])
@pytest.mark.parametrize("dt", ["bf16", "fp8_e4m3fn"])
def test_host_plan_matches_reference_planner_bit_exactly(shape, force, dt):
    B, S, H, L = shape
    p = params(batch=B, seqlen_qo=S, num_heads=H, max_context_len=L, kv_dtype=dt,
               kv_scale=1.0 if dt == "bf16" else 0.01)
    plan = mla.plan_host(p, mla.make_options(force_chunk=force), num_cu=256)
    ref = reference_plan(B, S, H, L, 256, RefOptions(force_chunk=force), kv_dtype=dt)
    got = mla.plan_to_dict(plan)
    assert got == {k: ref[k] for k in got}
    assert plan.magic == 0x4D4C4132
    # workspace layout: 256-aligned, disjoint, in order, large enough for every partial
    offs = [plan.ws_status_offset, plan.ws_nchunks_offset, plan.ws_partbase_offset, plan.ws_part_out_offset,
            plan.ws_part_lse_offset, plan.ws_work_offset, plan.ws_bytes]
    assert all(o % 256 == 0 for o in offs) and offs == sorted(offs)
    assert plan.ws_nchunks_offset - plan.ws_status_offset >= 16
    assert plan.ws_partbase_offset - plan.ws_nchunks_offset >= 4 * B
    assert plan.ws_part_lse_offset - plan.ws_part_out_offset >= 4 * 512 * ref["rows_per_group"] * ref["partial_capacity_records"]
    assert plan.ws_work_offset - plan.ws_part_lse_offset >= 4 * ref["rows_per_group"] * ref["partial_capacity_records"]
    assert plan.ws_bytes - plan.ws_work_offset >= 8 * ref["work_capacity"]
    assert mla.workspace_size(p, mla.make_options(force_chunk=force), 256) == plan.ws_bytes


def test_fp8_query_params_plan_like_bf16_query():
    # the query type changes no part of the plan (grid, chunking, workspace)
    for shape in SHAPES:
        B, S, H, L = shape
        a = mla.plan_to_dict(mla.plan_host(params(batch=B, seqlen_qo=S, num_heads=H, max_context_len=L), None, 256))
        b = mla.plan_to_dict(mla.plan_host(params(batch=B, seqlen_qo=S, num_heads=H, max_context_len=L,
                                                  q_dtype="fp8_e4m3fn", q_scale=0.02), None, 256))
        assert a == b


def test_default_options_match_the_header_and_the_oracle():
    # the defaults the header documents, the library's and the oracle planner's agree
    here = os.path.dirname(os.path.abspath(__file__))
    text = open(os.path.join(here, "..", "include", "mla_decode.h")).read()
    o, ro = mla.default_options(), RefOptions()
    for name in ("wg_per_cu", "chunk_min", "chunk_max"):
        doc = [int(x) for x in re.search(name + r" \{([\d, ]+)\}", text).group(1).split(",")]
        assert list(getattr(o, name)) == doc == list(getattr(ro, name)), name
    assert o.force_chunk == 0 == ro.force_chunk


def test_non_default_options_follow_the_rule():
    o = mla.make_options(wg_per_cu=[1, 1, 1, 3], chunk_min=[64, 64, 64, 64], chunk_max=[128, 128, 128, 512])
    ro = RefOptions(wg_per_cu=[1, 1, 1, 3], chunk_min=[64, 64, 64, 64], chunk_max=[128, 128, 128, 512])
    for shape in SHAPES:
        B, S, H, L = shape
        got = mla.plan_to_dict(mla.plan_host(params(batch=B, seqlen_qo=S, num_heads=H, max_context_len=L), o, 304))
        ref = reference_plan(B, S, H, L, 304, ro, kv_dtype="fp8_e4m3fn")
        assert got == {k: ref[k] for k in got}


def test_large_batches_plan():
    # no grid limit of 65535 applies: the decode grid is the persistent workgroups and the merge
    # grids are one-dimensional
    for B in (65535, 65536, 200000):
        plan = mla.plan_host(params(batch=B, max_context_len=64, num_slots=16 * 4 * B), None, 256)
        assert plan.num_workgroups == 256 and plan.work_capacity == B
    # past the 32-bit task count: rejected as unsupported, before any device work
    with pytest.raises(mla.MlaError) as e:
        mla.plan_host(params(batch=2 ** 20, num_heads=2048, max_context_len=2 ** 20, num_slots=16), None, 256)
    assert e.value.status == 2


def test_persistent_grid_follows_the_kernel_occupancy():
    # W = num_cu x min(requested workgroups per CU, what the class's kernel holds): the fp8 64-row
    # kernel holds two per CU, every other one
    for dt, S, H, want in (("fp8_e4m3fn", 4, 16, 2), ("bf16", 4, 16, 1), ("fp8_e4m3fn", 1, 128, 1),
                           ("fp8_e4m3fn", 1, 12, 1), ("bf16", 1, 128, 1)):
        kw = dict(kv_dtype=dt, kv_scale=1.0 if dt == "bf16" else 0.01, seqlen_qo=S, num_heads=H)
        plan = mla.plan_host(params(**kw), mla.make_options(wg_per_cu=[4, 4, 4, 4]), 100)
        assert (plan.wg_per_cu, plan.num_workgroups) == (want, 100 * want), (dt, S, H)


@pytest.mark.parametrize("bad, code", [
    (dict(batch=0), 1), (dict(seqlen_qo=0), 1), (dict(seqlen_qo=9), 2), (dict(num_heads=0), 1),
    (dict(page_size=0), 1), (dict(max_context_len=0), 1), (dict(causal=2), 1), (dict(kv_dtype=7), 1),
    (dict(softmax_scale=float("nan")), 1), (dict(softmax_scale=0.0), 1), (dict(kv_scale=0.0), 1),
    (dict(kv_scale=-1.0), 1), (dict(kv_dtype="bf16", kv_scale=0.5), 1), (dict(num_slots=0), 1),
    (dict(num_slots=4097), 1), (dict(seqlen_qo=4, max_context_len=3), 1),
    (dict(q_dtype=2), 1), (dict(q_dtype="fp8_e4m3fn", q_scale=0.0), 1),
    (dict(q_dtype="fp8_e4m3fn", q_scale=float("inf")), 1), (dict(q_scale=0.5), 1),
    (dict(q_dtype="fp8_e4m3fn", q_scale=0.5, kv_dtype="bf16", kv_scale=1.0), 2),
])
def test_invalid_params_are_rejected_before_device_work(bad, code):
    p = params(**bad)
    with pytest.raises(mla.MlaError) as e:
        mla.plan_host(p, None, num_cu=256)
    assert e.value.status == code
    assert mla.workspace_size(p, None, 256) == 0


@pytest.mark.parametrize("opt", [dict(force_chunk=63), dict(force_chunk=-64), dict(chunk_min=[0, 64, 64, 64]),
                                 dict(chunk_max=[32, 64, 64, 64]), dict(wg_per_cu=[0, 1, 1, 1])])
def test_invalid_options_are_rejected(opt):
    with pytest.raises(mla.MlaError) as e:
        mla.plan_host(params(), mla.make_options(**opt), num_cu=256)
    assert e.value.status == 1


def test_entry_points_reject_null_and_bad_plans_without_touching_the_device():
    lib = mla.lib()
    p = params()
    plan = mla.Plan()
    # null pointers -> invalid argument, before any HIP call
    assert lib.mla_decode_plan(ctypes.byref(p), None, 256, None, None, None, 0, None, ctypes.byref(plan)) == 1
    # a zeroed plan is not a plan
    assert lib.mla_decode(ctypes.byref(plan), *([None] * 8), 0, None) == 5
    assert lib.mla_split_combine(ctypes.byref(plan), None, 0, None, None, None) == 5
    assert lib.mla_debug_read_plan_arrays(ctypes.byref(plan), None, None, None, None) == 5
    good = mla.plan_host(p, None, 256)
    fake = ctypes.c_void_p(16)  # never dereferenced: rejected by the size check first
    assert lib.mla_decode(ctypes.byref(good), fake, fake, fake, fake, fake, fake, None, fake, 0, None) == 3
    assert lib.mla_decode(ctypes.byref(good), None, fake, fake, fake, fake, fake, None, fake,
                          good.ws_bytes, None) == 1
    assert lib.mla_split_combine(ctypes.byref(good), fake, 0, fake, None, None) == 3


def test_one_hip_runtime_whatever_the_import_order():
    # Importing the binding before torch must not map a second HIP runtime.
    code = ("import mla_paged_latent_02_amd, torch\n"
            "maps = {l.split()[-1] for l in open('/proc/self/maps') if 'libamdhip64' in l}\n"
            "print(len({os.path.realpath(m) for m in maps}))")
    out = subprocess.run([os.sys.executable, "-c", "import os\n" + code], cwd=ROOT, capture_output=True, text=True,
                         check=True).stdout.split()
    assert out[-1] == "1"


def test_build_script_loads_without_the_package():
    # __graft_entry__.build() loads the build script by path, so a missing or stale
    # library cannot stop the build that would replace it
    import importlib.util
    import sys
    spec = importlib.util.spec_from_file_location("_mla_build_check", os.path.join(ROOT, "mla_paged_latent_02_amd",
                                                                                  "build.py"))
    mod = importlib.util.module_from_spec(spec)
    before = set(sys.modules)
    spec.loader.exec_module(mod)
    assert callable(mod.build_library) and "mla_insert.hip" in mod.SOURCES
    assert not any(m.startswith("mla_paged_latent_02_amd") for m in set(sys.modules) - before)


@pytest.mark.parametrize("bad, code", [
    (dict(num_tokens=-1), 1), (dict(num_heads=0), 1), (dict(kv_dtype=5), 1), (dict(kv_scale=0.0), 1),
    (dict(kv_scale=float("nan")), 1), (dict(kv_dtype="bf16", kv_scale=2.0), 1), (dict(num_slots=0), 1),
    (dict(rope_positions=0), 1), (dict(rope_neox=2), 1),
])
def test_insert_rejects_bad_params_before_device_work(bad, code):
    kw = dict(num_tokens=4, num_heads=8, kv_dtype="fp8_e4m3fn", kv_scale=0.5, num_slots=16, rope_positions=8,
              rope_neox=0)
    kw.update(bad)
    p = mla.make_insert_params(**kw)
    if "rope_neox" in bad:
        p.rope_neox = bad["rope_neox"]
    assert mla.lib().mla_qcat_cache_insert(p, *([None] * 11)) == code


def test_insert_rejects_null_buffers():
    p = mla.make_insert_params(num_tokens=4, num_heads=8, kv_dtype="bf16", kv_scale=1.0, num_slots=16,
                               rope_positions=8, rope_neox=0)
    assert mla.lib().mla_qcat_cache_insert(p, *([None] * 11)) == 1
    assert mla.lib().mla_qcat_cache_insert(None, *([None] * 11)) == 1


@pytest.mark.parametrize("bad", [
    dict(batch=-1), dict(num_heads=0), dict(page_size=0), dict(kv_dtype=7), dict(kv_scale=0.0),
    dict(kv_scale=float("inf")), dict(kv_dtype="bf16", kv_scale=0.5), dict(max_context_len=-1), dict(num_slots=0),
    dict(num_out_rows=-1),
])
def test_kv_b_proj_rejects_bad_params_before_device_work(bad):
    kw = dict(batch=2, num_heads=12, page_size=1, kv_dtype="fp8_e4m3fn", kv_scale=0.5, max_context_len=100,
              num_slots=1000, num_out_rows=200)
    kw.update(bad)
    p = mla.make_kv_b_proj_params(**kw)
    assert mla.lib().mla_gather_kv_b_proj(p, *([None] * 9)) == 1


def test_kv_b_proj_nulls_and_empty_calls():
    kw = dict(batch=2, num_heads=12, page_size=1, kv_dtype="bf16", kv_scale=1.0, max_context_len=100,
              num_slots=1000, num_out_rows=200)
    assert mla.lib().mla_gather_kv_b_proj(mla.make_kv_b_proj_params(**kw), *([None] * 9)) == 1
    assert mla.lib().mla_gather_kv_b_proj(None, *([None] * 9)) == 1
    # nothing to do: returns before touching any buffer
    assert mla.lib().mla_gather_kv_b_proj(mla.make_kv_b_proj_params(**dict(kw, batch=0)), *([None] * 9)) == 0
    assert mla.lib().mla_gather_kv_b_proj(mla.make_kv_b_proj_params(**dict(kw, max_context_len=0)),
                                          *([None] * 9)) == 0


def test_kv_b_proj_rejects_more_programs_than_32_bits_count():
    # 2^20 sequences x ceil(4096 / 256) = 16 chunks x 128 heads = 2^31 programs of 256 cached rows
    # and one head: refused on the host, before any device work (the buffers are placeholders that
    # are never touched)
    kw = dict(batch=2 ** 20, num_heads=128, page_size=1, kv_dtype="bf16", kv_scale=1.0, max_context_len=4096,
              num_slots=1000, num_out_rows=200)
    fake = [ctypes.c_void_p(4096)] * 8 + [None]
    assert mla.lib().mla_gather_kv_b_proj(mla.make_kv_b_proj_params(**kw), *fake) == 2


def test_status_bits_of_the_header_match_the_binding():
    # every status bit the header defines (decode device bits, stale plan included; epilogue; expansion)
    # has a binding constant of the same value, and the bits of each group are distinct powers of two
    text = open(os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include",
                             "mla_decode.h")).read()
    defs = {m.group(1): int(m.group(2)) for m in re.finditer(r"#define MLA_((?:DEV|INSERT|KVB)_\w+) (\d+)u", text)}
    assert "DEV_STALE_PLAN" in defs and len(defs) >= 11
    for name, value in defs.items():
        assert getattr(mla, name) == value, name
    for group in ("DEV_", "INSERT_", "KVB_"):
        vals = [v for k, v in defs.items() if k.startswith(group)]
        assert all(v & (v - 1) == 0 for v in vals) and len(set(vals)) == len(vals), group
