"""Builds libmla_decode.so (gfx950) in-tree with hipcc.

    python mla_paged_latent_02_amd/build.py    # by path: importing the package loads the library

The library is the HIP kernels plus the C-ABI layer; nothing else is compiled.
"""

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_NAME = "libmla_decode.so"
LIB_PATH = os.path.join(HERE, LIB_NAME)
ARCH = "gfx950"

SOURCES = ["mla_kernels.hip", "mla_insert.hip", "mla_kv_b_proj.hip", "mla_scratch.hip", "mla_api.cpp", "mla_plan.cpp"]

# Packed fp32 ops are kept off in device code: hipcc -O3 would otherwise form
# v_pk_{add,mul,fma}_f32 from plain float code.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def _hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    return os.path.join(rocm, "bin", "hipcc")


def build_library(verbose: bool = False, resource_usage: bool = False) -> str:
    build_dir = os.path.join(HERE, "_build")
    os.makedirs(build_dir, exist_ok=True)
    objs = []
    for src in SOURCES:
        path = os.path.join(CSRC, src)
        obj = os.path.join(build_dir, src + ".o")
        cmd = [_hipcc(), "-c", "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-I", INCLUDE, "-I", CSRC,
               "-Wall", "-Wno-unused-function", path, "-o", obj]
        if src.endswith(".hip"):
            cmd += DEVICE_FLAGS
            if resource_usage:
                cmd += ["-Rpass-analysis=kernel-resource-usage"]
        if verbose:
            print(" ".join(cmd), flush=True)
        r = subprocess.run(cmd, capture_output=True, text=True)
        out = (r.stdout + r.stderr).strip()
        # hipcc's host pass does not know the device-only target feature; that note is harmless.
        lines = [ln for ln in out.splitlines() if "packed-fp32-ops" not in ln]
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed on {src}:\n" + "\n".join(lines))
        if lines and (verbose or resource_usage):
            print("\n".join(lines), flush=True)
        objs.append(obj)
    tmp = LIB_PATH + ".tmp"
    cmd = [_hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stdout + r.stderr)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build_library(verbose="-v" in sys.argv, resource_usage="--resources" in sys.argv))
