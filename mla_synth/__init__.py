"""Seeded synthetic inputs for MLA decode over a paged latent cache.

This module only *makes inputs*: random query rows, a random latent cache pool,
a shuffled page table and context lengths, plus the fp8 quantisation that turns
the random pool into e4m3fn bytes with a per-tensor scale; and, for the decode
epilogue, random query parts, latent rows, a rope table, positions and slots; and, for the
cached-prefix expansion, a random per-head projection matrix. It
holds none of the attention or epilogue arithmetic, so both the fp64 oracle and the HIP library can consume
its output without sharing any of the method's code.
"""

from .gen import WORKLOADS, MlaCase, make_case, workload_params
from .insert import INSERT_WORKLOADS, InsertCase, make_insert_case
from .kv_b_proj import KVB_WORKLOADS, KvbCase, make_kvb_case

__all__ = ["WORKLOADS", "MlaCase", "make_case", "workload_params", "INSERT_WORKLOADS", "InsertCase",
           "make_insert_case", "KVB_WORKLOADS", "KvbCase", "make_kvb_case"]
