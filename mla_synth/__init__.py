"""Seeded synthetic inputs for MLA decode over a paged latent cache.

This module only *makes inputs*: random query rows, a random latent cache pool,
a shuffled page table and context lengths, plus the fp8 quantisation that turns
the random pool into e4m3fn bytes with a per-tensor scale. It holds none of the
attention arithmetic, so both the fp64 oracle and the HIP library can consume
its output without sharing any of the method's code.
"""

from .gen import WORKLOADS, MlaCase, make_case, workload_params

__all__ = ["WORKLOADS", "MlaCase", "make_case", "workload_params"]
