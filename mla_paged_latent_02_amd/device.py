"""Device-side convenience around the C ABI: upload host arrays, own a workspace,
and run plan -> decode -> combine on a stream. Marshalling only."""

from dataclasses import dataclass
from typing import Optional

import numpy as np
import torch

from . import (DecodeParams, PlanOptions, Plan, decode, decode_plan, make_params, split_combine,
               workspace_size)


@dataclass
class DeviceInputs:
    q: torch.Tensor               # bf16 [B, S, H, 576]
    cache: torch.Tensor           # uint8 view of [num_slots, 576] bf16 or fp8 bytes
    kv_indptr: torch.Tensor       # int32 [B+1]
    kv_page_indices: torch.Tensor  # int32
    context_lens: torch.Tensor    # int32 [B]
    params: DecodeParams

    @staticmethod
    def from_host(*, q_bits, cache_raw, kv_indptr, kv_page_indices, context_lens, batch, seqlen_qo, num_heads,
                  page_size, max_context_len, causal, kv_dtype, softmax_scale, kv_scale, num_slots,
                  q_dtype="bf16", q_scale=1.0, device="cuda") -> "DeviceInputs":
        if q_dtype == "bf16":
            q = torch.from_numpy(np.ascontiguousarray(q_bits).view(np.int16)).view(torch.bfloat16).to(device)
        else:  # e4m3fn bytes
            q = torch.from_numpy(np.ascontiguousarray(q_bits).view(np.uint8)).to(device)
        cache = torch.from_numpy(np.ascontiguousarray(cache_raw).view(np.uint8)).to(device)
        params = make_params(batch=batch, seqlen_qo=seqlen_qo, num_heads=num_heads, page_size=page_size,
                             max_context_len=max_context_len, causal=causal, kv_dtype=kv_dtype,
                             softmax_scale=softmax_scale, kv_scale=kv_scale, num_slots=num_slots,
                             q_dtype=q_dtype, q_scale=q_scale)
        return DeviceInputs(
            q=q, cache=cache,
            kv_indptr=torch.from_numpy(np.ascontiguousarray(kv_indptr, dtype=np.int32)).to(device),
            kv_page_indices=torch.from_numpy(np.ascontiguousarray(kv_page_indices, dtype=np.int32)).to(device),
            context_lens=torch.from_numpy(np.ascontiguousarray(context_lens, dtype=np.int32)).to(device),
            params=params)


class Decoder:
    """Holds a workspace and a plan for one call shape; __call__ runs decode + combine."""

    def __init__(self, inputs: DeviceInputs, options: Optional[PlanOptions] = None, num_cu: int = 0,
                 stream=None, poison: bool = False):
        self.inputs = inputs
        p = inputs.params
        dev = inputs.q.device
        nbytes = workspace_size(p, options, num_cu)
        if nbytes == 0:
            raise ValueError("invalid decode parameters")
        self.workspace = torch.empty(nbytes, dtype=torch.uint8, device=dev)
        if poison:
            self.workspace.fill_(0xFF)  # 0xFFFFFFFF floats are NaN
        self.out = torch.empty((p.batch, p.seqlen_qo, p.num_heads, 512), dtype=torch.bfloat16, device=dev)
        self.lse = torch.empty((p.batch, p.seqlen_qo, p.num_heads), dtype=torch.float32, device=dev)
        if poison:
            self.out.fill_(float("nan"))
            self.lse.fill_(float("nan"))
        self.stream = stream
        self.plan: Plan = decode_plan(p, inputs.context_lens, inputs.kv_indptr, self.workspace, options, num_cu, stream)

    def __call__(self, with_lse: bool = True):
        i = self.inputs
        lse = self.lse if with_lse else None
        decode(self.plan, i.q, i.cache, i.kv_indptr, i.kv_page_indices, i.context_lens, self.out, lse,
               self.workspace, self.stream)
        split_combine(self.plan, self.workspace, self.out, lse, self.stream)
        return self.out, self.lse
