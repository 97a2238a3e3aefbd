"""Upload a generated Workload to device tensors and read results back.

Plumbing only: bf16 arrays travel as their raw 16-bit patterns and are
reinterpreted, never converted, so the device sees exactly the generated
bits.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Optional

import numpy as np
import torch

from .workloads import Workload


def to_device(arr: np.ndarray, dtype: str, device) -> torch.Tensor:
    a = np.ascontiguousarray(arr)
    if dtype == "bf16":
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(device)
    if dtype == "f32":
        return torch.from_numpy(a.astype(np.float32, copy=False)).to(device)
    raise ValueError(dtype)


def to_host(t: torch.Tensor, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return t.detach().view(torch.int16).cpu().numpy().view(np.uint16)
    return t.detach().cpu().numpy()


def torch_dtype(dtype: str):
    return torch.bfloat16 if dtype == "bf16" else torch.float32


@dataclass
class DeviceWorkload:
    w: Workload
    q: torch.Tensor
    k_pool: torch.Tensor
    v_pool: torch.Tensor
    block_tables: torch.Tensor
    context_lens: torch.Tensor
    k_new: torch.Tensor
    v_new: torch.Tensor
    slot_mapping: torch.Tensor
    out: torch.Tensor
    query_start: Optional[torch.Tensor] = None


def upload(w: Workload, device="cuda") -> DeviceWorkload:
    dt = w.dtype
    return DeviceWorkload(
        w=w,
        q=to_device(w.q, dt, device),
        k_pool=to_device(w.k_pool, dt, device),
        v_pool=to_device(w.v_pool, dt, device),
        block_tables=torch.from_numpy(np.ascontiguousarray(w.block_tables)).to(device),
        context_lens=torch.from_numpy(np.ascontiguousarray(w.context_lens)).to(device),
        k_new=to_device(w.k_new, dt, device),
        v_new=to_device(w.v_new, dt, device),
        slot_mapping=torch.from_numpy(np.ascontiguousarray(w.slot_mapping)).to(device),
        out=torch.empty(tuple(w.q.shape), dtype=torch_dtype(dt), device=device),
        query_start=(None if w.query_start is None else
                     torch.from_numpy(np.ascontiguousarray(w.query_start)).to(device)),
    )
