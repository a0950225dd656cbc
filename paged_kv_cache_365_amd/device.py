"""Host <-> device marshalling of workloads (numpy storage arrays <-> torch tensors).

Only copies bytes: bf16 arrays travel as their raw 16-bit patterns and are
re-viewed as ``torch.bfloat16`` on the device.
"""
from __future__ import annotations

import dataclasses

import numpy as np
import torch

TORCH_DTYPE = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


def to_torch(a: np.ndarray, dtype: str, device) -> torch.Tensor:
    """Storage array -> tensor of the element dtype on ``device`` (bit copy)."""
    a = np.ascontiguousarray(a)
    if dtype == "bf16":
        t = torch.from_numpy(a.view(np.int16)).view(torch.bfloat16)
    elif dtype == "f16":
        t = torch.from_numpy(a.view(np.float16))
    else:
        t = torch.from_numpy(a.view(np.float32))
    return t.to(device)


def to_numpy(t: torch.Tensor) -> np.ndarray:
    """Tensor -> storage array (bf16 as uint16 bits)."""
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def widen_f32(t: torch.Tensor) -> np.ndarray:
    """Device output -> float64 numpy, via an exact float32 widening on the host."""
    return t.detach().float().cpu().numpy().astype(np.float64)


@dataclasses.dataclass
class DeviceWorkload:
    q: torch.Tensor
    k_pool: torch.Tensor
    v_pool: torch.Tensor
    block_tables: torch.Tensor
    context_lens: torch.Tensor
    max_context_len: int
    scale: float
    partition_size: int


def upload(w, device="cuda") -> DeviceWorkload:
    return DeviceWorkload(
        q=to_torch(w.q, w.dtype, device),
        k_pool=to_torch(w.k_pool, w.dtype, device),
        v_pool=to_torch(w.v_pool, w.dtype, device),
        block_tables=torch.from_numpy(np.ascontiguousarray(w.block_tables)).to(device),
        context_lens=torch.from_numpy(np.ascontiguousarray(w.context_lens)).to(device),
        max_context_len=max(w.max_context_len, 0),
        scale=w.scale,
        partition_size=w.partition_size,
    )
