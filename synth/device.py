"""Move a drawn batch of inputs onto the GPU as torch tensors (data movement only)."""
from __future__ import annotations

from dataclasses import dataclass
from typing import Optional

import numpy as np
import torch

from .generate import Inputs


@dataclass
class DeviceInputs:
    q: Optional[torch.Tensor]
    k: Optional[torch.Tensor]
    v: Optional[torch.Tensor]
    block_table: Optional[torch.Tensor]
    prefix_len: torch.Tensor
    parent: torch.Tensor
    tokens: torch.Tensor
    logits: Optional[torch.Tensor]
    uniforms: torch.Tensor
    tau: float


def to_device(inp: Inputs, device="cuda") -> DeviceInputs:
    """bf16 workloads become torch.bfloat16 (exact: the values are bf16-representable)."""
    dt = torch.bfloat16 if inp.cfg.dtype == "bf16" else torch.float32

    def kv(a):
        return None if a is None else torch.from_numpy(a).to(device).to(dt).contiguous()

    def i32(a):
        return None if a is None else torch.from_numpy(np.ascontiguousarray(a, np.int32)).to(device)

    return DeviceInputs(
        q=kv(inp.q), k=kv(inp.k), v=kv(inp.v),
        block_table=i32(inp.block_table),
        prefix_len=i32(inp.prefix_len),
        parent=i32(inp.parent),
        tokens=i32(inp.tokens),
        logits=None if inp.logits is None else torch.from_numpy(inp.logits).to(device),
        uniforms=torch.from_numpy(inp.uniforms).to(device),
        tau=float(inp.tau),
    )
