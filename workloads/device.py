"""Move generated workload arrays to the GPU with their exact storage bits.

Plumbing only: float32 arrays holding bf16 values become torch.bfloat16 device
tensors through their upper 16 bits (no rounding happens here), fp32 arrays
are copied as they are.
"""
from __future__ import annotations

import numpy as np
import torch

from .configs import Workload
from .generate import bf16_bits


def torch_dtype(wl: Workload) -> torch.dtype:
    return torch.bfloat16 if wl.dtype == "bf16" else torch.float32


def to_device(x: np.ndarray, wl: Workload, device="cuda") -> torch.Tensor:
    if wl.dtype == "bf16":
        t = torch.from_numpy(bf16_bits(x).view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(device)


def from_device(t: torch.Tensor) -> np.ndarray:
    """Exact float64 values of a device tensor."""
    return t.detach().to("cpu", torch.float32).numpy().astype(np.float64)
