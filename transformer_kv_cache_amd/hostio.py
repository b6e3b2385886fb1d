"""Moving seeded numpy arrays to the GPU and back (bf16 travels as its raw
16-bit patterns, numpy having no bf16 type).  Shared by the benchmark and
the GPU tests; holds no arithmetic of the method."""
from __future__ import annotations

import numpy as np
import torch


def to_dev(a: np.ndarray) -> torch.Tensor:
    """numpy array (uint16 = bf16 bit patterns) -> CUDA tensor."""
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def to_host(t: torch.Tensor) -> np.ndarray:
    """CUDA tensor -> numpy array (bf16 as uint16 bit patterns)."""
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16).copy()
    return t.numpy().copy()


def torch_dtype(dtype: str):
    return {"f32": torch.float32, "bf16": torch.bfloat16}[dtype]
