"""Move a generated `Case` to the GPU as torch tensors (bf16 bit patterns become torch.bfloat16)."""

from __future__ import annotations

from typing import Dict

import numpy as np
import torch


def to_torch(a: np.ndarray, dtype: str) -> torch.Tensor:
    if dtype == "bf16" and a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a))


def to_numpy_bits(t: torch.Tensor) -> np.ndarray:
    """Host copy of a device tensor; bf16 comes back as uint16 bit patterns."""
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def case_to_device(case, device="cuda") -> Dict[str, torch.Tensor]:
    dt = case.workload.dtype
    return {
        "q": to_torch(case.q, dt).to(device),
        "k_new": to_torch(case.k_new, dt).to(device),
        "v_new": to_torch(case.v_new, dt).to(device),
        "k_cache": to_torch(case.k_cache, dt).to(device),
        "v_cache": to_torch(case.v_cache, dt).to(device),
        "block_tables": torch.from_numpy(case.block_tables).to(device),
        "context_lens": torch.from_numpy(case.context_lens).to(device),
    }
