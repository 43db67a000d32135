"""Move a generated workload to device tensors (layout-preserving copies only)."""
from __future__ import annotations

import numpy as np
import torch


def tensor(x: np.ndarray, device) -> torch.Tensor:
    """numpy -> torch on device; uint16 arrays are bf16 bit patterns."""
    if x.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).to(device).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(x)).to(device)


def to_device(w, device="cuda"):
    """Dict of device tensors for a Workload: table, alive, ctx_len, q, k_pool,
    v_pool and (prefill) q_pos0."""
    d = dict(block_table=tensor(w.block_table.astype(np.int32), device),
             alive=tensor(w.alive.astype(np.uint8), device),
             ctx_len=tensor(w.ctx_len.astype(np.int32), device),
             q=tensor(w.q, device), k_pool=tensor(w.k_pool, device), v_pool=tensor(w.v_pool, device))
    if w.q_pos0 is not None:
        d["q_pos0"] = tensor(w.q_pos0.astype(np.int32), device)
    return d


def from_device(t: torch.Tensor) -> np.ndarray:
    """Device tensor -> float64 numpy (bf16 converted exactly)."""
    return t.detach().to("cpu").to(torch.float64).numpy()
