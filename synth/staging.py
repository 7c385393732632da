"""Device staging of the seeded inputs (test and benchmark plumbing, not part
of the dispatch/combine path): host arrays to GPU tensors, and the synthetic
expert outputs placed at the rows the layout assigned, as an expert kernel that
writes its output in its input order would leave them."""
from __future__ import annotations

import numpy as np
import torch


def rows_to_device(bits_u16: np.ndarray, device) -> torch.Tensor:
    """bf16 bit patterns (uint16) -> torch.bfloat16 tensor on `device`."""
    t = torch.from_numpy(np.ascontiguousarray(bits_u16).view(np.int16))
    return t.to(device).view(torch.bfloat16)


def rows_to_host(t: torch.Tensor) -> np.ndarray:
    """16-bit row tensor -> uint16 bit patterns on the host."""
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def place_expert_outputs(y_slots: torch.Tensor, pair_row: torch.Tensor, rows: int,
                         out: torch.Tensor | None = None) -> torch.Tensor:
    """y_slots [T, k, H] in (token, slot) order -> [rows, H] expert-grouped."""
    T, k, H = y_slots.shape
    if out is None:
        out = torch.zeros((rows, H), dtype=y_slots.dtype, device=y_slots.device)
    pr = pair_row.reshape(-1).long()
    ok = (pr >= 0) & (pr < rows)
    out.index_copy_(0, pr[ok], y_slots.reshape(T * k, H)[ok])
    return out
