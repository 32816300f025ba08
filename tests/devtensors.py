"""Moving seeded host arrays to and from device tensors for the GPU tests.

float32 arrays map to float32 tensors; uint16 arrays (bfloat16 bit patterns)
map to bfloat16 tensors with the same bits.  No arithmetic happens here.
"""
from __future__ import annotations

import numpy as np
import torch


def to_dev(a: np.ndarray) -> torch.Tensor:
    if a.dtype == np.float32:
        return torch.from_numpy(np.ascontiguousarray(a)).cuda()
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()
    raise TypeError(a.dtype)


def bits(t: torch.Tensor) -> np.ndarray:
    """Host copy of a device tensor as raw bits (uint32 for fp32, uint16 for bf16)."""
    h = t.detach().cpu()
    if h.dtype == torch.float32:
        return h.numpy().view(np.uint32)
    if h.dtype == torch.bfloat16:
        return h.view(torch.int16).numpy().view(np.uint16)
    if h.dtype == torch.uint8:
        return h.numpy()
    raise TypeError(h.dtype)


def oracle_bits(a: np.ndarray) -> np.ndarray:
    return a.view(np.uint32) if a.dtype == np.float32 else a.view(np.uint16)


def empty_like_host(a: np.ndarray, numel=None) -> torch.Tensor:
    n = a.size if numel is None else numel
    dt = torch.float32 if a.dtype == np.float32 else torch.bfloat16
    return torch.empty(n, dtype=dt, device="cuda")


def filled(numel: int, dtype: torch.dtype, pattern: int = 0x5A) -> torch.Tensor:
    """A device buffer filled with a byte pattern (to catch unwritten outputs)."""
    es = 4 if dtype == torch.float32 else 2
    t = torch.full((numel * es,), pattern, dtype=torch.uint8, device="cuda")
    return t.view(dtype)


def first_mismatch(got: np.ndarray, want: np.ndarray) -> str:
    bad = np.nonzero(got != want)[0]
    if bad.size == 0:
        return "none"
    i = int(bad[0])
    return f"{bad.size} mismatches, first at {i}: got {got[i]:#x} want {want[i]:#x}"
