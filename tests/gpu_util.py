"""Helpers for the GPU tests: move seeded numpy inputs to the device and read
results back.  Only marshalling; no arithmetic of the method."""
import math

import numpy as np
import torch


def dev(x: np.ndarray) -> torch.Tensor:
    """numpy -> contiguous tensor on cuda:0 (uint16 arrays become bf16)."""
    x = np.ascontiguousarray(x)
    if x.dtype == np.uint16:
        return torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(x).cuda()


def host(t: torch.Tensor) -> np.ndarray:
    """device tensor -> float64/int numpy (bf16 widened exactly)."""
    t = t.detach().cpu()
    if t.dtype in (torch.bfloat16, torch.float32):
        return t.to(torch.float64).numpy()
    return t.numpy()


def max_err(a, b) -> float:
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    both_inf = np.isinf(a) & np.isinf(b) & (np.sign(a) == np.sign(b))
    d = np.where(both_inf, 0.0, np.abs(a - b))
    return float(np.nanmax(d)) if d.size else 0.0


# Parity bar for bf16 inputs with float32 accumulation
O_TOL = 2e-2
LSE_TOL = 1e-3


def note(msg: str) -> None:
    print(f"[gpu-case] {msg}", flush=True)


def scale_of(d: int) -> float:
    return 1.0 / math.sqrt(d)
