"""Seeded synthetic inputs (no method arithmetic here).

The HIP path and the CPU oracle both consume exactly the bytes produced here:
tests copy a device tensor to the host and decode its bf16 bit patterns for
the oracle.  Each (workload, batch element, tensor) gets its own seed, so batch
elements are independent draws and a B=1 run reproduces element b of a B=2 run.
"""
from __future__ import annotations

import torch

Q, K, V = 0, 1, 2


def seed_of(workload_id: int, batch_index: int, tensor: int) -> int:
    return 1_000_003 * (workload_id + 1) + 1_009 * batch_index + tensor


def normal(shape, seed: int, sigma: float = 1.0, device="cuda", dtype=torch.bfloat16):
    """N(0, sigma^2) draws in fp32 from torch's generator on `device`, then
    cast to `dtype` (round to nearest even for bf16)."""
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    x = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    if sigma != 1.0:
        x.mul_(sigma)
    return x.to(dtype)


def qkv(workload_id: int, batch: int, L: int, heads: int, head_dim: int, sigma: float = 1.0, device="cuda",
        dtype=torch.bfloat16, batch_offset: int = 0):
    """Canonical-order Q, K, V of shape [batch, L, heads, head_dim]; batch
    element b is drawn from seed_of(workload_id, b + batch_offset, tensor)."""
    out = []
    for t in (Q, K, V):
        x = torch.empty((batch, L, heads, head_dim), dtype=dtype, device=device)
        for b in range(batch):
            x[b] = normal((L, heads, head_dim), seed_of(workload_id, b + batch_offset, t), sigma, device, dtype)
        out.append(x)
    return tuple(out)


def bf16_bits(x: torch.Tensor):
    """Host numpy uint16 view of a bf16 tensor's bit patterns."""
    return x.detach().contiguous().cpu().view(torch.int16).numpy().view("uint16")
