"""Moves a seeded Problem (synth) to device tensors in the documented layouts.
Plumbing only: a dtype cast of values that are already exactly representable."""
from __future__ import annotations

import numpy as np


def tensor(x, dtype="bf16", device="cuda"):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    t = t.to(torch.bfloat16) if dtype == "bf16" else t
    return t.to(device)


def to_device(p, device="cuda"):
    import torch
    d = dict(
        q=tensor(p.q, p.dtype, device), k=tensor(p.k, p.dtype, device), v=tensor(p.v, p.dtype, device),
        k_blk=tensor(p.k_blk, p.dtype, device), v_blk=tensor(p.v_blk, p.dtype, device),
        cu=torch.from_numpy(p.cu.astype(np.int32)).to(device),
    )
    return d


def device_normal(seed: int, shape, std: float = 1.0, dtype="bf16", device="cuda"):
    """Seeded N(0, std^2) draw made on the device (torch's Philox generator), for inputs too
    large to draw on the host; rounded to bf16 by the dtype cast.  Both sides of a parity
    test read the same tensor (the oracle its host copy)."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    x = torch.randn(*shape, generator=g, device=device) * std
    return x.to(torch.bfloat16) if dtype == "bf16" else x
