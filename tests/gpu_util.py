"""Shared helpers of the GPU parity tests: tolerances and device set-up."""
from __future__ import annotations

import numpy as np

# bf16 inputs, fp32 accumulation: elementwise |g - o| <= 2e-2 + 2e-2 |o|, and — so that the
# test can fail on the nearly uniform N(0,1)/sqrt(d) workloads — max |g - o| <= 2e-2 max |o|.
BF16_ATOL = BF16_RTOL = 2e-2
F32_TOL = 1e-5
MERGE_TOL = 1e-6


def check_attn(g, o, dtype, what=""):
    g = np.asarray(g, dtype=np.float64)
    o = np.asarray(o, dtype=np.float64)
    assert g.shape == o.shape, (g.shape, o.shape)
    assert np.isfinite(g).all(), f"{what}: non-finite output"
    err = np.abs(g - o)
    if dtype == "bf16":
        bad = err > BF16_ATOL + BF16_RTOL * np.abs(o)
        assert not bad.any(), f"{what}: {bad.sum()} elements out of tolerance, max err {err.max():.3e}"
        scale = np.abs(o).max()
        assert err.max() <= 2e-2 * scale + 1e-30, f"{what}: max err {err.max():.3e} vs 2e-2 * max|o| = {2e-2 * scale:.3e}"
    else:
        bad = err > F32_TOL + F32_TOL * np.abs(o)
        assert not bad.any(), f"{what}: {bad.sum()} elements out of tolerance, max err {err.max():.3e}"


def check_lse(g, o, dtype, what=""):
    g = np.asarray(g, dtype=np.float64)
    o = np.asarray(o, dtype=np.float64)
    assert g.shape == o.shape
    same_inf = np.isneginf(g) == np.isneginf(o)
    assert same_inf.all(), f"{what}: -inf pattern differs"
    fin = np.isfinite(o)
    tol = (1e-4 if dtype == "bf16" else 1e-5) * (1 + np.abs(o[fin]))
    err = np.abs(g[fin] - o[fin])
    assert (err <= tol).all(), f"{what}: L max err {err.max():.3e}"


# ---------------------------------------------------------------------- guard bands
# Buffers a parity test hands to the library are cut out of a larger allocation with
# GUARD_BYTES of canary bytes on each side.  After the test, every canary must still hold
# its pattern: a kernel that writes (or a host path that clears) past either end of an
# output, a cache or a workspace fails the test.  Input buffers get NaN canaries (0xFF
# bytes are NaN in fp32 and bf16), so a kernel that reads past an input and uses the
# value turns its output non-finite.
GUARD_BYTES = 4096
GUARD_BYTE = 0xFF
GUARDS = []   # (raw uint8 tensor, payload bytes, name), checked and cleared after each test


def guarded(shape, dtype, fill=None, name="buffer"):
    """A device tensor of `shape`/`dtype` with canary regions before and after it; `fill`
    (a number) initialises the payload, else it holds whatever the allocation held."""
    import torch
    el = torch.empty((), dtype=dtype).element_size()
    n = 1
    for x in shape:
        n *= int(x)
    nb = n * el
    raw = torch.full((nb + 2 * GUARD_BYTES,), GUARD_BYTE, dtype=torch.uint8, device="cuda")
    t = raw[GUARD_BYTES:GUARD_BYTES + nb].view(dtype).view(*shape) if n else raw[:0].view(dtype).view(*shape)
    if fill is not None and n:
        t.fill_(fill)
    GUARDS.append((raw, nb, name))
    return t


def guarded_copy(x, name="input"):
    """A guarded device copy of tensor `x` (same dtype and shape)."""
    t = guarded(tuple(x.shape), x.dtype, name=name)
    t.copy_(x)
    return t


def to_device_guarded(p):
    """synth.device.to_device with every float input in a guarded buffer (the offsets `cu`
    stay a plain tensor: an index read past its end must not be steered by a canary)."""
    from synth.device import to_device
    d = to_device(p)
    for key in ("q", "k", "v", "k_blk", "v_blk"):
        d[key] = guarded_copy(d[key], name=key)
    return d


def check_guards():
    """Every registered canary region is untouched; clears the registry."""
    items = list(GUARDS)
    GUARDS.clear()
    if not items:
        return
    import torch
    torch.cuda.synchronize()
    for raw, nb, name in items:
        head = raw[:GUARD_BYTES]
        tail = raw[GUARD_BYTES + nb:]
        for part, where in ((head, "before"), (tail, "after")):
            bad = (part != GUARD_BYTE).nonzero()
            assert bad.numel() == 0, f"{name}: {bad.numel()} guard bytes changed {where} the buffer " \
                                     f"(first at offset {int(bad[0])})"


def np_of(t):
    import torch
    return t.detach().float().cpu().numpy() if t.dtype == torch.bfloat16 else t.detach().cpu().numpy()


def say(msg):
    print(msg, flush=True)
