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


def np_of(t):
    import torch
    return t.detach().float().cpu().numpy() if t.dtype == torch.bfloat16 else t.detach().cpu().numpy()


def say(msg):
    print(msg, flush=True)
