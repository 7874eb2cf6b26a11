"""FlashBlock step with cached block-external attention, and the two reuse rules.

TEST INFRASTRUCTURE (oracle): plain fp64 CPU code; see oracle/attention.py for the
import rule and the source key ([FB-pt], [FB-ja], [FB-abs]).

What a step computes [FB-pt §2 Mecanismo Central and "Estratégias de Reutilização
Adaptativa"; FB-ja §2 適応型再利用戦略]:
  * (A_in, L_in) over the current block, every step;
  * (A_out, L_out) over the prefix, only where the reuse mask is 0; there the cache
    takes the new values; where the mask is 1 the cache is left as it was (stale values
    persist across consecutive reuse steps);
  * A_full = merge(cache, (A_in, L_in)).
Readings: step 0 of a block has nothing cached, so its mask is all zero; the threshold
rule is the strict M < tau with M the number of tokens updated since the previous step;
the per-head rule is the strict sim > gamma.
"""
from __future__ import annotations

import numpy as np

from .attention import block_attention, lse_merge, prefix_attention, _kv_head, attend


def mask_threshold(m_updated, tau: int, h_q: int) -> np.ndarray:
    """Threshold reuse: reuse (1) when the updated-token count M < tau, else recompute (0).
    m_updated [b] -> mask uint8 [b, H_q]   [FB-pt §2, threshold-based reuse]"""
    m = np.asarray(m_updated).reshape(-1)
    row = (m < tau).astype(np.uint8)
    return np.repeat(row[:, None], h_q, axis=1)


def mask_similarity(sim, gamma: float) -> np.ndarray:
    """Per-head reuse (video): only heads whose similarity is above gamma reuse.
    sim [b, H_q] (float32 values) -> mask uint8 [b, H_q]   [FB-pt §2, per-head selection]
    The comparison is taken on the float32 similarity against float32(gamma)."""
    s = np.asarray(sim, dtype=np.float32)
    return (s > np.float32(gamma)).astype(np.uint8)


def head_cosine(a_prev, a_cur) -> np.ndarray:
    """Per-head similarity estimate: cosine between two block-external outputs of one head
    (all B x d entries).  a_* [b, B, H_q, d] -> sim [b, H_q].
    The pages say that a per-head similarity is estimated but not of what; this reading
    compares A_out of two consecutive computed steps.  A zero vector gives sim 0."""
    x = np.asarray(a_prev, dtype=np.float64)
    y = np.asarray(a_cur, dtype=np.float64)
    b, B, h, d = x.shape
    sim = np.zeros((b, h))
    for bi in range(b):
        for hi in range(h):
            xv = x[bi, :, hi, :].reshape(-1)
            yv = y[bi, :, hi, :].reshape(-1)
            nx, ny = np.sqrt(xv @ xv), np.sqrt(yv @ yv)
            sim[bi, hi] = 0.0 if nx == 0.0 or ny == 0.0 else (xv @ yv) / (nx * ny)
    return sim


def step(q, k, v, cu, k_blk, v_blk, mask, cache_a, cache_l, scale: float):
    """One FlashBlock denoising step.

    q [b,B,H_q,d]; k,v [sum N,H_kv,d] by cu; k_blk,v_blk [b,B,H_kv,d];
    mask uint8 [b,H_q] (1 = reuse cache); cache_a [b,B,H_q,d], cache_l [b,B,H_q] or None.
    Returns (A_full, L_full, new_cache_a, new_cache_l).
    """
    b, B, h_q, d = q.shape
    h_kv = k_blk.shape[2]
    mask = np.asarray(mask, dtype=np.uint8).reshape(b, h_q)
    if cache_a is None:
        if mask.any():
            raise ValueError("reuse requested with nothing cached")
        cache_a = np.zeros((b, B, h_q, d))
        cache_l = np.full((b, B, h_q), -np.inf)
    new_a = np.array(cache_a, dtype=np.float64, copy=True)
    new_l = np.array(cache_l, dtype=np.float64, copy=True)
    for bi in range(b):
        lo, hi = int(cu[bi]), int(cu[bi + 1])
        for h in range(h_q):
            if mask[bi, h]:
                continue                       # reuse: cache untouched, prefix not read
            g = _kv_head(h, h_q, h_kv)
            new_a[bi, :, h], new_l[bi, :, h] = attend(q[bi, :, h], k[lo:hi, g], v[lo:hi, g], scale)
    a_in, l_in = block_attention(q, k_blk, v_blk, scale)
    a_full, l_full = lse_merge(new_a, new_l, a_in, l_in)
    return a_full, l_full, new_a, new_l


def split_prefix_attention(q, k, v, cu, h_kv: int, scale: float, n_splits: int):
    """The prefix pass computed as n_splits contiguous key chunks merged with lse_merge.
    Mathematically equal to prefix_attention (the merge is exact up to rounding); used
    by tests to show that split count does not change the result."""
    b, B, h_q, d = q.shape
    A = np.zeros((b, B, h_q, d))
    L = np.full((b, B, h_q), -np.inf)
    for bi in range(b):
        lo, hi = int(cu[bi]), int(cu[bi + 1])
        edges = np.linspace(lo, hi, n_splits + 1).round().astype(int)
        for h in range(h_q):
            g = _kv_head(h, h_q, h_kv)
            acc_a = np.zeros((B, d))
            acc_l = np.full(B, -np.inf)
            for s in range(n_splits):
                pa, pl = attend(q[bi, :, h], k[edges[s]:edges[s + 1], g], v[edges[s]:edges[s + 1], g], scale)
                acc_a, acc_l = lse_merge(acc_a, acc_l, pa, pl)
            A[bi, :, h], L[bi, :, h] = acc_a, acc_l
    return A, L
