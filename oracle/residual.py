"""FlashBlock combined with sparse attention: the prefix keys that a sparse selection leaves
out play the role of the block-external set, and their attention (the residual) is cached
and reused, while the selected keys and the block are attended to at every step.

TEST INFRASTRUCTURE (oracle): plain fp64 CPU code; see oracle/attention.py for the import
rule and the source key.

Source: [FB-pt] §2 Metodologia, "Compatibilidade com Atenção Esparsa" (the keys not
selected by the sparse attention are treated as the block-external set and their residual
contribution is cached); [FB-ja] §2 states the same; [FB-abs]: FlashBlock as a
complementary residual-reuse strategy under aggressive sparsification.

Readings (the pages leave these open):
  * the selection is a set S of pages (page_size consecutive tokens) per (sequence, KV
    head), given to the step;
  * every query row attends to the tokens of S at every step (the sparse part, fresh);
  * the residual is the attention over the prefix tokens outside S (the complement pages;
    tokens past the prefix end do not exist); mask 0 (refresh) recomputes it and stores it
    in the cache, mask 1 (reuse) reads the cache, which then stays as it was;
  * the block part is computed at every step;
  * the output is the three-way log-space merge of the parts (the two-way merge of the
    pages with a third term): m = max_i L_i, A = sum_i e^{L_i - m} A_i / sum_i e^{L_i - m},
    L = m + log sum_i e^{L_i - m}; parts with L = -inf weigh nothing, all empty gives
    A = 0, L = -inf.
"""
from __future__ import annotations

import numpy as np

from .attention import attend, block_attention, _kv_head

NEG_INF = -np.inf


def complement_pages(sel, n_pages: int) -> np.ndarray:
    """Pages 0 .. n_pages-1 that are not in sel, ascending (int64)."""
    keep = np.ones(n_pages, dtype=bool)
    s = np.asarray(sel, dtype=np.int64)
    keep[s[(s >= 0) & (s < n_pages)]] = False
    return np.nonzero(keep)[0]


def page_tokens(pages, page: int, n: int) -> np.ndarray:
    """Token indices (within the sequence) of the given pages; tokens >= n do not exist."""
    p = np.asarray(pages, dtype=np.int64)
    if p.size == 0:
        return np.zeros(0, dtype=np.int64)
    t = (p[:, None] * page + np.arange(page)[None, :]).reshape(-1)
    return t[t < n]


def lse_merge3(a1, l1, a2, l2, a3, l3):
    """Three-way log-space merge of self-normalised parts.
    a* [..., d], l* [...] -> A [..., d], L [...]."""
    As = [np.asarray(a, dtype=np.float64) for a in (a1, a2, a3)]
    Ls = [np.asarray(l, dtype=np.float64) for l in (l1, l2, l3)]
    m = np.maximum(np.maximum(Ls[0], Ls[1]), Ls[2])
    empty = np.isneginf(m)
    m_safe = np.where(empty, 0.0, m)
    ws = [np.where(np.isneginf(l), 0.0, np.exp(np.where(np.isneginf(l), 0.0, l - m_safe))) for l in Ls]
    den = ws[0] + ws[1] + ws[2]
    den_safe = np.where(empty, 1.0, den)
    a = (ws[0][..., None] * As[0] + ws[1][..., None] * As[1] + ws[2][..., None] * As[2]) / den_safe[..., None]
    a = np.where(empty[..., None], 0.0, a)
    L = np.where(empty, NEG_INF, m_safe + np.log(den_safe))
    return a, L


def selected_and_residual(q, k, v, cu, sel, page: int, scale: float):
    """Both prefix parts of every row: (A_s, L_s) over the tokens of S and (A_r, L_r) over the
    complement.  q [b, B, H_q, d]; k, v [sum N, H_kv, d] by cu; sel[b][h_kv] page arrays."""
    b, B, h_q, d = q.shape
    h_kv = k.shape[1]
    As = np.zeros((b, B, h_q, d))
    Ls = np.full((b, B, h_q), NEG_INF)
    Ar = np.zeros((b, B, h_q, d))
    Lr = np.full((b, B, h_q), NEG_INF)
    for bi in range(b):
        lo, hi = int(cu[bi]), int(cu[bi + 1])
        n = hi - lo
        n_pages = (n + page - 1) // page
        for h in range(h_q):
            g = _kv_head(h, h_q, h_kv)
            ts = page_tokens(sel[bi][g], page, n) + lo
            tr = page_tokens(complement_pages(sel[bi][g], n_pages), page, n) + lo
            As[bi, :, h], Ls[bi, :, h] = attend(q[bi, :, h], k[ts, g], v[ts, g], scale)
            Ar[bi, :, h], Lr[bi, :, h] = attend(q[bi, :, h], k[tr, g], v[tr, g], scale)
    return As, Ls, Ar, Lr


def step(q, k, v, cu, k_blk, v_blk, sel, page: int, mask, cache_a, cache_l, scale: float):
    """One step with a cached residual.  mask [b, H_q] (0 = refresh the residual, 1 = reuse
    the cached one); cache_* [b, B, H_q, (d)] hold the residual.
    Returns (A_full, L_full, new_cache_a, new_cache_l)."""
    As, Ls, Ar, Lr = selected_and_residual(q, k, v, cu, sel, page, scale)
    new_a = np.array(cache_a, dtype=np.float64, copy=True)
    new_l = np.array(cache_l, dtype=np.float64, copy=True)
    mask = np.asarray(mask)
    for bi in range(q.shape[0]):
        for h in range(q.shape[2]):
            if mask[bi, h] == 0:
                new_a[bi, :, h] = Ar[bi, :, h]
                new_l[bi, :, h] = Lr[bi, :, h]
    a_in, l_in = block_attention(q, k_blk, v_blk, scale)
    a_full, l_full = lse_merge3(As, Ls, new_a, new_l, a_in, l_in)
    return a_full, l_full, new_a, new_l
