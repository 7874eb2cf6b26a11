"""Attention over a key set, the log-space merge, and the split/full multi-head forms.

TEST INFRASTRUCTURE (oracle): plain, slow fp64 CPU code.  Only tests/,
__graft_entry__.smoke() and bench.py's cpu_baseline leg may import it.  It shares no
code, constants or helpers with the HIP library.

Sources ("the pages"):
  [FB-pt]  "Resumo Técnico: FlashBlock" (gist.science, Portuguese), §2 Metodologia,
           "Mecanismo Central": A_in over J_in, A_out over J_out, L_out = log Z_out and
           the merge equation with m = max(L_out, L_in).
  [FB-ja]  "技術概要: FlashBlock" (gist.science, Japanese), §2 手法 / コアメカニズム:
           the same decomposition and the same merge equation.
  [FB-abs] "FlashBlock: Attention Caching for Efficient Long-Context Block Diffusion"
           (abstract): block-wise causal inference over a growing KV cache.

Readings where the pages are silent (each one is listed in the design notes):
  * scores are s_ij = scale * <q_i, k_j>, scale = 1/sqrt(d) unless given;
  * L is the natural logarithm of the softmax normaliser Z (L = log Z);
  * each part A_in / A_out is normalised within its own key set (this is what makes
    the merge a convex combination);
  * an empty key set gives A = 0 and L = -inf;
  * a block query sees the whole prefix of its sequence and the whole block
    (bidirectional inside the block).
"""
from __future__ import annotations

import numpy as np

NEG_INF = -np.inf


def attend(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float):
    """Softmax attention of query rows over one key set.

    q [R, d], k [N, d], v [N, d]  ->  A [R, d], L [R]   (all float64)

    With s_j = scale * <q, k_j>:  L = log sum_j exp(s_j)  (computed as
    m + log sum_j exp(s_j - m) with m = max_j s_j), and A = sum_j exp(s_j - L) v_j.
    [FB-pt §2 Mecanismo Central: A_out over J_out with L_out = log Z_out.]
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    R = q.shape[0]
    if k.shape[0] == 0:
        return np.zeros((R, v.shape[1])), np.full(R, NEG_INF)
    s = scale * (q @ k.T)                     # [R, N]
    m = s.max(axis=1)
    L = m + np.log(np.exp(s - m[:, None]).sum(axis=1))
    p = np.exp(s - L[:, None])
    return p @ v, L


def lse_merge(a1: np.ndarray, l1: np.ndarray, a2: np.ndarray, l2: np.ndarray):
    """Log-space merge of two self-normalised partial results.

    a* [..., d], l* [...]  ->  A [..., d], L [...]
    m = max(l1, l2); w1 = e^{l1 - m}; w2 = e^{l2 - m};
    A = (w1 a1 + w2 a2) / (w1 + w2)     [FB-pt §2 merge equation; FB-ja §2 same]
    L = m + log(w1 + w2)                (the merged normaliser; not printed on the pages,
                                         needed to merge again or to cache)
    Both sides empty (l1 = l2 = -inf) gives A = 0, L = -inf.
    """
    a1 = np.asarray(a1, dtype=np.float64)
    a2 = np.asarray(a2, dtype=np.float64)
    l1 = np.asarray(l1, dtype=np.float64)
    l2 = np.asarray(l2, dtype=np.float64)
    m = np.maximum(l1, l2)
    both_empty = np.isneginf(m)
    m_safe = np.where(both_empty, 0.0, m)
    w1 = np.where(np.isneginf(l1), 0.0, np.exp(np.where(np.isneginf(l1), 0.0, l1 - m_safe)))
    w2 = np.where(np.isneginf(l2), 0.0, np.exp(np.where(np.isneginf(l2), 0.0, l2 - m_safe)))
    den = w1 + w2
    den_safe = np.where(both_empty, 1.0, den)
    a = (w1[..., None] * a1 + w2[..., None] * a2) / den_safe[..., None]
    a = np.where(both_empty[..., None], 0.0, a)
    L = np.where(both_empty, NEG_INF, m_safe + np.log(den_safe))
    return a, L


def _kv_head(h: int, h_q: int, h_kv: int) -> int:
    """Grouped-query mapping: query head h reads KV head floor(h / (h_q / h_kv))."""
    return h // (h_q // h_kv)


def prefix_attention(q, k, v, cu, h_kv: int, scale: float):
    """Block-external part over J_out = the cached prefix of each sequence.

    q [b, B, H_q, d]; k, v [sum N, H_kv, d] packed by cu [b+1]
    -> A_out [b, B, H_q, d], L_out [b, B, H_q]          [FB-pt §2: A_out, L_out]
    """
    b, B, h_q, d = q.shape
    A = np.zeros((b, B, h_q, d))
    L = np.full((b, B, h_q), NEG_INF)
    for bi in range(b):
        lo, hi = int(cu[bi]), int(cu[bi + 1])
        for h in range(h_q):
            g = _kv_head(h, h_q, h_kv)
            A[bi, :, h], L[bi, :, h] = attend(q[bi, :, h], k[lo:hi, g], v[lo:hi, g], scale)
    return A, L


def block_attention(q, k_blk, v_blk, scale: float):
    """Block-internal part over J_in = the B tokens of the current block (bidirectional).

    q [b, B, H_q, d]; k_blk, v_blk [b, B, H_kv, d] -> A_in [b, B, H_q, d], L_in [b, B, H_q]
    [FB-pt §2: A_in over J_in]
    """
    b, B, h_q, d = q.shape
    h_kv = k_blk.shape[2]
    A = np.zeros((b, B, h_q, d))
    L = np.full((b, B, h_q), NEG_INF)
    for bi in range(b):
        for h in range(h_q):
            g = _kv_head(h, h_q, h_kv)
            A[bi, :, h], L[bi, :, h] = attend(q[bi, :, h], k_blk[bi, :, g], v_blk[bi, :, g], scale)
    return A, L


def full_attention(q, k, v, cu, k_blk, v_blk, scale: float):
    """Unsplit attention of each block query over prefix + block (the dense baseline that
    every standard block-diffusion step recomputes).  [FB-pt §1; FB-abs]"""
    b, B, h_q, d = q.shape
    h_kv = k_blk.shape[2]
    A = np.zeros((b, B, h_q, d))
    L = np.full((b, B, h_q), NEG_INF)
    for bi in range(b):
        lo, hi = int(cu[bi]), int(cu[bi + 1])
        for h in range(h_q):
            g = _kv_head(h, h_q, h_kv)
            kk = np.concatenate([k[lo:hi, g], k_blk[bi, :, g]], axis=0)
            vv = np.concatenate([v[lo:hi, g], v_blk[bi, :, g]], axis=0)
            A[bi, :, h], L[bi, :, h] = attend(q[bi, :, h], kk, vv, scale)
    return A, L
