"""LoSA-style sparse step: locality scores, active set, QUEST page selection for the
active queries only, union of the selected pages, sparse prefix for the active rows,
reuse of the cached prefix statistics for the stable rows, and the final merge.

TEST INFRASTRUCTURE (oracle): plain fp64 CPU code; see oracle/attention.py for the
import rule.

Sources:
  [LoSA] "LoSA: Locality Aware Sparse Attention for Block-Wise Diffusion Language
         Models" (gist.science, Spanish).  §1: each query's selection differs, so the
         memory cost is the size of the union of the B selections.  §2 "El Algoritmo
         LoSA": (1) locality pruning by the per-token MSE between this step's and the
         previous step's queries, the tokens with the largest change form the active set
         A; (2) stable tokens do no attention and reuse the stored prefix outputs o_p and
         log-normalisers L_p; (3) a QUEST-like selector runs for the active tokens only and
         I is the union of their selections; (4) prefix and block are merged by online
         softmax and the cache is updated.

Readings (the pages leave these open):
  * locality score of token i = mean over (head, dim) of (q^t - q^{t-1})^2, summed as
    sum over heads of (sum over dims, left to right), each sum left to right, in fp64;
  * A = the |A| tokens with the largest score, ties to the lower index, listed ascending;
  * QUEST page score for query q and page p = sum_d max(q_d kmin_{p,d}, q_d kmax_{p,d}),
    the exact maximum of q.k over the page's per-dimension key box, with kmin/kmax the
    element-wise min/max over the page's valid keys; summed left to right over d in
    fp64 (every product of two bfloat16 values is exact in fp64);
  * top-k by (score descending, page index ascending), listed ascending;
  * the union is per KV head over the active tokens and the query heads of its group;
  * an active row attends to every token of its group's union pages (tokens past the
    prefix end excluded), and its cache row takes the result; stable rows keep theirs;
  * the block part is computed for every row and merged with the cache.
"""
from __future__ import annotations

import numpy as np

from .attention import attend, block_attention, lse_merge, _kv_head


def locality_scores(q_cur, q_prev) -> np.ndarray:
    """[LoSA §2 step 1] q_* [b, B, H, d] -> score [b, B] (fp64)."""
    x = np.asarray(q_cur, dtype=np.float64)
    y = np.asarray(q_prev, dtype=np.float64)
    b, B, H, d = x.shape
    diff = x - y
    total = np.zeros((b, B))
    for h in range(H):
        inner = np.zeros((b, B))
        for j in range(d):
            inner = inner + diff[:, :, h, j] * diff[:, :, h, j]
        total = total + inner
    return total / float(H * d)


def active_set(scores, n_active: int) -> np.ndarray:
    """[LoSA §2 step 1] the n_active largest scores (ties: lower index), ascending.
    scores [b, B] -> int32 [b, n_active]."""
    scores = np.asarray(scores, dtype=np.float64)
    b, B = scores.shape
    out = np.zeros((b, n_active), dtype=np.int32)
    for bi in range(b):
        order = sorted(range(B), key=lambda i: (-scores[bi, i], i))
        out[bi] = np.sort(np.array(order[:n_active], dtype=np.int32))
    return out


def page_count(n: int, page: int) -> int:
    return (n + page - 1) // page


def page_minmax(k, cu, page: int):
    """Per-page, per-KV-head element-wise min and max over the page's valid keys.
    k [sum N, H_kv, d] by cu -> (kmin, kmax) lists per sequence, each [pages_b, H_kv, d]."""
    kmins, kmaxs = [], []
    for bi in range(len(cu) - 1):
        lo, hi = int(cu[bi]), int(cu[bi + 1])
        n = hi - lo
        P = page_count(n, page)
        kk = k[lo:hi]              # min / max are exact in the input precision
        mn = np.zeros((P, kk.shape[1], kk.shape[2]))
        mx = np.zeros_like(mn)
        for p in range(P):
            seg = kk[p * page:min((p + 1) * page, n)]
            mn[p] = np.asarray(seg.min(axis=0), dtype=np.float64)
            mx[p] = np.asarray(seg.max(axis=0), dtype=np.float64)
        kmins.append(mn)
        kmaxs.append(mx)
    return kmins, kmaxs


def quest_scores(qa, kmin, kmax) -> np.ndarray:
    """qa [R, d] queries; kmin/kmax [P, d] of one KV head -> S [R, P] in fp64,
    S[r, p] = sum_d max(qa[r,d] kmin[p,d], qa[r,d] kmax[p,d]), left to right over d."""
    qa = np.asarray(qa, dtype=np.float64)
    kmin = np.asarray(kmin, dtype=np.float64)
    kmax = np.asarray(kmax, dtype=np.float64)
    R, d = qa.shape
    S = np.zeros((R, kmin.shape[0]))
    for j in range(d):
        S = S + np.maximum(qa[:, j:j + 1] * kmin[None, :, j], qa[:, j:j + 1] * kmax[None, :, j])
    return S


def topk_pages(S, k: int) -> np.ndarray:
    """S [R, P] -> int32 [R, k]: the k best pages by (score desc, index asc), ascending;
    when P < k the tail is filled with -1."""
    S = np.asarray(S, dtype=np.float64)
    R, P = S.shape
    out = np.full((R, k), -1, dtype=np.int32)
    for r in range(R):
        order = np.lexsort((np.arange(P), -S[r]))[:k]
        sel = np.sort(order)
        out[r, :sel.size] = sel
    return out


def select_union(q_cur, q_prev, k, cu, h_kv: int, n_active: int, page: int, topk: int):
    """Selection half of the sparse step [LoSA §2 steps 1 and 3].
    Returns dict with scores [b,B], active [b,|A|], topk [b,H_q,|A|,topk],
    union list per (b, h_kv) (ascending int32 arrays), and the page metadata."""
    b, B, h_q, d = q_cur.shape
    scores = locality_scores(q_cur, q_prev)
    act = active_set(scores, n_active)
    kmins, kmaxs = page_minmax(k, cu, page)
    tk = np.full((b, h_q, n_active, topk), -1, dtype=np.int32)
    unions = []
    for bi in range(b):
        qa = np.asarray(q_cur[bi, act[bi]], dtype=np.float64)       # [|A|, H_q, d]
        per_kv = [set() for _ in range(h_kv)]
        for h in range(h_q):
            g = _kv_head(h, h_q, h_kv)
            S = quest_scores(qa[:, h], kmins[bi][:, g], kmaxs[bi][:, g])
            tk[bi, h] = topk_pages(S, topk)
            per_kv[g].update(int(x) for x in tk[bi, h].reshape(-1) if x >= 0)
        unions.append([np.array(sorted(s), dtype=np.int32) for s in per_kv])
    return dict(scores=scores, active=act, topk=tk, unions=unions, kmin=kmins, kmax=kmaxs)


def union_tokens(pages: np.ndarray, page: int, n: int) -> np.ndarray:
    """Token indices (within the sequence) of the given pages, tokens >= n dropped."""
    if len(pages) == 0:
        return np.zeros(0, dtype=np.int64)
    t = (np.asarray(pages, dtype=np.int64)[:, None] * page + np.arange(page)[None, :]).reshape(-1)
    return t[t < n]


def sparse_prefix(q_cur, k, v, cu, active, unions, h_kv: int, page: int, scale: float):
    """[LoSA §2 step 3] active rows attend over the tokens of their group's union pages.
    Returns (o_p [b, |A|, H_q, d], L_p [b, |A|, H_q])."""
    b, B, h_q, d = q_cur.shape
    nA = active.shape[1]
    o = np.zeros((b, nA, h_q, d))
    L = np.full((b, nA, h_q), -np.inf)
    for bi in range(b):
        lo, hi = int(cu[bi]), int(cu[bi + 1])
        for h in range(h_q):
            g = _kv_head(h, h_q, h_kv)
            t = union_tokens(unions[bi][g], page, hi - lo) + lo
            o[bi, :, h], L[bi, :, h] = attend(q_cur[bi, active[bi], h], k[t, g], v[t, g], scale)
    return o, L


def step(q_cur, q_prev, k, v, cu, k_blk, v_blk, cache_a, cache_l, n_active: int,
         page: int, topk: int, scale: float):
    """One LoSA-style sparse step t >= 1 [LoSA §2 steps 1-4].
    cache_* hold the prefix statistics (o_p, L_p) of every row from the previous step.
    Returns (A_full, L_full, new_cache_a, new_cache_l, selection dict)."""
    h_kv = k_blk.shape[2]
    sel = select_union(q_cur, q_prev, k, cu, h_kv, n_active, page, topk)
    o_p, l_p = sparse_prefix(q_cur, k, v, cu, sel["active"], sel["unions"], h_kv, page, scale)
    new_a = np.array(cache_a, dtype=np.float64, copy=True)
    new_l = np.array(cache_l, dtype=np.float64, copy=True)
    for bi in range(q_cur.shape[0]):
        new_a[bi, sel["active"][bi]] = o_p[bi]
        new_l[bi, sel["active"][bi]] = l_p[bi]
    a_in, l_in = block_attention(q_cur, k_blk, v_blk, scale)
    a_full, l_full = lse_merge(new_a, new_l, a_in, l_in)
    return a_full, l_full, new_a, new_l, sel
