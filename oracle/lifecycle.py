"""The block lifecycle around the FlashBlock step: the denoising steps of one block with a
reuse rule, then the block's K/V appended to the growing prefix.

TEST INFRASTRUCTURE (oracle): plain fp64 CPU code; see oracle/attention.py for the import
rule and the source key.

Sources: [FB-abs] (block-wise causal inference over a KV cache that grows block by block);
[FB-pt] §2 "Mecanismo Central" (the step) and "Estratégias de Reutilização Adaptativa" (the
threshold rule M < tau and the per-head rule sim > gamma).

Readings (the pages leave these open):
  * once its steps are done, a block's B tokens join the prefix: every sequence's prefix
    becomes its old prefix followed by the block's K/V (the block K/V of the last step);
  * threshold rule: step 0 of a block refreshes every head; step s >= 1 reuses the heads of
    sequence b when M_s[b] < tau;
  * per-head rule: the similarity of head h after step s >= 1 is the cosine between the
    cached A_out before and after that step (two consecutive computed A_out of the head;
    a head that reused keeps its cache, so its similarity is 1 and it keeps reusing); steps
    0 and 1 refresh every head (two computed A_out are needed); step s >= 2 reuses head h
    when the similarity after step s - 1 is above gamma.
"""
from __future__ import annotations

import numpy as np

from . import flashblock as F
from .losa import page_minmax


def append_block(k, v, cu, k_blk, v_blk):
    """Prefix of every sequence followed by its block tokens.
    k, v [sum N, H_kv, d] by cu; k_blk, v_blk [b, B, H_kv, d] -> (k', v', cu')."""
    b, B = k_blk.shape[0], k_blk.shape[1]
    ks, vs, lens = [], [], []
    for bi in range(b):
        lo, hi = int(cu[bi]), int(cu[bi + 1])
        ks += [k[lo:hi], k_blk[bi]]
        vs += [v[lo:hi], v_blk[bi]]
        lens.append(hi - lo + B)
    cu_new = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    return np.concatenate(ks, axis=0), np.concatenate(vs, axis=0), cu_new


def page_meta_after_append(k_new, cu_new, page: int):
    """Per-page key min/max of the grown prefix: by definition the metadata of the new
    prefix (an incremental update must reach exactly this)."""
    return page_minmax(k_new, cu_new, page)


def block_run(q_steps, k, v, cu, kb_steps, vb_steps, scale: float, rule: str, m_steps=None, tau=None,
              gamma=None):
    """All steps of one block.  q_steps [S, b, B, H_q, d]; kb_steps, vb_steps [S, b, B, H_kv, d];
    rule "threshold" (m_steps [S, b], tau) or "similarity" (gamma).
    Returns dict(a_full [S,...], l_full [S,...], masks [S, b, H_q], sims [S, b, H_q] (nan
    where not defined), caches_a [S, b, B, H_q, d] and caches_l [S, b, B, H_q] (the cache
    after each step), cache_a, cache_l (after the last step))."""
    S, b, B, h_q, d = np.asarray(q_steps).shape
    cache_a = np.zeros((b, B, h_q, d))
    cache_l = np.full((b, B, h_q), -np.inf)
    sim = None
    out = dict(a_full=[], l_full=[], masks=[], sims=[], caches_a=[], caches_l=[])
    for s in range(S):
        if rule == "threshold":
            mask = np.zeros((b, h_q), np.uint8) if s == 0 else F.mask_threshold(m_steps[s], tau, h_q)
        elif rule == "similarity":
            mask = np.zeros((b, h_q), np.uint8) if s < 2 else F.mask_similarity(sim.astype(np.float32), gamma)
        else:
            raise ValueError(rule)
        a, l, new_a, new_l = F.step(q_steps[s], k, v, cu, kb_steps[s], vb_steps[s], mask, cache_a, cache_l, scale)
        sim = F.head_cosine(cache_a, new_a) if s >= 1 else np.full((b, h_q), np.nan)
        out["a_full"].append(a)
        out["l_full"].append(l)
        out["masks"].append(mask)
        out["sims"].append(sim)
        out["caches_a"].append(new_a)
        out["caches_l"].append(new_l)
        cache_a, cache_l = new_a, new_l
    res = {key: np.stack(val) for key, val in out.items()}
    res["cache_a"], res["cache_l"] = cache_a, cache_l
    return res
