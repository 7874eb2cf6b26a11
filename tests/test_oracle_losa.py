"""Pins for oracle/losa.py: locality scores, the active set, page min/max, QUEST scores
(exact rational arithmetic and the upper-bound invariant), top-k, union, sparse prefix."""
import json
import os
from fractions import Fraction

import numpy as np
import pytest

import synth
from oracle.attention import attend, lse_merge, prefix_attention, block_attention
from oracle import losa

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def test_golden_locality():
    ex = json.load(open(os.path.join(GOLD, "losa_locality.json")))
    qc = np.array(ex["q_cur"])[None]
    qp = np.array(ex["q_prev"])[None]
    s = losa.locality_scores(qc, qp)
    assert s[0].tolist() == ex["scores"]
    assert losa.active_set(s, ex["n_active"])[0].tolist() == ex["active"]


def test_golden_quest():
    ex = json.load(open(os.path.join(GOLD, "quest_page_score.json")))
    k = np.array(ex["page_keys"])[:, None, :]
    mn, mx = losa.page_minmax(k, np.array([0, 2]), 2)
    assert mn[0][0, 0].tolist() == ex["kmin"] and mx[0][0, 0].tolist() == ex["kmax"]
    S = losa.quest_scores(np.array([ex["q"]]), mn[0][:, 0], mx[0][:, 0])
    assert S[0, 0] == ex["score"]
    assert max(float(np.dot(ex["q"], kk)) for kk in ex["page_keys"]) == ex["true_max"]


def test_locality_brute_force():
    g = np.random.default_rng(0)
    qc, qp = g.normal(size=(2, 5, 3, 4)), g.normal(size=(2, 5, 3, 4))
    s = losa.locality_scores(qc, qp)
    for b in range(2):
        for i in range(5):
            ref = sum(float(qc[b, i, h, j] - qp[b, i, h, j]) ** 2 for h in range(3) for j in range(4)) / 12
            assert abs(s[b, i] - ref) < 1e-14


def test_active_set_ties_and_order():
    s = np.array([[0.5, 2.0, 0.5, 2.0, 1.0, 0.5]])
    assert losa.active_set(s, 3)[0].tolist() == [1, 3, 4]
    assert losa.active_set(s, 4)[0].tolist() == [0, 1, 3, 4]       # tie 0/2/5 -> 0
    assert losa.active_set(s, 6)[0].tolist() == list(range(6))


def test_perturbed_tokens_are_the_active_set():
    """By construction: the tokens perturbed with sigma 0.5 are exactly A (sigma 0.01 rest)."""
    p = synth.losa(n_prefix=64)
    s = losa.locality_scores(p.extra["q_cur"], p.extra["q_prev"])
    act = losa.active_set(s, p.extra["n_active"])
    assert act[0].tolist() == p.extra["moved"].tolist()


def test_page_minmax_brute_force_with_tail():
    g = np.random.default_rng(1)
    k = g.normal(size=(37 + 16, 2, 3))
    cu = np.array([0, 37, 53])
    mn, mx = losa.page_minmax(k, cu, 16)
    assert mn[0].shape == (3, 2, 3) and mn[1].shape == (1, 2, 3)
    for b, (lo, hi) in enumerate([(0, 37), (37, 53)]):
        for p in range(mn[b].shape[0]):
            for h in range(2):
                for j in range(3):
                    vals = [k[t, h, j] for t in range(lo + 16 * p, min(lo + 16 * p + 16, hi))]
                    assert mn[b][p, h, j] == min(vals) and mx[b][p, h, j] == max(vals)


def test_quest_exact_rational_and_bound():
    """Scores on bf16-valued inputs equal the exact rational sum (every product is exact in
    fp64 and the sums here stay exact), bound every key in the page from above, and equal
    the best key's dot product at page size 1."""
    g = synth.rng(5)
    k = synth.normal(g, (40, 1, 6))
    q = synth.normal(g, (3, 6))
    cu = np.array([0, 40])
    for page in (1, 4, 16):
        mn, mx = losa.page_minmax(k, cu, page)
        S = losa.quest_scores(q, mn[0][:, 0], mx[0][:, 0])
        for r in range(3):
            for p in range(S.shape[1]):
                exact = sum(max(Fraction(float(q[r, j])) * Fraction(float(mn[0][p, 0, j])),
                                Fraction(float(q[r, j])) * Fraction(float(mx[0][p, 0, j]))) for j in range(6))
                assert Fraction(S[r, p]) == exact
                keys = range(p * page, min(p * page + page, 40))
                best = max(sum(Fraction(float(q[r, j])) * Fraction(float(k[t, 0, j])) for j in range(6)) for t in keys)
                assert exact >= best
                if page == 1:
                    assert exact == best


def test_topk_brute_force_with_ties():
    S = np.array([[3.0, 1.0, 3.0, 2.0, 3.0, -1.0], [0.0, 0.0, 0.0, 0.0, 0.0, 0.0]])
    assert losa.topk_pages(S, 2).tolist() == [[0, 2], [0, 1]]
    assert losa.topk_pages(S, 4).tolist() == [[0, 2, 3, 4], [0, 1, 2, 3]]
    assert losa.topk_pages(S, 8).tolist() == [[0, 1, 2, 3, 4, 5, -1, -1], [0, 1, 2, 3, 4, 5, -1, -1]]
    g = np.random.default_rng(2)
    R = g.integers(0, 5, size=(4, 30)).astype(float)    # many exact ties
    tk = losa.topk_pages(R, 7)
    for r in range(4):
        ref = sorted(sorted(range(30), key=lambda p: (-R[r, p], p))[:7])
        assert tk[r].tolist() == ref


def _small_losa(h_q=4, h_kv=2, n=150, B=6, nA=2, page=16, topk=3, seed=3):
    p = synth.custom(seed, 1, h_q, h_kv, 8, B, [n], dtype="bf16")
    g = np.random.default_rng(seed)
    q_prev = p.q
    q_cur = synth.round_bf16(q_prev + 0.01 * g.normal(size=q_prev.shape).astype(np.float32))
    return p, q_cur, q_prev, nA, page, topk


def test_union_brute_force():
    p, qc, qp, nA, page, topk = _small_losa()
    sel = losa.select_union(qc, qp, p.k, p.cu, p.h_kv, nA, page, topk)
    G = p.h_q // p.h_kv
    for g in range(p.h_kv):
        ref = set()
        for h in range(g * G, g * G + G):
            for a in range(nA):
                ref |= {int(x) for x in sel["topk"][0, h, a] if x >= 0}
        assert sel["unions"][0][g].tolist() == sorted(ref)
        assert len(ref) <= nA * G * topk


def test_sparse_prefix_brute_force_and_full_cover():
    p, qc, qp, nA, page, topk = _small_losa()
    sel = losa.select_union(qc, qp, p.k, p.cu, p.h_kv, nA, page, topk)
    o, L = losa.sparse_prefix(qc, p.k, p.v, p.cu, sel["active"], sel["unions"], p.h_kv, page, p.scale)
    n = int(p.seqlens[0])
    for h in range(p.h_q):
        g = h // (p.h_q // p.h_kv)
        toks = [t for pg in sel["unions"][0][g] for t in range(pg * page, pg * page + page) if t < n]
        for a in range(nA):
            ai, li = attend(qc[0, sel["active"][0, a], h][None], p.k[toks, g], p.v[toks, g], p.scale)
            np.testing.assert_allclose(o[0, a, h], ai[0], rtol=1e-13, atol=1e-14)
            np.testing.assert_allclose(L[0, a, h], li[0], rtol=1e-13)
    allp = [[np.arange(losa.page_count(n, page), dtype=np.int32)] * p.h_kv]
    o2, L2 = losa.sparse_prefix(qc, p.k, p.v, p.cu, sel["active"], allp, p.h_kv, page, p.scale)
    ad, ld = prefix_attention(qc, p.k, p.v, p.cu, p.h_kv, p.scale)
    np.testing.assert_allclose(o2[0], ad[0, sel["active"][0]], rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(L2[0], ld[0, sel["active"][0]], rtol=1e-13)


def test_losa_step_composition():
    """Stable rows keep their cached statistics; active rows take the sparse result; every
    row merges with the block part."""
    p, qc, qp, nA, page, topk = _small_losa()
    ca, cl = prefix_attention(qp, p.k, p.v, p.cu, p.h_kv, p.scale)
    a, l, na, nl, sel = losa.step(qc, qp, p.k, p.v, p.cu, p.k_blk, p.v_blk, ca, cl, nA, page, topk, p.scale)
    act = set(sel["active"][0].tolist())
    o, L = losa.sparse_prefix(qc, p.k, p.v, p.cu, sel["active"], sel["unions"], p.h_kv, page, p.scale)
    for i in range(p.B):
        if i in act:
            j = sel["active"][0].tolist().index(i)
            assert np.array_equal(na[0, i], o[0, j]) and np.array_equal(nl[0, i], L[0, j])
        else:
            assert np.array_equal(na[0, i], ca[0, i]) and np.array_equal(nl[0, i], cl[0, i])
    ai, li = block_attention(qc, p.k_blk, p.v_blk, p.scale)
    e, le = lse_merge(na, nl, ai, li)
    assert np.array_equal(a, e) and np.array_equal(l, le)


def test_union_is_smaller_with_fewer_active_queries():
    """The KV-inflation effect [LoSA §1]: a union over all B queries is at least as large as
    the union over the active subset."""
    p, qc, qp, nA, page, topk = _small_losa(n=400, B=8, topk=4)
    s_act = losa.select_union(qc, qp, p.k, p.cu, p.h_kv, 2, page, topk)
    s_all = losa.select_union(qc, qp, p.k, p.cu, p.h_kv, p.B, page, topk)
    for g in range(p.h_kv):
        assert set(s_act["unions"][0][g]) <= set(s_all["unions"][0][g])
