"""Pins for oracle/attention.py: closed forms, brute force, a library cross-check and the
split-plus-merge identity."""
import json
import math
import os

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

from oracle.attention import attend, block_attention, full_attention, lse_merge, prefix_attention
from oracle.flashblock import split_prefix_attention

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def brute_attend(q, k, v, scale):
    """Direct softmax with math.exp and no max shift; small magnitudes only."""
    R, d = len(q), len(v[0]) if len(v) else 0
    A, L = [], []
    for r in range(R):
        w = [math.exp(scale * sum(q[r][t] * k[j][t] for t in range(len(q[r])))) for j in range(len(k))]
        z = sum(w)
        A.append([sum(w[j] * v[j][t] for j in range(len(k))) / z for t in range(d)])
        L.append(math.log(z))
    return np.array(A), np.array(L)


@settings(max_examples=40, deadline=None)
@given(R=st.integers(1, 4), N=st.integers(1, 9), d=st.sampled_from([1, 3, 8]),
       seed=st.integers(0, 10_000), scale=st.sampled_from([1.0, 0.125, 0.7]))
def test_attend_matches_brute_force(R, N, d, seed, scale):
    g = np.random.default_rng(seed)
    q, k, v = g.normal(size=(R, d)), g.normal(size=(N, d)), g.normal(size=(N, d))
    A, L = attend(q, k, v, scale)
    Ab, Lb = brute_attend(q.tolist(), k.tolist(), v.tolist(), scale)
    np.testing.assert_allclose(A, Ab, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(L, Lb, rtol=1e-12, atol=1e-12)


def test_attend_closed_forms():
    g = np.random.default_rng(1)
    q, k, v = g.normal(size=(3, 5)), g.normal(size=(1, 5)), g.normal(size=(1, 5))
    A, L = attend(q, k, v, 0.3)                      # one key: A = v, L = s
    np.testing.assert_allclose(A, np.repeat(v, 3, axis=0), rtol=0, atol=1e-15)
    np.testing.assert_allclose(L, 0.3 * (q @ k[0]), rtol=1e-15)
    kk = np.repeat(k, 7, axis=0)                     # identical keys: A = mean(V), L = s + ln N
    vv = g.normal(size=(7, 5))
    A, L = attend(q, kk, vv, 0.3)
    np.testing.assert_allclose(A, np.repeat(vv.mean(0, keepdims=True), 3, 0), atol=1e-14)
    np.testing.assert_allclose(L, 0.3 * (q @ k[0]) + math.log(7), rtol=1e-14)
    A, L = attend(q, np.zeros((0, 5)), np.zeros((0, 5)), 0.3)   # empty: A = 0, L = -inf
    assert np.all(A == 0) and np.all(np.isneginf(L))


def test_attend_large_logits_stay_finite():
    q = np.array([[100.0, 0.0]])
    k = np.array([[10.0, 0.0], [9.0, 0.0]])
    v = np.array([[1.0, 0.0], [0.0, 1.0]])
    A, L = attend(q, k, v, 1.0)        # s = [1000, 900]: e^1000 overflows without the shift
    assert np.isfinite(A).all() and abs(L[0] - (1000 + math.log1p(math.exp(-100)))) < 1e-9
    np.testing.assert_allclose(A[0], [1.0, math.exp(-100)], rtol=1e-12, atol=1e-300)


def test_attend_matches_torch_sdpa_fp64():
    torch = pytest.importorskip("torch")
    g = np.random.default_rng(7)
    q, k, v = g.normal(size=(5, 16)), g.normal(size=(11, 16)), g.normal(size=(11, 16))
    A, L = attend(q, k, v, 0.25)
    tq, tk, tv = (torch.from_numpy(x)[None, None] for x in (q, k, v))
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, scale=0.25)[0, 0].numpy()
    lse = torch.logsumexp(0.25 * (torch.from_numpy(q) @ torch.from_numpy(k).T), dim=1).numpy()
    np.testing.assert_allclose(A, ref, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(L, lse, rtol=1e-13)


def test_golden_two_key_merge():
    ex = json.load(open(os.path.join(GOLD, "merge_two_keys.json")))
    q = np.array(ex["q"])
    ao, lo = attend(q, np.array(ex["k_out"]), np.array(ex["v_out"]), ex["scale"])
    ai, li = attend(q, np.array(ex["k_in"]), np.array(ex["v_in"]), ex["scale"])
    np.testing.assert_allclose(ao[0], ex["A_out"], atol=1e-15)
    np.testing.assert_allclose(ai[0], ex["A_in"], atol=1e-15)
    assert lo[0] == ex["L_out"] and li[0] == ex["L_in"]
    a, l = lse_merge(ao, lo, ai, li)
    np.testing.assert_allclose(a[0], ex["A_full"], rtol=1e-15)
    np.testing.assert_allclose(l[0], ex["L_full"], rtol=1e-15)
    af, lf = attend(q, np.array(ex["k_out"] + ex["k_in"]), np.array(ex["v_out"] + ex["v_in"]), 1.0)
    np.testing.assert_allclose(af[0], ex["A_full"], rtol=1e-15)
    np.testing.assert_allclose(lf[0], ex["L_full"], rtol=1e-15)


def test_merge_conventions():
    g = np.random.default_rng(3)
    a1, a2, a3 = g.normal(size=(3, 4, 6))
    l1, l2, l3 = g.normal(size=(3, 4)) * 5
    x, lx = lse_merge(a1, l1, a2, l2)
    y, ly = lse_merge(a2, l2, a1, l1)
    np.testing.assert_allclose(x, y, rtol=1e-14)                        # commutative
    np.testing.assert_allclose(lx, ly, rtol=1e-14)
    p, lp = lse_merge(*lse_merge(a1, l1, a2, l2), a3, l3)
    r, lr = lse_merge(a1, l1, *lse_merge(a2, l2, a3, l3))
    np.testing.assert_allclose(p, r, rtol=1e-13)                        # associative
    np.testing.assert_allclose(lp, lr, rtol=1e-13)
    ninf = np.full(4, -np.inf)
    e, le = lse_merge(a1, l1, np.zeros_like(a1), ninf)                  # empty side
    np.testing.assert_array_equal(e, a1)
    np.testing.assert_array_equal(le, l1)
    z, lz = lse_merge(a1, ninf, a2, ninf)                               # both empty
    assert np.all(z == 0) and np.all(np.isneginf(lz))
    w, lw = lse_merge(a1, l1, a2, l1)                                   # equal L: plain mean
    np.testing.assert_allclose(w, (a1 + a2) / 2, rtol=1e-14)
    np.testing.assert_allclose(lw, l1 + math.log(2), rtol=1e-14)
    big, lb = lse_merge(a1, l1 + 1000.0, a2, l2)                        # one side dominates
    np.testing.assert_allclose(big, a1, rtol=1e-14)


def brute_multihead(q, k, v, cu, kb, vb, scale, part):
    """Per (b, h, i) loops; the KV head is computed as h * H_kv // H_q (an independent form
    of the grouped-query mapping)."""
    b, B, hq, d = q.shape
    hkv = kb.shape[2]
    A = np.zeros((b, B, hq, d))
    L = np.zeros((b, B, hq))
    for bi in range(b):
        for h in range(hq):
            g = h * hkv // hq
            keys, vals = [], []
            if part in ("prefix", "full"):
                keys += [k[t, g] for t in range(cu[bi], cu[bi + 1])]
                vals += [v[t, g] for t in range(cu[bi], cu[bi + 1])]
            if part in ("block", "full"):
                keys += [kb[bi, t, g] for t in range(B)]
                vals += [vb[bi, t, g] for t in range(B)]
            for i in range(B):
                s = np.array([scale * float(np.dot(q[bi, i, h], kk)) for kk in keys])
                mx = s.max()
                w = np.exp(s - mx)
                A[bi, i, h] = sum(w[j] * vals[j] for j in range(len(keys))) / w.sum()
                L[bi, i, h] = mx + math.log(w.sum())
    return A, L


@pytest.mark.parametrize("b,B,hq,hkv,d,lens", [(1, 4, 2, 2, 8, [5]), (2, 3, 4, 2, 4, [6, 1]),
                                                 (3, 2, 8, 2, 3, [2, 7, 4])])
def test_multihead_layouts_brute_force(b, B, hq, hkv, d, lens):
    g = np.random.default_rng(11)
    cu = np.concatenate([[0], np.cumsum(lens)])
    q = g.normal(size=(b, B, hq, d))
    k, v = g.normal(size=(cu[-1], hkv, d)), g.normal(size=(cu[-1], hkv, d))
    kb, vb = g.normal(size=(b, B, hkv, d)), g.normal(size=(b, B, hkv, d))
    for part, fn in (("prefix", lambda: prefix_attention(q, k, v, cu, hkv, 0.4)),
                     ("block", lambda: block_attention(q, kb, vb, 0.4)),
                     ("full", lambda: full_attention(q, k, v, cu, kb, vb, 0.4))):
        A, L = fn()
        Ab, Lb = brute_multihead(q, k, v, cu, kb, vb, 0.4, part)
        np.testing.assert_allclose(A, Ab, rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(L, Lb, rtol=1e-12, atol=1e-13)


@settings(max_examples=25, deadline=None)
@given(B=st.integers(1, 8), n=st.integers(0, 80), d=st.sampled_from([8, 64]),
       heads=st.sampled_from([(1, 1), (2, 1), (4, 2), (4, 4)]), seed=st.integers(0, 999))
def test_split_plus_merge_equals_full_attention(B, n, d, heads, seed):
    """The block-external / block-internal split merged in log space reproduces the unsplit
    softmax over prefix + block, within 1e-12 in fp64 [FB-pt §2]."""
    hq, hkv = heads
    g = np.random.default_rng(seed)
    cu = np.array([0, n])
    q = g.normal(size=(1, B, hq, d))
    k, v = g.normal(size=(n, hkv, d)), g.normal(size=(n, hkv, d))
    kb, vb = g.normal(size=(1, B, hkv, d)), g.normal(size=(1, B, hkv, d))
    s = 1 / math.sqrt(d)
    ao, lo = prefix_attention(q, k, v, cu, hkv, s)
    ai, li = block_attention(q, kb, vb, s)
    am, lm = lse_merge(ao, lo, ai, li)
    af, lf = full_attention(q, k, v, cu, kb, vb, s)
    assert np.max(np.abs(am - af)) <= 1e-12
    assert np.max(np.abs(lm - lf)) <= 1e-12


@pytest.mark.parametrize("splits", [1, 2, 3, 7, 16])
def test_split_count_does_not_change_prefix(splits):
    g = np.random.default_rng(5)
    cu = np.array([0, 50, 53])
    q = g.normal(size=(2, 4, 4, 16))
    k, v = g.normal(size=(53, 2, 16)), g.normal(size=(53, 2, 16))
    a0, l0 = prefix_attention(q, k, v, cu, 2, 0.25)
    a1, l1 = split_prefix_attention(q, k, v, cu, 2, 0.25, splits)
    np.testing.assert_allclose(a1, a0, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(l1, l0, rtol=1e-13)
