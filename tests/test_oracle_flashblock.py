"""Pins for oracle/flashblock.py: the reuse rules, the step semantics and the cosine helper."""
import json
import math
import os

import numpy as np

import synth
from oracle.attention import attend, full_attention, lse_merge
from oracle.flashblock import head_cosine, mask_similarity, mask_threshold, step

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def test_golden_reuse_rules():
    ex = json.load(open(os.path.join(GOLD, "reuse_rules.json")))
    m = mask_threshold(np.array(ex["m_updated"]), ex["tau"], 3)
    assert m.shape == (4, 3) and (m[:, 0] == ex["mask_threshold"]).all() and (m == m[:, :1]).all()
    ms = mask_similarity(np.array([ex["sim"]], dtype=np.float32), ex["gamma"])
    assert ms[0].tolist() == ex["mask_similarity"]


def test_masks_brute_force():
    g = np.random.default_rng(0)
    M = g.integers(0, 9, size=50)
    mt = mask_threshold(M, 4, 5)
    for i in range(50):
        for h in range(5):
            assert mt[i, h] == (1 if M[i] < 4 else 0)
    sim = g.uniform(0.9, 1.0, size=(3, 7)).astype(np.float32)
    ms = mask_similarity(sim, 0.95)
    for i in range(3):
        for h in range(7):
            assert ms[i, h] == (1 if float(sim[i, h]) > float(np.float32(0.95)) else 0)


def test_threshold_reuse_rate_matches_construction():
    """tau = 4 with M ~ U{0..8}: P(reuse) = 4/9 on steps >= 1 (counted on the seeded draws)."""
    g = np.random.default_rng(123)
    M = g.integers(0, 9, size=200_000)
    rate = mask_threshold(M, 4, 1).mean()
    assert abs(rate - 4 / 9) < 0.005


def _problem(seed=0, b=2, B=4, hq=4, hkv=2, d=16, lens=(9, 3)):
    p = synth.custom(seed, b, hq, hkv, d, B, list(lens), dtype="f32")
    return p


def test_fresh_step_equals_full_attention():
    p = _problem()
    mask = np.zeros((p.batch, p.h_q), np.uint8)
    a, l, ca, cl = step(p.q, p.k, p.v, p.cu, p.k_blk, p.v_blk, mask, None, None, p.scale)
    af, lf = full_attention(p.q, p.k, p.v, p.cu, p.k_blk, p.v_blk, p.scale)
    assert np.max(np.abs(a - af)) <= 1e-12 and np.max(np.abs(l - lf)) <= 1e-12


def test_reuse_with_unchanged_inputs_is_bit_identical():
    p = _problem(1)
    z = np.zeros((p.batch, p.h_q), np.uint8)
    a0, l0, ca, cl = step(p.q, p.k, p.v, p.cu, p.k_blk, p.v_blk, z, None, None, p.scale)
    a1, l1, ca1, cl1 = step(p.q, p.k, p.v, p.cu, p.k_blk, p.v_blk, 1 - z, ca, cl, p.scale)
    a2, l2, ca2, cl2 = step(p.q, p.k, p.v, p.cu, p.k_blk, p.v_blk, z, ca, cl, p.scale)
    for x, y in ((a1, a2), (l1, l2), (ca1, ca2), (cl1, cl2), (a0, a1)):
        assert np.array_equal(x, y)


def test_reuse_step_semantics():
    """mask 1: the cache is untouched and A_full merges the stale cache with the new block
    part; mask 0: the cache is recomputed from the new queries."""
    p = _problem(2)
    z = np.zeros((p.batch, p.h_q), np.uint8)
    _, _, ca, cl = step(p.q, p.k, p.v, p.cu, p.k_blk, p.v_blk, z, None, None, p.scale)
    q2 = p.q + 0.3 * np.random.default_rng(9).normal(size=p.q.shape)
    kb2 = p.k_blk + 0.3
    mask = np.array([[1, 0, 1, 0], [0, 0, 1, 1]], np.uint8)
    a, l, ca2, cl2 = step(q2, p.k, p.v, p.cu, kb2, p.v_blk, mask, ca, cl, p.scale)
    hkv = p.h_kv
    for b in range(p.batch):
        lo, hi = p.cu[b], p.cu[b + 1]
        for h in range(p.h_q):
            g = h * hkv // p.h_q
            ai, li = attend(q2[b, :, h], kb2[b, :, g], p.v_blk[b, :, g], p.scale)
            if mask[b, h]:
                assert np.array_equal(ca2[b, :, h], ca[b, :, h]) and np.array_equal(cl2[b, :, h], cl[b, :, h])
                exp_a, exp_l = lse_merge(ca[b, :, h], cl[b, :, h], ai, li)
            else:
                ao, lo_ = attend(q2[b, :, h], p.k[lo:hi, g], p.v[lo:hi, g], p.scale)
                np.testing.assert_allclose(ca2[b, :, h], ao, rtol=1e-13, atol=1e-14)
                np.testing.assert_allclose(cl2[b, :, h], lo_, rtol=1e-13)
                kk = np.concatenate([p.k[lo:hi, g], kb2[b, :, g]])
                vv = np.concatenate([p.v[lo:hi, g], p.v_blk[b, :, g]])
                exp_a, exp_l = attend(q2[b, :, h], kk, vv, p.scale)
            np.testing.assert_allclose(a[b, :, h], exp_a, rtol=1e-12, atol=1e-13)
            np.testing.assert_allclose(l[b, :, h], exp_l, rtol=1e-12, atol=1e-13)


def test_tiny_workload_two_steps():
    """The tiny fp32 workload: a fresh step, then a reuse step with perturbed queries."""
    p = synth.tiny()
    z = np.zeros((1, 2), np.uint8)
    a0, l0, ca, cl = step(p.q, p.k, p.v, p.cu, p.k_blk, p.v_blk, z, None, None, p.scale)
    af, lf = full_attention(p.q, p.k, p.v, p.cu, p.k_blk, p.v_blk, p.scale)
    assert np.max(np.abs(a0 - af)) <= 1e-12
    q1 = p.extra["q_step1"]
    a1, l1, ca1, cl1 = step(q1, p.k, p.v, p.cu, p.k_blk, p.v_blk, 1 - z, ca, cl, p.scale)
    assert np.array_equal(ca1, ca)
    af1, _ = full_attention(q1, p.k, p.v, p.cu, p.k_blk, p.v_blk, p.scale)
    assert 0 < np.max(np.abs(a1 - af1)) < 0.05      # stale prefix: close to, not equal to, dense


def test_head_cosine_closed_forms():
    g = np.random.default_rng(4)
    a = g.normal(size=(2, 5, 3, 8))
    s = head_cosine(a, a)
    np.testing.assert_allclose(s, 1.0, rtol=1e-14)
    np.testing.assert_allclose(head_cosine(a, -a), -1.0, rtol=1e-14)
    np.testing.assert_allclose(head_cosine(a, 3.5 * a), 1.0, rtol=1e-14)
    x = np.zeros((1, 1, 1, 2)); x[..., 0] = 1
    y = np.zeros((1, 1, 1, 2)); y[..., 1] = 1
    assert head_cosine(x, y)[0, 0] == 0.0
    assert head_cosine(x, np.zeros_like(x))[0, 0] == 0.0
    b = g.normal(size=(2, 5, 3, 8))
    for i in range(2):
        for h in range(3):
            u, w = a[i, :, h].ravel().tolist(), b[i, :, h].ravel().tolist()
            dot = sum(x_ * y_ for x_, y_ in zip(u, w))
            ref = dot / math.sqrt(sum(x_ * x_ for x_ in u) * sum(y_ * y_ for y_ in w))
            assert abs(head_cosine(a, b)[i, h] - ref) < 1e-13


def test_video_similarity_draws_give_seven_of_twelve():
    p = synth.video(n_prefix=16, block=8)
    m = mask_similarity(p.extra["sim"], p.extra["gamma"])
    assert m.sum() == 7 and m.shape == (1, 12)
