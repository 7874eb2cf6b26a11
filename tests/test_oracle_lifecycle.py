"""Pins for oracle/lifecycle.py (block append, page metadata after an append, the steps of a
block under each reuse rule)."""
import numpy as np

import synth
from oracle import attention as A
from oracle import flashblock as F
from oracle import lifecycle as LC
from oracle.losa import page_minmax


def _problem(seed=0, b=2, B=6, hq=4, hkv=2, d=16, lens=(37, 20)):
    return synth.custom(seed, b, hq, hkv, d, B, list(lens), dtype="f32")


def _steps(p, S, seed, sigma):
    """Per-step queries and block K/V: the problem's plus N(0, sigma_h^2) drift per head."""
    g = synth.rng(seed)
    sig = np.asarray(sigma, dtype=np.float32).reshape(1, 1, -1, 1)
    q = np.stack([p.q + (g.standard_normal(p.q.shape, dtype=np.float32) * sig if s else 0) for s in range(S)])
    kb = np.stack([p.k_blk + 0.1 * s * g.standard_normal(p.k_blk.shape, dtype=np.float32) for s in range(S)])
    vb = np.stack([p.v_blk + 0.1 * s * g.standard_normal(p.v_blk.shape, dtype=np.float32) for s in range(S)])
    return q.astype(np.float64), kb.astype(np.float64), vb.astype(np.float64)


def test_append_tokens_by_brute_force():
    p = _problem(1)
    k2, v2, cu2 = LC.append_block(p.k, p.v, p.cu, p.k_blk, p.v_blk)
    assert cu2.tolist() == [0, 37 + 6, 37 + 6 + 20 + 6]
    for bi in range(p.batch):
        n = int(p.seqlens[bi])
        for t in range(n + p.B):
            want_k = p.k[p.cu[bi] + t] if t < n else p.k_blk[bi, t - n]
            want_v = p.v[p.cu[bi] + t] if t < n else p.v_blk[bi, t - n]
            assert (k2[cu2[bi] + t] == want_k).all() and (v2[cu2[bi] + t] == want_v).all()


def test_appended_prefix_is_the_block_causal_key_set():
    """Attention over the grown prefix equals full attention over old prefix + block
    (J_out u J_in of the finished block)."""
    p = _problem(2)
    k2, v2, cu2 = LC.append_block(p.k, p.v, p.cu, p.k_blk, p.v_blk)
    a1, l1 = A.prefix_attention(p.q, k2, v2, cu2, p.h_kv, p.scale)
    a2, l2 = A.full_attention(p.q, p.k, p.v, p.cu, p.k_blk, p.v_blk, p.scale)
    assert np.max(np.abs(a1 - a2)) <= 1e-12 and np.max(np.abs(l1 - l2)) <= 1e-12


def test_page_meta_after_append_keeps_old_full_pages():
    p = _problem(3, lens=(37, 32))
    page = 8
    k2, v2, cu2 = LC.append_block(p.k, p.v, p.cu, p.k_blk, p.v_blk)
    old_min, old_max = page_minmax(p.k, p.cu, page)
    new_min, new_max = LC.page_meta_after_append(k2, cu2, page)
    for bi in range(p.batch):
        full = int(p.seqlens[bi]) // page        # pages with no new token
        assert (new_min[bi][:full] == old_min[bi][:full]).all() and (new_max[bi][:full] == old_max[bi][:full]).all()
        n2 = int(cu2[bi + 1] - cu2[bi])
        kk = k2[cu2[bi]:cu2[bi + 1]]
        for pg in range(len(new_min[bi])):
            seg = [kk[t] for t in range(pg * page, min(n2, (pg + 1) * page))]
            assert (new_min[bi][pg] == np.minimum.reduce(seg)).all()
            assert (new_max[bi][pg] == np.maximum.reduce(seg)).all()


def test_threshold_run_fresh_steps_are_full_attention_and_reuse_keeps_step0():
    p = _problem(4)
    q, kb, vb = _steps(p, 4, 5, [0.5] * p.h_q)
    m = np.array([[99, 99], [9, 0], [0, 9], [9, 9]])       # step 0 ignored; tau 4
    r = LC.block_run(q, p.k, p.v, p.cu, kb, vb, p.scale, "threshold", m_steps=m, tau=4)
    assert (r["masks"][0] == 0).all()
    assert (r["masks"][1] == np.array([[0] * 4, [1] * 4])).all() and (r["masks"][2] == np.array([[1] * 4, [0] * 4])).all()
    for s in range(4):
        af, lf = A.full_attention(q[s], p.k, p.v, p.cu, kb[s], vb[s], p.scale)
        ao, lo = A.prefix_attention(q[s], p.k, p.v, p.cu, p.h_kv, p.scale)
        for bi in range(2):
            last_fresh = max(t for t in range(s + 1) if t == 0 or m[t][bi] >= 4)
            if last_fresh == s:
                assert np.max(np.abs(r["a_full"][s][bi] - af[bi])) <= 1e-12
            else:   # merge of the prefix part computed at the last fresh step with this step's block
                co, cl = A.prefix_attention(q[last_fresh], p.k, p.v, p.cu, p.h_kv, p.scale)
                ai, li = A.block_attention(q[s], kb[s], vb[s], p.scale)
                want, _ = A.lse_merge(co[bi], cl[bi], ai[bi], li[bi])
                assert np.max(np.abs(r["a_full"][s][bi] - want)) <= 1e-12


def test_similarity_run_rule_and_cosines():
    p = _problem(6)
    sig = [1e-3, 1.0, 1e-3, 1.0]                                # heads 0, 2 drift little
    q, kb, vb = _steps(p, 5, 7, sig)
    r = LC.block_run(q, p.k, p.v, p.cu, kb, vb, p.scale, "similarity", gamma=0.95)
    assert (r["masks"][0] == 0).all() and (r["masks"][1] == 0).all() and np.isnan(r["sims"][0]).all()
    for s in range(2, 5):
        assert (r["masks"][s] == (r["sims"][s - 1].astype(np.float32) > np.float32(0.95))).all()
    # after step 1 both steps were computed: the cosine of the two prefix outputs
    a0, _ = A.prefix_attention(q[0], p.k, p.v, p.cu, p.h_kv, p.scale)
    a1, _ = A.prefix_attention(q[1], p.k, p.v, p.cu, p.h_kv, p.scale)
    for bi in range(p.batch):
        for h in range(p.h_q):
            x, y = a0[bi, :, h].reshape(-1), a1[bi, :, h].reshape(-1)
            assert abs(r["sims"][1][bi, h] - x @ y / np.sqrt((x @ x) * (y @ y))) <= 1e-12
    assert (r["masks"][2][:, [0, 2]] == 1).all() and (r["masks"][2][:, [1, 3]] == 0).all()
    # a reusing head's cache does not change, so its similarity is 1 (to rounding) and it keeps reusing
    assert (np.abs(r["sims"][2][:, [0, 2]] - 1.0) <= 1e-15).all() and (r["masks"][3][:, [0, 2]] == 1).all()


def test_similarity_run_extremes():
    p = _problem(8)
    q, kb, vb = _steps(p, 4, 9, [0.3] * p.h_q)
    never = LC.block_run(q, p.k, p.v, p.cu, kb, vb, p.scale, "similarity", gamma=2.0)
    for s in range(4):
        af, _ = A.full_attention(q[s], p.k, p.v, p.cu, kb[s], vb[s], p.scale)
        assert np.max(np.abs(never["a_full"][s] - af)) <= 1e-12
    always = LC.block_run(q, p.k, p.v, p.cu, kb, vb, p.scale, "similarity", gamma=-2.0)
    co, cl = A.prefix_attention(q[1], p.k, p.v, p.cu, p.h_kv, p.scale)
    for s in (2, 3):
        assert (always["masks"][s] == 1).all()
        ai, li = A.block_attention(q[s], kb[s], vb[s], p.scale)
        want, _ = A.lse_merge(co, cl, ai, li)
        assert np.max(np.abs(always["a_full"][s] - want)) <= 1e-12
