"""Pins for oracle/residual.py (FlashBlock with a cached sparse-attention residual)."""
import numpy as np

import synth
from oracle.attention import attend, full_attention, lse_merge
from oracle.residual import complement_pages, lse_merge3, page_tokens, selected_and_residual, step


def _problem(seed=0, b=2, B=5, hq=4, hkv=2, d=16, lens=(37, 21)):
    return synth.custom(seed, b, hq, hkv, d, B, list(lens), dtype="f32")


def _selections(p, page, seed=0):
    """Per (sequence, KV head): an empty set, every page, and random subsets (one includes
    the tail page)."""
    g = np.random.default_rng(seed)
    sel = []
    for bi in range(p.batch):
        n = int(p.seqlens[bi])
        P = (n + page - 1) // page
        row = []
        for hk in range(p.h_kv):
            kind = (bi + hk) % 3
            if kind == 0:
                row.append(np.zeros(0, np.int64))
            elif kind == 1:
                row.append(np.arange(P))
            else:
                s = np.sort(g.choice(P, size=max(1, P // 2), replace=False))
                row.append(np.unique(np.concatenate([s, [P - 1]])))
        sel.append(row)
    return sel


def test_complement_pages_brute_force():
    g = np.random.default_rng(3)
    for _ in range(50):
        P = int(g.integers(0, 40))
        sel = g.choice(max(P, 1), size=int(g.integers(0, max(P, 1) + 1)), replace=False) if P else np.zeros(0, int)
        comp = complement_pages(sel, P)
        assert comp.tolist() == [x for x in range(P) if x not in set(sel.tolist())]


def test_page_tokens_drop_tokens_past_the_prefix():
    assert page_tokens([0, 2], 4, 10).tolist() == [0, 1, 2, 3, 8, 9]
    assert page_tokens([], 4, 10).tolist() == []


def test_merge3_against_two_way_merges_and_permutations():
    g = np.random.default_rng(4)
    a = [g.standard_normal((6, 8)) for _ in range(3)]
    l = [g.standard_normal(6) * 3 for _ in range(3)]
    A, L = lse_merge3(a[0], l[0], a[1], l[1], a[2], l[2])
    A12, L12 = lse_merge(a[0], l[0], a[1], l[1])
    A2, L2 = lse_merge(A12, L12, a[2], l[2])
    assert np.max(np.abs(A - A2)) <= 1e-13 and np.max(np.abs(L - L2)) <= 1e-13
    for perm in ([1, 2, 0], [2, 0, 1], [0, 2, 1]):
        Ap, Lp = lse_merge3(a[perm[0]], l[perm[0]], a[perm[1]], l[perm[1]], a[perm[2]], l[perm[2]])
        assert np.max(np.abs(A - Ap)) <= 1e-13 and np.max(np.abs(L - Lp)) <= 1e-13
    # closed forms: three equal parts; one or all parts empty
    A3, L3 = lse_merge3(a[0], l[0], a[0], l[0], a[0], l[0])
    assert np.max(np.abs(A3 - a[0])) <= 1e-14 and np.max(np.abs(L3 - (l[0] + np.log(3.0)))) <= 1e-13
    ninf = np.full(6, -np.inf)
    Ae, Le = lse_merge3(a[0], l[0], np.zeros((6, 8)), ninf, a[1], l[1])
    A01, L01 = lse_merge(a[0], l[0], a[1], l[1])
    assert np.max(np.abs(Ae - A01)) <= 1e-14 and np.max(np.abs(Le - L01)) <= 1e-14
    Z, LZ = lse_merge3(np.zeros((6, 8)), ninf, np.zeros((6, 8)), ninf, np.zeros((6, 8)), ninf)
    assert (Z == 0).all() and np.isneginf(LZ).all()


def test_refresh_step_equals_full_attention():
    """Selected pages + residual + block cover every key exactly once, so a refresh step is
    full attention over prefix and block, whatever the selection."""
    for seed, page in ((0, 4), (1, 8), (2, 16)):
        p = _problem(seed)
        sel = _selections(p, page, seed)
        mask = np.zeros((p.batch, p.h_q), np.uint8)
        a, l, ca, cl = step(p.q, p.k, p.v, p.cu, p.k_blk, p.v_blk, sel, page, mask,
                            np.zeros_like(p.q, dtype=np.float64), np.zeros(p.q.shape[:3]), p.scale)
        af, lf = full_attention(p.q, p.k, p.v, p.cu, p.k_blk, p.v_blk, p.scale)
        assert np.max(np.abs(a - af)) <= 1e-12 and np.max(np.abs(l - lf)) <= 1e-12


def test_selected_part_by_brute_force():
    p = _problem(5, b=1, lens=(23,))
    page = 4
    sel = [[np.array([0, 3, 5]), np.array([1, 2])]]
    As, Ls, Ar, Lr = selected_and_residual(p.q, p.k, p.v, p.cu, sel, page, p.scale)
    for h in range(p.h_q):
        g = h // (p.h_q // p.h_kv)
        toks = [t for t in range(23) if (t // page) in set(sel[0][g].tolist())]
        rest = [t for t in range(23) if t not in toks]
        ea, el = attend(p.q[0, :, h], p.k[toks, g], p.v[toks, g], p.scale)
        ra, rl = attend(p.q[0, :, h], p.k[rest, g], p.v[rest, g], p.scale)
        assert np.max(np.abs(As[0, :, h] - ea)) <= 1e-14 and np.max(np.abs(Ar[0, :, h] - ra)) <= 1e-14
        assert np.max(np.abs(Ls[0, :, h] - el)) <= 1e-14 and np.max(np.abs(Lr[0, :, h] - rl)) <= 1e-14


def test_reuse_with_unchanged_inputs_equals_refresh_and_keeps_the_cache():
    p = _problem(6)
    page = 4
    sel = _selections(p, page, 6)
    z = np.zeros((p.batch, p.h_q), np.uint8)
    c0a, c0l = np.zeros_like(p.q, dtype=np.float64), np.zeros(p.q.shape[:3])
    a1, l1, ca, cl = step(p.q, p.k, p.v, p.cu, p.k_blk, p.v_blk, sel, page, z, c0a, c0l, p.scale)
    one = np.ones_like(z)
    a2, l2, ca2, cl2 = step(p.q, p.k, p.v, p.cu, p.k_blk, p.v_blk, sel, page, one, ca, cl, p.scale)
    assert np.array_equal(a1, a2) and np.array_equal(l1, l2)
    assert np.array_equal(ca, ca2) and np.array_equal(cl, cl2)


def test_stale_residual_persists_and_only_reusing_heads_keep_it():
    p = _problem(7)
    page = 8
    sel = _selections(p, page, 7)
    z = np.zeros((p.batch, p.h_q), np.uint8)
    c0a, c0l = np.zeros_like(p.q, dtype=np.float64), np.zeros(p.q.shape[:3])
    _, _, ca, cl = step(p.q, p.k, p.v, p.cu, p.k_blk, p.v_blk, sel, page, z, c0a, c0l, p.scale)
    q2 = p.q * 0.5
    mask = np.zeros((p.batch, p.h_q), np.uint8)
    mask[:, ::2] = 1                              # even heads reuse, odd heads refresh
    _, _, ca2, cl2 = step(q2, p.k, p.v, p.cu, p.k_blk, p.v_blk, sel, page, mask, ca, cl, p.scale)
    assert np.array_equal(ca2[:, :, ::2], ca[:, :, ::2]) and np.array_equal(cl2[:, :, ::2], cl[:, :, ::2])
    _, _, ar, lr = selected_and_residual(q2, p.k, p.v, p.cu, sel, page, p.scale)
    assert np.array_equal(ca2[:, :, 1::2], ar[:, :, 1::2]) and np.array_equal(cl2[:, :, 1::2], lr[:, :, 1::2])
