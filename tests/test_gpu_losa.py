"""GPU parity of the LoSA-style sparse path through the C ABI against the fp64 oracle.
Indices (active set, top-k pages, union) must match bit for bit."""
import numpy as np
import pytest

import synth
from synth.device import tensor, to_device
from oracle import losa as OL
from oracle.attention import prefix_attention
from tests.gpu_util import check_attn, check_lse, guarded, guarded_copy, np_of, say, to_device_guarded

pytestmark = pytest.mark.gpu


def _setup(fb, p, q_cur, q_prev, n_active, page, topk):
    import torch
    dev = to_device_guarded(p)
    code = fb.FB_BF16 if p.dtype == "bf16" else fb.FB_F32
    if p.batch == 1:
        s = fb.make_shape(p.batch, p.h_q, p.h_kv, p.d, p.B, dtype=code, seqlen_k=int(p.seqlens[0]))
    else:
        s = fb.make_shape(p.batch, p.h_q, p.h_kv, p.d, p.B, dtype=code, cu_seqlens_k=dev["cu"],
                          max_seqlen_k=int(p.seqlens.max()))
    ls = fb.make_losa_shape(s, page_size=page, topk=topk, n_active=n_active)
    el = 2 if p.dtype == "bf16" else 4
    nb = fb.losa_meta_bytes(ls)
    kmin = guarded((nb // el,), dev["k"].dtype, name="kmin")
    kmax = guarded((nb // el,), dev["k"].dtype, name="kmax")
    fb.losa_page_meta(ls, dev["k"], kmin, kmax)
    cap = fb.losa_union_capacity(ls)
    out = dict(
        active=guarded((p.batch, n_active), torch.int32, -7, "active"),
        topk=guarded((p.batch, p.h_q, n_active, topk), torch.int32, -7, "topk_pages"),
        union=guarded((p.batch, p.h_kv, cap), torch.int32, -7, "union_pages"),
        count=guarded((p.batch, p.h_kv), torch.int32, -7, "union_count"),
        ws=guarded((fb.losa_workspace_size(ls),), torch.uint8, name="losa workspace"),
    )
    dev.update(q_cur=tensor(q_cur, p.dtype), q_prev=tensor(q_prev, p.dtype), kmin=kmin, kmax=kmax)
    for key in ("q_cur", "q_prev"):
        dev[key] = guarded_copy(dev[key], key)
    return dev, s, ls, out


def _meta_as_pages(t, p, ls):
    b, hk, d = p.batch, p.h_kv, p.d
    x = np_of(t).reshape(b, hk, d // 8, ls.max_pages, 8)
    return x.transpose(0, 3, 1, 2, 4).reshape(b, ls.max_pages, hk, d)


def _check_selection(p, out, exp, n_active):
    act = np_of(out["active"])
    assert (act == exp["active"]).all(), (act, exp["active"])
    tk = np_of(out["topk"])
    assert (tk == exp["topk"]).all(), f"top-k pages differ at {np.argwhere(tk != exp['topk'])[:5]}"
    cnt, uni = np_of(out["count"]), np_of(out["union"])
    for b in range(p.batch):
        for g in range(p.h_kv):
            e = exp["unions"][b][g]
            assert cnt[b, g] == len(e)
            assert (uni[b, g, :len(e)] == e).all()


SMALL = [
    # name, batch, h_q, h_kv, d, B, lens, n_active, page, topk, dtype
    ("mha_bf16", 1, 4, 4, 128, 16, [1000], 3, 16, 8, "bf16"),
    ("gqa_tail_pages", 2, 8, 2, 128, 24, [517, 93], 4, 16, 5, "bf16"),
    ("few_pages", 1, 2, 1, 64, 8, [40], 2, 16, 8, "bf16"),
    ("page1", 1, 2, 2, 64, 8, [70], 2, 1, 9, "bf16"),
    ("f32", 1, 2, 1, 64, 8, [300], 3, 16, 4, "f32"),
    # the active set is ranked inside the page-score launch up to 256 block tokens, in a
    # launch of its own above that
    ("block256_rank_in_quest", 1, 2, 2, 64, 256, [400], 7, 16, 5, "bf16"),
    ("block300_rank_own_launch", 1, 2, 2, 64, 300, [500], 5, 16, 6, "bf16"),
    # top-k above 256: the selection runs over all keys (no threshold from the thread maxima)
    ("topk300_over_all_keys", 1, 2, 2, 64, 8, [1000], 2, 1, 300, "bf16"),
    # every block token active (no stable rows)
    ("all_active", 1, 2, 2, 64, 8, [300], 8, 16, 4, "bf16"),
    # one sequence with an empty prefix: no pages, an empty union, the cache stays (0, -inf)
    ("empty_prefix_sequence", 2, 4, 2, 64, 8, [0, 200], 3, 16, 4, "bf16"),
    # a page size that is not a power of two (token = page * 12 + offset)
    ("page12", 1, 4, 2, 128, 16, [777], 3, 12, 6, "bf16"),
    # 4 query heads x 8 active tokens = 32 rows per KV head, the most the streaming pass takes
    ("gqa4_32_active_rows", 1, 8, 2, 128, 32, [2000], 8, 16, 16, "bf16"),
]


@pytest.mark.parametrize("case", SMALL, ids=[c[0] for c in SMALL])
def test_select_union_and_step_small(gpu_lib, case):
    import torch
    fb = gpu_lib
    name, b, hq, hkv, d, B, lens, nA, page, topk, dt = case
    say(f"[losa] {name}")
    p = synth.custom(21, b, hq, hkv, d, B, lens, dtype=dt, std=1.0)
    g = synth.rng(22)
    q_prev = p.q
    noise = g.standard_normal(p.q.shape, dtype=np.float32) * 0.01
    noise[:, ::3] *= 30.0
    q_cur = synth.round_bf16(q_prev + noise) if dt == "bf16" else (q_prev + noise).astype(np.float32)
    dev, s, ls, out = _setup(fb, p, q_cur, q_prev, nA, page, topk)
    torch.cuda.synchronize()
    mins, maxs = OL.page_minmax(p.k, p.cu, page)
    gmin, gmax = _meta_as_pages(dev["kmin"], p, ls), _meta_as_pages(dev["kmax"], p, ls)
    for bi in range(b):
        P = mins[bi].shape[0]
        assert (gmin[bi, :P] == mins[bi]).all() and (gmax[bi, :P] == maxs[bi]).all()
    fb.losa_select_union(ls, dev["q_cur"], dev["q_prev"], dev["kmin"], dev["kmax"], out["active"], out["topk"],
                         out["union"], out["count"], out["ws"])
    torch.cuda.synchronize()
    exp = OL.select_union(q_cur, q_prev, p.k, p.cu, hkv, nA, page, topk)
    _check_selection(p, out, exp, nA)

    # full sparse step on top of a cache filled by a dense step on q_prev
    ca = guarded((b, B, hq, d), torch.float32, 0.0, "cache_a")
    cl = guarded((b, B, hq), torch.float32, 0.0, "cache_l")
    a_full = guarded((b, B, hq, d), dev["q"].dtype, 0.0, "a_full")
    l_full = guarded((b, B, hq), torch.float32, 0.0, "l_full")
    ws = guarded((max(fb.workspace_size(s), 16),), torch.uint8, name="step workspace")
    fb.step(s, dev["q_prev"], dev["k"], dev["v"], dev["k_blk"], dev["v_blk"], None, ca, cl, a_full, l_full, ws)
    torch.cuda.synchronize()
    cache0_a, cache0_l = np_of(ca).astype(np.float64), np_of(cl).astype(np.float64)
    ea0, el0 = prefix_attention(q_prev, p.k, p.v, p.cu, hkv, p.scale)
    check_attn(cache0_a, ea0, dt, f"{name} dense cache")
    for k_ in ("active", "topk", "union", "count"):
        out[k_].fill_(-7)
    fb.losa_step(ls, dev["q_cur"], dev["q_prev"], dev["k"], dev["v"], dev["k_blk"], dev["v_blk"], dev["kmin"],
                 dev["kmax"], ca, cl, a_full, l_full, out["active"], out["topk"], out["union"], out["count"],
                 out["ws"])
    torch.cuda.synchronize()
    _check_selection(p, out, exp, nA)
    # the oracle continues from its own dense cache (an all-oracle chain)
    ea, el, na, nl, _ = OL.step(q_cur, q_prev, p.k, p.v, p.cu, p.k_blk, p.v_blk, ea0, el0, nA, page, topk, p.scale)
    check_attn(np_of(a_full), ea, dt, f"{name} A_full")
    check_lse(np_of(l_full), el, dt, f"{name} L_full")
    check_attn(np_of(ca), na, dt, f"{name} new cache")
    check_lse(np_of(cl), nl, dt, f"{name} new cache L")
    stable = np.ones(B, bool)
    stable[exp["active"][0]] = False
    assert (np_of(ca)[0, stable] == cache0_a[0, stable]).all()


def test_topk_ties_go_to_lower_pages(gpu_lib):
    """Keys repeat with a period of 4 pages, so page scores tie in groups; the selection
    must keep the lowest page indices of each tied group (bit-exact with the oracle)."""
    import torch
    fb = gpu_lib
    p = synth.custom(5, 1, 2, 2, 64, 8, [16 * 40], std=1.0)
    p.k = np.tile(p.k[:64], (10, 1, 1))
    q_prev = p.q
    q_cur = synth.round_bf16(p.q + 0.5 * synth.rng(6).standard_normal(p.q.shape, dtype=np.float32))
    dev, s, ls, out = _setup(fb, p, q_cur, q_prev, 3, 16, 6)
    fb.losa_select_union(ls, dev["q_cur"], dev["q_prev"], dev["kmin"], dev["kmax"], out["active"], out["topk"],
                         out["union"], out["count"], out["ws"])
    torch.cuda.synchronize()
    exp = OL.select_union(q_cur, q_prev, p.k, p.cu, 2, 3, 16, 6)
    _check_selection(p, out, exp, 3)
    assert np_of(out["topk"]).max() < 40


def test_topk_all_scores_equal_take_the_lowest_pages(gpu_lib):
    """Every page holds the same keys, so all 2000 page scores are equal: more keys pass the
    top-k threshold than the candidate buffer holds, the selection runs over all keys, and
    each row takes the lowest pages (bit-exact with the oracle)."""
    import torch
    fb = gpu_lib
    say("[losa] top-k with 2000 equal page scores")
    p = synth.custom(8, 1, 2, 2, 64, 8, [16 * 2000], std=1.0)
    p.k = np.tile(p.k[:16], (2000, 1, 1))
    q_prev = p.q
    q_cur = synth.round_bf16(p.q + 0.5 * synth.rng(9).standard_normal(p.q.shape, dtype=np.float32))
    dev, s, ls, out = _setup(fb, p, q_cur, q_prev, 3, 16, 64)
    fb.losa_select_union(ls, dev["q_cur"], dev["q_prev"], dev["kmin"], dev["kmax"], out["active"], out["topk"],
                         out["union"], out["count"], out["ws"])
    torch.cuda.synchronize()
    exp = OL.select_union(q_cur, q_prev, p.k, p.cu, 2, 3, 16, 64)
    assert (exp["topk"] == np.arange(64)).all()
    _check_selection(p, out, exp, 3)


@pytest.mark.parametrize("B", [16, 300])
def test_active_set_ties_go_to_lower_tokens(gpu_lib, B):
    """Unchanged queries give every block token the locality score 0: the active set is
    then the lowest tokens, on both ranking paths (inside the page-score launch, and in a
    launch of its own for blocks of more than 256 tokens)."""
    import torch
    fb = gpu_lib
    say(f"[losa] ranking ties, B {B}")
    p = synth.custom(7, 1, 2, 2, 64, B, [200], std=1.0)
    dev, s, ls, out = _setup(fb, p, p.q, p.q, 5, 16, 4)
    fb.losa_select_union(ls, dev["q_cur"], dev["q_prev"], dev["kmin"], dev["kmax"], out["active"], out["topk"],
                         out["union"], out["count"], out["ws"])
    torch.cuda.synchronize()
    exp = OL.select_union(p.q, p.q, p.k, p.cu, 2, 5, 16, 4)
    assert (exp["active"] == np.arange(5)).all()
    _check_selection(p, out, exp, 5)


def test_losa_full_size(gpu_lib):
    """The LoSA workload at full size: prefix 131072 (8192 pages of 16), B 64, 32 heads,
    |A| 8, top-64 pages.  Selection bit-exact; A_full on every row against the oracle."""
    import torch
    fb = gpu_lib
    p = synth.losa()
    q_cur, q_prev = p.extra["q_cur"], p.extra["q_prev"]
    dev, s, ls, out = _setup(fb, p, q_cur, q_prev, 8, 16, 64)
    say("[losa full] dense step 0")
    ca = guarded((1, 64, 32, 128), torch.float32, 0.0, "cache_a")
    cl = guarded((1, 64, 32), torch.float32, 0.0, "cache_l")
    a_full = guarded((1, 64, 32, 128), torch.bfloat16, 0.0, "a_full")
    l_full = guarded((1, 64, 32), torch.float32, 0.0, "l_full")
    ws = guarded((fb.workspace_size(s),), torch.uint8, name="step workspace")
    fb.step(s, dev["q_prev"], dev["k"], dev["v"], dev["k_blk"], dev["v_blk"], None, ca, cl, a_full, l_full, ws)
    torch.cuda.synchronize()
    cache0_a, cache0_l = np_of(ca).astype(np.float64), np_of(cl).astype(np.float64)
    say("[losa full] sparse step")
    fb.losa_step(ls, dev["q_cur"], dev["q_prev"], dev["k"], dev["v"], dev["k_blk"], dev["v_blk"], dev["kmin"],
                 dev["kmax"], ca, cl, a_full, l_full, out["active"], out["topk"], out["union"], out["count"],
                 out["ws"])
    torch.cuda.synchronize()
    say("[losa full] oracle (dense step 0, then the sparse step on the oracle's own cache)")
    ea0, el0 = prefix_attention(q_prev, p.k, p.v, p.cu, p.h_kv, p.scale)
    check_attn(cache0_a, ea0, "bf16", "losa dense cache")
    ea, el, na, nl, sel = OL.step(q_cur, q_prev, p.k, p.v, p.cu, p.k_blk, p.v_blk, ea0, el0, 8, 16, 64, p.scale)
    assert (sel["active"][0] == p.extra["moved"]).all()
    _check_selection(p, out, sel, 8)
    check_attn(np_of(a_full), ea, "bf16", "losa A_full")
    check_lse(np_of(l_full), el, "bf16", "losa L_full")
    check_attn(np_of(ca), na, "bf16", "losa cache")
    check_lse(np_of(cl), nl, "bf16", "losa cache L")
    stable = np.ones(64, bool)
    stable[sel["active"][0]] = False
    assert (np_of(ca)[0, stable] == cache0_a[0, stable]).all()
    say(f"[losa full] union pages per head: mean {np_of(out['count']).mean():.1f} of 8192")
