"""GPU parity of FlashBlock with a cached sparse residual (fb_residual_step) through the C
ABI against the fp64 oracle (oracle/residual.py)."""
import numpy as np
import pytest

import synth
from synth.device import tensor, to_device
from oracle import residual as OR
from tests.gpu_util import check_attn, check_lse, guarded, np_of, say, to_device_guarded

pytestmark = pytest.mark.gpu


def _shape(fb, p, page, max_sel):
    dev = to_device_guarded(p)
    code = fb.FB_BF16 if p.dtype == "bf16" else fb.FB_F32
    if p.batch == 1:
        s = fb.make_shape(p.batch, p.h_q, p.h_kv, p.d, p.B, dtype=code, seqlen_k=int(p.seqlens[0]))
    else:
        s = fb.make_shape(p.batch, p.h_q, p.h_kv, p.d, p.B, dtype=code, cu_seqlens_k=dev["cu"],
                          max_seqlen_k=int(p.seqlens.max()))
    rs = fb.make_residual_shape(s, page_size=page, max_sel=max_sel)
    return dev, s, rs


def _bufs(fb, p, rs, dev):
    import torch
    b, B, hq, d = p.batch, p.B, p.h_q, p.d
    return dict(ca=guarded((b, B, hq, d), torch.float32, 7.0, "cache_a"),
                cl=guarded((b, B, hq), torch.float32, 7.0, "cache_l"),
                af=guarded((b, B, hq, d), dev["q"].dtype, 0.0, "a_full"),
                lf=guarded((b, B, hq), torch.float32, 0.0, "l_full"),
                ws=guarded((fb.residual_workspace_size(rs),), torch.uint8, name="workspace"))


def _sel_dev(sel, max_sel, seed):
    import torch
    pages, count = synth.pack_selection(sel, max_sel, shuffle_seed=seed)
    return torch.from_numpy(pages).cuda(), torch.from_numpy(count).cuda()


def _run(fb, rs, q, dev, sp, sc, mask, bf):
    fb.residual_step(rs, q, dev["k"], dev["v"], dev["k_blk"], dev["v_blk"], sp, sc, mask, bf["ca"], bf["cl"], bf["af"],
                     bf["lf"], bf["ws"])


SMALL = [
    # name, batch, h_q, h_kv, d, B, lens, page, n_sel, dtype
    ("mha_stream", 1, 4, 4, 128, 16, [1000], 16, 20, "bf16"),
    ("gqa_ragged_stream", 2, 8, 2, 128, 8, [517, 93], 16, 9, "bf16"),
    ("rows64_tiled", 1, 2, 2, 128, 64, [700], 16, 11, "bf16"),
    ("rows64_page256", 1, 4, 2, 128, 32, [3000], 256, 5, "bf16"),
    ("gqa_rows128_page32", 2, 8, 2, 128, 32, [2100, 700], 32, 30, "bf16"),
    ("rows160_generic", 1, 5, 1, 128, 32, [800], 16, 12, "bf16"),
    ("page8", 1, 4, 2, 128, 16, [333], 8, 13, "bf16"),
    ("page48_long", 1, 2, 2, 128, 16, [9000], 48, 40, "bf16"),
    ("d64", 2, 4, 2, 64, 8, [260, 129], 16, 6, "bf16"),
    ("f32", 1, 4, 2, 64, 8, [300], 16, 5, "f32"),
    ("empty_prefix", 1, 2, 2, 128, 8, [0], 16, 1, "bf16"),
]


@pytest.mark.parametrize("case", SMALL, ids=[c[0] for c in SMALL])
def test_residual_steps_small(gpu_lib, case):
    """Refresh step, then a mixed step (even heads reuse, new queries, new selection), then
    reuse == refresh bit for bit on unchanged inputs."""
    import torch
    fb = gpu_lib
    name, b, hq, hkv, d, B, lens, page, n_sel, dt = case
    say(f"[residual] {name}")
    p = synth.custom(31, b, hq, hkv, d, B, lens, dtype=dt, std=1.0)
    max_pages = max(1, max(-(-n // page) for n in lens))
    max_sel = max(1, min(max_pages, n_sel + 3))
    dev, s, rs = _shape(fb, p, page, max_sel)
    kinds = ("tail", "empty", "all", "random") if max_sel >= max_pages else ("tail", "empty", "random")
    sel1 = synth.page_selection(32, p.seqlens, hkv, page, min(n_sel, max_sel), kinds)
    sel2 = synth.page_selection(33, p.seqlens, hkv, page, min(n_sel, max_sel), kinds[::-1])
    bf = _bufs(fb, p, rs, dev)

    # step 1: refresh every head
    sp, sc = _sel_dev(sel1, max_sel, 34)
    _run(fb, rs, dev["q"], dev, sp, sc, None, bf)
    torch.cuda.synchronize()
    z = np.zeros((b, hq), np.uint8)
    c0a, c0l = np.zeros((b, B, hq, d)), np.zeros((b, B, hq))
    ea, el, na, nl = OR.step(p.q, p.k, p.v, p.cu, p.k_blk, p.v_blk, sel1, page, z, c0a, c0l, p.scale)
    check_attn(np_of(bf["af"]), ea, dt, f"{name} refresh A_full")
    check_lse(np_of(bf["lf"]), el, dt, f"{name} refresh L_full")
    check_attn(np_of(bf["ca"]), na, dt, f"{name} refresh residual")
    check_lse(np_of(bf["cl"]), nl, dt, f"{name} refresh residual L")

    # step 2: even heads reuse the cache; new queries and a new selection.  The oracle
    # continues from its own step-1 cache (an all-oracle chain); the GPU's reused rows must
    # stay bit for bit what the GPU wrote in step 1.
    cache1_a, cache1_l = np_of(bf["ca"]).astype(np.float64), np_of(bf["cl"]).astype(np.float64)
    o1a, o1l = na, nl
    g = synth.rng(35)
    q2 = p.q + 0.1 * g.standard_normal(p.q.shape, dtype=np.float32)
    q2 = synth.round_bf16(q2) if dt == "bf16" else q2.astype(np.float32)
    mask = np.zeros((b, hq), np.uint8)
    mask[:, ::2] = 1
    sp, sc = _sel_dev(sel2, max_sel, 36)
    q2d = tensor(q2, dt)
    _run(fb, rs, q2d, dev, sp, sc, torch.from_numpy(mask).cuda(), bf)
    torch.cuda.synchronize()
    ea, el, na, nl = OR.step(q2, p.k, p.v, p.cu, p.k_blk, p.v_blk, sel2, page, mask, o1a, o1l, p.scale)
    check_attn(np_of(bf["af"]), ea, dt, f"{name} mixed A_full")
    check_lse(np_of(bf["lf"]), el, dt, f"{name} mixed L_full")
    ga, gl = np_of(bf["ca"]), np_of(bf["cl"])
    assert (ga[:, :, ::2] == cache1_a[:, :, ::2]).all() and (gl[:, :, ::2] == cache1_l[:, :, ::2]).all()
    check_attn(ga, na, dt, f"{name} mixed residual")
    check_lse(gl, nl, dt, f"{name} mixed residual L")

    # reuse with unchanged inputs and cache gives the refresh output bit for bit
    _run(fb, rs, q2d, dev, sp, sc, None, bf)
    torch.cuda.synchronize()
    af_ref, lf_ref = bf["af"].clone(), bf["lf"].clone()
    ca_ref, cl_ref = bf["ca"].clone(), bf["cl"].clone()
    _run(fb, rs, q2d, dev, sp, sc, torch.ones((b, hq), dtype=torch.uint8, device="cuda"), bf)
    torch.cuda.synchronize()
    assert torch.equal(bf["af"], af_ref) and torch.equal(bf["lf"], lf_ref)
    assert torch.equal(bf["ca"], ca_ref) and torch.equal(bf["cl"], cl_ref)


def test_residual_full_size(gpu_lib):
    """The sparse workload's shape at full size (prefix 131072 = 8192 pages of 16, B 64, 32
    heads, 512 selected pages per head): a refresh step on every row, then a reuse step with
    new queries, both against the oracle; heads are sampled to bound the oracle's time."""
    import torch
    fb = gpu_lib
    p = synth.losa()
    page, n_sel = 16, 512
    sel = synth.page_selection(synth.SEED_RESIDUAL, p.seqlens, p.h_kv, page, n_sel, ("tail", "random"))
    dev, s, rs = _shape(fb, p, page, n_sel)
    bf = _bufs(fb, p, rs, dev)
    sp, sc = _sel_dev(sel, n_sel, synth.SEED_RESIDUAL + 1)
    q1, q2 = p.extra["q_prev"], p.extra["q_cur"]
    say("[residual full] refresh step")
    _run(fb, rs, tensor(q1), dev, sp, sc, None, bf)
    torch.cuda.synchronize()
    cache_a, cache_l = np_of(bf["ca"]).astype(np.float64), np_of(bf["cl"]).astype(np.float64)
    af1, lf1 = np_of(bf["af"]), np_of(bf["lf"])
    say("[residual full] reuse step")
    _run(fb, rs, tensor(q2), dev, sp, sc, torch.ones((1, 32), dtype=torch.uint8, device="cuda"), bf)
    torch.cuda.synchronize()
    af2, lf2 = np_of(bf["af"]), np_of(bf["lf"])
    assert (np_of(bf["ca"]) == cache_a).all()
    heads = [0, 13, 31]
    hsel = [[sel[0][h] for h in heads]]
    sub = lambda x: x[:, :, heads]
    k, v = p.k[:, heads], p.v[:, heads]
    kb, vb = p.k_blk[:, :, heads], p.v_blk[:, :, heads]
    say("[residual full] oracle")
    z = np.zeros((1, 3), np.uint8)
    ea, el, na, nl = OR.step(sub(q1), k, v, p.cu, kb, vb, hsel, page, z, np.zeros((1, 64, 3, 128)), np.zeros((1, 64, 3)),
                             p.scale)
    check_attn(sub(af1), ea, "bf16", "full refresh A_full")
    check_lse(sub(lf1), el, "bf16", "full refresh L_full")
    check_attn(sub(cache_a), na, "bf16", "full residual")
    ea, el, _, _ = OR.step(sub(q2), k, v, p.cu, kb, vb, hsel, page, np.ones((1, 3), np.uint8), na, nl, p.scale)
    check_attn(sub(af2), ea, "bf16", "full reuse A_full")
    check_lse(sub(lf2), el, "bf16", "full reuse L_full")


def test_out_of_range_pages_are_skipped(gpu_lib):
    """Selections holding negative and too-large page indices, and a count above the list's
    capacity, give the result of the valid pages alone (on the streaming, query-tiled and
    generic paged kernels)."""
    import torch
    fb = gpu_lib
    for name, hq, hkv, B, page in (("stream", 4, 4, 16, 16), ("tiled", 2, 2, 64, 16), ("generic", 4, 2, 16, 8)):
        say(f"[residual bad pages] {name}")
        p = synth.custom(37, 1, hq, hkv, 128, B, [700], std=1.0)
        n_pages = -(-700 // page)
        dev, s, rs = _shape(fb, p, page, 8)
        good = [np.array([3, 0, n_pages - 1]), np.array([5, 2])] + [np.array([1])] * (hkv - 2)
        pages = np.full((1, hkv, 8), -1, np.int32)
        count = np.zeros((1, hkv), np.int32)
        pages[0, 0, :6] = [3, -3, 0, n_pages + 7, n_pages - 1, 1 << 30]
        count[0, 0] = 6
        pages[0, 1, :] = [5, -1, 2, n_pages, -(1 << 30), n_pages * 3, -2, 9999]
        count[0, 1] = 12                      # above the capacity of 8: reads 8 entries
        for g in range(2, hkv):
            pages[0, g, 0] = 1
            count[0, g] = 1
        bf = _bufs(fb, p, rs, dev)
        _run(fb, rs, dev["q"], dev, torch.from_numpy(pages).cuda(), torch.from_numpy(count).cuda(), None, bf)
        torch.cuda.synchronize()
        sel = [[good[g] for g in range(hkv)]]
        ea, el, na, nl = OR.step(p.q, p.k, p.v, p.cu, p.k_blk, p.v_blk, sel, page, np.zeros((1, hq), np.uint8),
                                 np.zeros((1, B, hq, 128)), np.zeros((1, B, hq)), p.scale)
        check_attn(np_of(bf["af"]), ea, "bf16", f"{name} A_full")
        check_attn(np_of(bf["ca"]), na, "bf16", f"{name} residual")
