"""The debug cache check (fb_shape.flags = FB_FLAG_CHECK_CACHE) through the C ABI: a call
that would reuse a cache row holding NaN in cache_l (never written) returns
FB_ERR_CACHE_INVALID and writes nothing; a call that reuses only written rows, or reuses
nothing, runs, and gives the same bits as without the flag."""
import numpy as np
import pytest

import synth
from synth.device import tensor, to_device
from tests.gpu_util import say

pytestmark = pytest.mark.gpu

NAN = float("nan")


def _expect_invalid(fb, call):
    with pytest.raises(fb.FlashBlockError) as e:
        call()
    assert e.value.status == 4, e.value


def _step_setup(fb, flags):
    import torch
    p = synth.custom(71, 2, 8, 2, 128, 32, [1200, 500])
    dev = to_device(p)
    s = fb.make_shape(p.batch, p.h_q, p.h_kv, p.d, p.B, cu_seqlens_k=dev["cu"], max_seqlen_k=1200, flags=flags)
    b, B, h, d = p.q.shape
    o = dict(ca=torch.zeros((b, B, h, d), device="cuda"), cl=torch.full((b, B, h), NAN, device="cuda"),
             af=torch.full((b, B, h, d), 3.0, dtype=torch.bfloat16, device="cuda"),
             lf=torch.full((b, B, h), 3.0, device="cuda"),
             ws=torch.empty(fb.workspace_size(s), dtype=torch.uint8, device="cuda"))
    return p, dev, s, o


def test_step_rejects_reuse_of_unwritten_rows(gpu_lib):
    import torch
    fb = gpu_lib
    say("[cache check] fb_step / fb_step_threshold")
    p, dev, s, o = _step_setup(fb, fb.FB_FLAG_CHECK_CACHE)
    step = lambda m: fb.step(s, dev["q"], dev["k"], dev["v"], dev["k_blk"], dev["v_blk"], m, o["ca"], o["cl"], o["af"],
                             o["lf"], o["ws"])
    thr = lambda m: fb.step_threshold(s, dev["q"], dev["k"], dev["v"], dev["k_blk"], dev["v_blk"], m, 4, o["ca"],
                                      o["cl"], o["af"], o["lf"], o["ws"])
    ones = torch.ones((2, 8), dtype=torch.uint8, device="cuda")
    zero = torch.zeros((2, 8), dtype=torch.uint8, device="cuda")
    one_head = zero.clone()
    one_head[1, 5] = 1
    before = [o[k].clone() for k in ("ca", "cl", "af", "lf")]
    _expect_invalid(fb, lambda: step(ones))
    _expect_invalid(fb, lambda: step(one_head))
    _expect_invalid(fb, lambda: thr(torch.tensor([9, 0], dtype=torch.int32, device="cuda")))
    torch.cuda.synchronize()
    for x, y in zip(before, (o[k] for k in ("ca", "cl", "af", "lf"))):
        assert torch.equal(x, y) or (torch.isnan(x).all() and torch.isnan(y).all())
    # nothing reused: runs and writes every cache row
    step(zero)
    thr(torch.tensor([9, 9], dtype=torch.int32, device="cuda"))
    torch.cuda.synchronize()
    assert not torch.isnan(o["cl"]).any()
    af0 = o["af"].clone()
    # every row written: reuse runs, bit for bit as without the flag
    step(ones)
    thr(torch.tensor([0, 9], dtype=torch.int32, device="cuda"))
    torch.cuda.synchronize()
    assert torch.equal(o["af"], af0)
    _, dev2, s2, o2 = _step_setup(fb, 0)
    o2["ca"].copy_(o["ca"])
    o2["cl"].copy_(o["cl"])
    fb.step(s2, dev["q"], dev["k"], dev["v"], dev["k_blk"], dev["v_blk"], ones, o2["ca"], o2["cl"], o2["af"], o2["lf"],
            o2["ws"])
    torch.cuda.synchronize()
    assert torch.equal(o2["af"], af0) and torch.equal(o2["lf"], o["lf"])
    # one unwritten row of a reused head is enough to refuse; recomputing that head runs
    o["cl"][1, 17, 5] = NAN
    _expect_invalid(fb, lambda: step(ones))
    partly = ones.clone()
    partly[1, 5] = 0
    step(partly)
    torch.cuda.synchronize()
    assert not torch.isnan(o["cl"]).any()


def test_flag_bits_other_than_the_check_are_invalid(gpu_lib):
    fb = gpu_lib
    p, dev, s, o = _step_setup(fb, 2)
    with pytest.raises(fb.FlashBlockError) as e:
        fb.step(s, dev["q"], dev["k"], dev["v"], dev["k_blk"], dev["v_blk"], None, o["ca"], o["cl"], o["af"], o["lf"],
                o["ws"])
    assert e.value.status == 1


def test_losa_step_needs_written_rows(gpu_lib):
    """LoSA: the stable rows reuse their cached rows, so every row must have been written
    (by a dense step) before a sparse step."""
    import torch
    fb = gpu_lib
    say("[cache check] losa_step")
    p = synth.custom(73, 1, 4, 2, 128, 16, [900], std=1.0)
    g = synth.rng(74)
    q_cur = synth.round_bf16(p.q + 0.3 * g.standard_normal(p.q.shape, dtype=np.float32))
    dev = to_device(p)
    s = fb.make_shape(1, 4, 2, 128, 16, seqlen_k=900, flags=fb.FB_FLAG_CHECK_CACHE)
    ls = fb.make_losa_shape(s, page_size=16, topk=6, n_active=3)
    nb = fb.losa_meta_bytes(ls)
    kmin = torch.empty(nb // 2, dtype=torch.bfloat16, device="cuda")
    kmax = torch.empty_like(kmin)
    fb.losa_page_meta(ls, dev["k"], kmin, kmax)
    cap = fb.losa_union_capacity(ls)
    act = torch.full((1, 3), -7, dtype=torch.int32, device="cuda")
    topk = torch.full((1, 4, 3, 6), -7, dtype=torch.int32, device="cuda")
    uni = torch.full((1, 2, cap), -7, dtype=torch.int32, device="cuda")
    cnt = torch.full((1, 2), -7, dtype=torch.int32, device="cuda")
    ca = torch.zeros((1, 16, 4, 128), device="cuda")
    cl = torch.full((1, 16, 4), NAN, device="cuda")
    af = torch.zeros((1, 16, 4, 128), dtype=torch.bfloat16, device="cuda")
    lf = torch.zeros((1, 16, 4), device="cuda")
    lws = torch.empty(fb.losa_workspace_size(ls), dtype=torch.uint8, device="cuda")
    q_cur_d = tensor(q_cur, "bf16")
    run = lambda: fb.losa_step(ls, q_cur_d, dev["q"], dev["k"], dev["v"], dev["k_blk"], dev["v_blk"], kmin, kmax, ca,
                               cl, af, lf, act, topk, uni, cnt, lws)
    _expect_invalid(fb, run)
    torch.cuda.synchronize()
    assert (act == -7).all() and (cnt == -7).all() and torch.isnan(cl).all()
    ws = torch.empty(fb.workspace_size(s), dtype=torch.uint8, device="cuda")
    fb.step(s, dev["q"], dev["k"], dev["v"], dev["k_blk"], dev["v_blk"], None, ca, cl, af, lf, ws)
    run()
    torch.cuda.synchronize()
    assert (act >= 0).all() and not torch.isnan(cl).any()


def test_residual_step_checks_reused_heads(gpu_lib):
    import torch
    fb = gpu_lib
    say("[cache check] fb_residual_step")
    p = synth.custom(75, 1, 4, 2, 128, 16, [1000])
    dev = to_device(p)
    s = fb.make_shape(1, 4, 2, 128, 16, seqlen_k=1000, flags=fb.FB_FLAG_CHECK_CACHE)
    rs = fb.make_residual_shape(s, page_size=16, max_sel=10)
    sel = synth.page_selection(76, p.seqlens, 2, 16, 10)
    pages, count = synth.pack_selection(sel, 10, shuffle_seed=77)
    sp, sc = torch.from_numpy(pages).cuda(), torch.from_numpy(count).cuda()
    ca = torch.zeros((1, 16, 4, 128), device="cuda")
    cl = torch.full((1, 16, 4), NAN, device="cuda")
    af = torch.full((1, 16, 4, 128), 3.0, dtype=torch.bfloat16, device="cuda")
    lf = torch.zeros((1, 16, 4), device="cuda")
    ws = torch.empty(fb.residual_workspace_size(rs), dtype=torch.uint8, device="cuda")
    run = lambda m: fb.residual_step(rs, dev["q"], dev["k"], dev["v"], dev["k_blk"], dev["v_blk"], sp, sc, m, ca, cl,
                                     af, lf, ws)
    mask = torch.tensor([[0, 1, 0, 0]], dtype=torch.uint8, device="cuda")
    _expect_invalid(fb, lambda: run(mask))
    torch.cuda.synchronize()
    assert (af == 3.0).all()
    run(None)   # every head refreshes its residual
    run(mask)
    torch.cuda.synchronize()
    assert not torch.isnan(cl).any()
