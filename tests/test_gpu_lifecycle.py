"""GPU parity of the block lifecycle through the C ABI against the fp64 oracle
(oracle/lifecycle.py): block append and page metadata bit for bit, the block driver's
reuse masks exactly and its outputs within the attention tolerance."""
import numpy as np
import pytest

import synth
from synth.device import tensor, to_device
from oracle import lifecycle as LC
from oracle.losa import page_minmax
from tests.gpu_util import check_attn, check_lse, np_of, say

pytestmark = pytest.mark.gpu


def _shape(fb, p, dev, varlen):
    code = fb.FB_BF16 if p.dtype == "bf16" else fb.FB_F32
    if varlen:
        return fb.make_shape(p.batch, p.h_q, p.h_kv, p.d, p.B, dtype=code, cu_seqlens_k=dev["cu"],
                             max_seqlen_k=int(p.seqlens.max()))
    return fb.make_shape(p.batch, p.h_q, p.h_kv, p.d, p.B, dtype=code, seqlen_k=int(p.seqlens[0]))


APPEND = [
    # name, batch, h_kv, d, B, lens, dtype, varlen, in_place
    ("uniform2", 2, 4, 128, 32, [300, 300], "bf16", False, False),
    ("varlen3", 3, 2, 128, 16, [517, 0, 93], "bf16", True, False),
    ("inplace_uniform", 1, 4, 128, 32, [1000], "bf16", False, True),
    ("inplace_varlen", 1, 2, 64, 8, [77], "bf16", True, True),
    ("f32_narrow_rows", 2, 1, 3, 5, [11, 11], "f32", False, False),
    ("empty_prefix", 2, 2, 64, 4, [0, 0], "bf16", False, False),
]


@pytest.mark.parametrize("case", APPEND, ids=[c[0] for c in APPEND])
def test_append_block(gpu_lib, case):
    import torch
    fb = gpu_lib
    name, b, hkv, d, B, lens, dt, varlen, in_place = case
    say(f"[append] {name}")
    p = synth.custom(51, b, hkv, hkv, d, B, lens, dtype=dt)
    dev = to_device(p)
    s = _shape(fb, p, dev, varlen)
    ek, ev, ecu = LC.append_block(p.k, p.v, p.cu, p.k_blk, p.v_blk)
    tdt = dev["k_blk"].dtype
    if in_place:
        kbuf = torch.zeros((ek.shape[0],) + ek.shape[1:], dtype=tdt, device="cuda")
        vbuf = torch.zeros_like(kbuf)
        kbuf[:p.k.shape[0]] = dev["k"]
        vbuf[:p.v.shape[0]] = dev["v"]
        k_in, v_in, k_out, v_out = kbuf, vbuf, kbuf, vbuf
    else:
        k_in = dev["k"] if p.k.shape[0] else None
        v_in = dev["v"] if p.v.shape[0] else None
        k_out = torch.full(ek.shape, float("nan"), dtype=tdt, device="cuda")
        v_out = torch.full(ev.shape, float("nan"), dtype=tdt, device="cuda")
    cu_out = torch.full((b + 1,), -1, dtype=torch.int32, device="cuda")
    fb.append_block(s, k_in, v_in, dev["k_blk"], dev["v_blk"], k_out, v_out, cu_out)
    torch.cuda.synchronize()
    assert np_of(cu_out).tolist() == ecu.tolist()
    assert np.array_equal(np_of(k_out), ek) and np.array_equal(np_of(v_out), ev)


def test_page_meta_after_append(gpu_lib):
    """Metadata of the old prefix, append, rebuild the pages of the new tokens only: equal
    bit for bit to a full rebuild and to the oracle."""
    import torch
    fb = gpu_lib
    page = 16
    p = synth.custom(52, 2, 4, 2, 128, 24, [1000, 333], std=1.0)
    dev = to_device(p)
    s_old = _shape(fb, p, dev, True)
    ek, ev, ecu = LC.append_block(p.k, p.v, p.cu, p.k_blk, p.v_blk)
    max_pages = -(-int(np.diff(ecu).max()) // page)
    ls_old = fb.make_losa_shape(s_old, page_size=page, topk=4, n_active=2, max_pages=max_pages)
    nel = fb.losa_meta_bytes(ls_old) // 2
    kmin = torch.zeros(nel, dtype=torch.bfloat16, device="cuda")
    kmax = torch.zeros_like(kmin)
    fb.losa_page_meta(ls_old, dev["k"], kmin, kmax)
    k_new = torch.empty(ek.shape, dtype=torch.bfloat16, device="cuda")
    v_new = torch.empty_like(k_new)
    cu_new = torch.empty(3, dtype=torch.int32, device="cuda")
    fb.append_block(s_old, dev["k"], dev["v"], dev["k_blk"], dev["v_blk"], k_new, v_new, cu_new)
    s_new = fb.make_shape(2, 4, 2, 128, 24, cu_seqlens_k=cu_new, max_seqlen_k=int(np.diff(ecu).max()))
    ls_new = fb.make_losa_shape(s_new, page_size=page, topk=4, n_active=2, max_pages=max_pages)
    fb.losa_page_meta_append(ls_new, 24, k_new, kmin, kmax)
    full_min = torch.zeros_like(kmin)
    full_max = torch.zeros_like(kmin)
    fb.losa_page_meta(ls_new, k_new, full_min, full_max)
    torch.cuda.synchronize()
    mins, maxs = page_minmax(ek, ecu, page)
    for got, full, want in ((kmin, full_min, mins), (kmax, full_max, maxs)):
        x = np_of(got).reshape(2, 2, 16, max_pages, 8).transpose(0, 3, 1, 2, 4).reshape(2, max_pages, 2, 128)
        y = np_of(full).reshape(2, 2, 16, max_pages, 8).transpose(0, 3, 1, 2, 4).reshape(2, max_pages, 2, 128)
        for bi in range(2):
            P = want[bi].shape[0]
            assert np.array_equal(x[bi, :P], want[bi]) and np.array_equal(y[bi, :P], want[bi])


def _step_inputs(p, S, seed, sigma):
    g = synth.rng(seed)
    sig = np.asarray(sigma, dtype=np.float32).reshape(1, 1, -1, 1)
    q = [p.q] + [synth.round_bf16(p.q + g.standard_normal(p.q.shape, dtype=np.float32) * sig) for _ in range(1, S)]
    kb = [p.k_blk] + [synth.round_bf16(p.k_blk + 0.1 * g.standard_normal(p.k_blk.shape, dtype=np.float32))
                      for _ in range(1, S)]
    vb = [p.v_blk] + [synth.round_bf16(p.v_blk + 0.1 * g.standard_normal(p.v_blk.shape, dtype=np.float32))
                      for _ in range(1, S)]
    return np.stack(q), np.stack(kb), np.stack(vb)


def _run_block(fb, s, plan, dev, q, kb, vb, m, k, v):
    import torch
    S = plan.n_steps
    b, B, hq, d = q.shape[1:]
    out = dict(ca=torch.zeros((b, B, hq, d), device="cuda"), cl=torch.zeros((b, B, hq), device="cuda"),
               af=torch.zeros((S, b, B, hq, d), dtype=torch.bfloat16, device="cuda"),
               lf=torch.zeros((S, b, B, hq), device="cuda"),
               masks=torch.full((S, b, hq), 7, dtype=torch.uint8, device="cuda"),
               sims=torch.zeros((S, b, hq), device="cuda"))
    ws = torch.empty(fb.block_workspace_size(s), dtype=torch.uint8, device="cuda")
    md = None if m is None else torch.from_numpy(np.ascontiguousarray(m, dtype=np.int32)).cuda()
    fb.block_run(s, plan, tensor(q), k, v, tensor(kb), tensor(vb), md, out["ca"], out["cl"], out["af"], out["lf"],
                 out["masks"], out["sims"], ws)
    torch.cuda.synchronize()
    return {key: np_of(val) for key, val in out.items()}


def _check_run(got, exp, what):
    assert np.array_equal(got["masks"], exp["masks"]), f"{what}: masks {got['masks']} vs {exp['masks']}"
    for s in range(exp["a_full"].shape[0]):
        check_attn(got["af"][s], exp["a_full"][s], "bf16", f"{what} step {s}")
        check_lse(got["lf"][s], exp["l_full"][s], "bf16", f"{what} L step {s}")
    fin = ~np.isnan(exp["sims"])
    assert np.isnan(got["sims"][~fin]).all()
    # The cosine of two vectors moves by at most the angles their errors turn them through,
    # arcsin(|dx| / |x|) + arcsin(|dy| / |y|).  The error of a cached A_out (mostly the bf16
    # rounding of the probabilities in the PV product, whose pattern depends on the split
    # layout) is measured per (sequence, head) on the final cache and taken as the scale of
    # every step's cache, with a factor 2 for the steps not observed.
    check_attn(got["ca"], exp["cache_a"], "bf16", f"{what} final cache")
    ca, ea = got["ca"].astype(np.float64), exp["cache_a"]
    rel = np.sqrt(((ca - ea) ** 2).sum(axis=(1, 3)) / (ea ** 2).sum(axis=(1, 3)))   # [b, h_q]
    tol = 2 * 2 * np.arcsin(np.minimum(rel.max(), 1.0)) + 1e-6
    err = np.max(np.abs(got["sims"][fin] - exp["sims"][fin]))
    say(f"   {what}: similarity error {err:.2e}, bound {tol:.2e} (A_out relative error {rel.max():.2e})")
    assert err <= tol


def test_block_run_threshold(gpu_lib):
    fb = gpu_lib
    p = synth.custom(53, 2, 8, 2, 128, 32, [2000, 700], std=1.0)
    dev = to_device(p)
    s = _shape(fb, p, dev, True)
    S = 6
    q, kb, vb = _step_inputs(p, S, 54, [0.2] * 8)
    m = np.array([[99, 99], [9, 0], [0, 9], [3, 4], [4, 3], [0, 0]], np.int32)
    plan = fb.BlockPlan(S, fb.FB_RULE_THRESHOLD, 4, 0.0)
    say("[block] threshold")
    got = _run_block(fb, s, plan, dev, q, kb, vb, m, dev["k"], dev["v"])
    exp = LC.block_run(q, p.k, p.v, p.cu, kb, vb, p.scale, "threshold", m_steps=m, tau=4)
    _check_run(got, exp, "threshold")


def test_block_run_similarity(gpu_lib):
    """Heads 0, 2, 4, 6 drift by 1e-3 per step (similarity near 1), the others by 1.0 (far
    below gamma): the decisions are not near the threshold, so both sides take them alike."""
    fb = gpu_lib
    p = synth.custom(55, 1, 8, 4, 128, 48, [1500], std=1.0)
    dev = to_device(p)
    s = _shape(fb, p, dev, False)
    S = 5
    q, kb, vb = _step_inputs(p, S, 56, [1e-3, 1.0] * 4)
    plan = fb.BlockPlan(S, fb.FB_RULE_SIMILARITY, 0, 0.95)
    say("[block] similarity")
    got = _run_block(fb, s, plan, dev, q, kb, vb, None, dev["k"], dev["v"])
    exp = LC.block_run(q, p.k, p.v, p.cu, kb, vb, p.scale, "similarity", gamma=0.95)
    fin = ~np.isnan(exp["sims"])
    assert (np.abs(exp["sims"][fin] - 0.95) > 1e-3).all()
    assert exp["masks"][2:, 0, ::2].all() and not exp["masks"][2:, 0, 1::2].any()
    _check_run(got, exp, "similarity")


def test_block_run_similarity_large_block(gpu_lib):
    """Block 2100 with 8 heads (16800 rows, past the size where the combine reads each
    row's decision before its loads): the similarity after step 1 is the cosine between
    the block-external outputs of steps 0 and 1 (computed here by two prefix passes), so
    a fresh row still reads its cached row; the cache ends as step 1's prefix output."""
    import torch
    from oracle.flashblock import head_cosine
    fb = gpu_lib
    p = synth.custom(61, 1, 8, 2, 128, 2100, [1500], std=1.0)
    dev = to_device(p)
    s = _shape(fb, p, dev, False)
    q, kb, vb = _step_inputs(p, 2, 62, [1e-3, 1.0] * 4)
    plan = fb.BlockPlan(2, fb.FB_RULE_SIMILARITY, 0, 0.95)
    say("[block] similarity, block 2100")
    got = _run_block(fb, s, plan, dev, q, kb, vb, None, dev["k"], dev["v"])
    ws = torch.empty(max(fb.workspace_size(s), 16), dtype=torch.uint8, device="cuda")
    outs = []
    for t in range(2):
        a = torch.empty(p.q.shape, dtype=torch.float32, device="cuda")
        l = torch.empty(p.q.shape[:3], dtype=torch.float32, device="cuda")
        fb.prefix_attn(s, tensor(q[t]), dev["k"], dev["v"], a, l, ws)
        torch.cuda.synchronize()
        outs.append(np_of(a))
    assert not got["masks"].any()          # no mask before step 2: every head recomputes
    assert np.isnan(got["sims"][0]).all()
    exp = head_cosine(outs[0], outs[1])
    assert np.max(np.abs(got["sims"][1] - exp)) <= 1e-5, (got["sims"][1], exp)
    assert np.max(np.abs(got["ca"] - outs[1]) / (1.0 + np.abs(outs[1]))) <= 1e-5


def test_block_run_large_block_matches_single_steps(gpu_lib):
    """Block 2100 with 8 heads, three steps under the per-head rule: from step 2 half of the
    heads reuse, and the combine (past the size where each row reads its decision before
    its loads) also writes the cosine sums.  Every step's A_full, L_full and the final
    cache equal, bit for bit, fb_step calls fed the masks the block run recorded."""
    import torch
    fb = gpu_lib
    p = synth.custom(63, 1, 8, 2, 128, 2100, [1500], std=1.0)
    dev = to_device(p)
    s = _shape(fb, p, dev, False)
    S = 3
    q, kb, vb = _step_inputs(p, S, 64, [1e-3, 1.0] * 4)
    plan = fb.BlockPlan(S, fb.FB_RULE_SIMILARITY, 0, 0.95)
    say("[block] similarity, block 2100, three steps")
    got = _run_block(fb, s, plan, dev, q, kb, vb, None, dev["k"], dev["v"])
    assert got["masks"][2, 0, ::2].all() and not got["masks"][2, 0, 1::2].any(), got["masks"][2]
    ca = torch.zeros(p.q.shape, device="cuda")
    cl = torch.zeros(p.q.shape[:3], device="cuda")
    af = torch.zeros(p.q.shape, dtype=torch.bfloat16, device="cuda")
    lf = torch.zeros(p.q.shape[:3], device="cuda")
    ws = torch.empty(max(fb.workspace_size(s), 16), dtype=torch.uint8, device="cuda")
    for t in range(S):
        m = None if t < 2 else torch.from_numpy(np.ascontiguousarray(got["masks"][t])).cuda()
        fb.step(s, tensor(q[t]), dev["k"], dev["v"], tensor(kb[t]), tensor(vb[t]), m, ca, cl, af, lf, ws)
        torch.cuda.synchronize()
        assert np.array_equal(np_of(af).view(np.uint32), got["af"][t].view(np.uint32)), f"A_full step {t}"
        assert np.array_equal(np_of(lf), got["lf"][t]), f"L_full step {t}"
    assert np.array_equal(np_of(ca), got["ca"]) and np.array_equal(np_of(cl), got["cl"])


def test_three_blocks(gpu_lib):
    """A multi-block run: the steps of a block under the threshold rule, then the block's
    last K/V appended to the prefix, three times; each block against the oracle chain."""
    import torch
    fb = gpu_lib
    p = synth.custom(57, 2, 4, 2, 128, 16, [900, 400], std=1.0)
    dev = to_device(p)
    k_np, v_np, cu_np = p.k, p.v, p.cu
    k_d, v_d, cu_d = dev["k"], dev["v"], dev["cu"]
    g = synth.rng(58)
    for blk in range(3):
        say(f"[three blocks] block {blk}")
        S = 4
        p.q = synth.round_bf16(g.standard_normal(p.q.shape, dtype=np.float32))
        p.k_blk = synth.round_bf16(g.standard_normal(p.k_blk.shape, dtype=np.float32))
        p.v_blk = synth.round_bf16(g.standard_normal(p.v_blk.shape, dtype=np.float32))
        q, kb, vb = _step_inputs(p, S, 59 + blk, [0.3] * 4)
        m = g.integers(0, 9, size=(S, 2)).astype(np.int32)
        s = fb.make_shape(2, 4, 2, 128, 16, cu_seqlens_k=cu_d, max_seqlen_k=int(np.diff(cu_np).max()))
        plan = fb.BlockPlan(S, fb.FB_RULE_THRESHOLD, 4, 0.0)
        got = _run_block(fb, s, plan, dev, q, kb, vb, m, k_d, v_d)
        exp = LC.block_run(q, k_np, v_np, cu_np, kb, vb, p.scale, "threshold", m_steps=m, tau=4)
        _check_run(got, exp, f"block {blk}")
        k2, v2, cu2 = LC.append_block(k_np, v_np, cu_np, kb[-1], vb[-1])
        k_new = torch.empty(k2.shape, dtype=torch.bfloat16, device="cuda")
        v_new = torch.empty_like(k_new)
        cu_new = torch.empty(3, dtype=torch.int32, device="cuda")
        fb.append_block(s, k_d, v_d, tensor(kb[-1]), tensor(vb[-1]), k_new, v_new, cu_new)
        torch.cuda.synchronize()
        assert np.array_equal(np_of(k_new), k2) and np_of(cu_new).tolist() == cu2.tolist()
        k_np, v_np, cu_np, k_d, v_d, cu_d = k2, v2, cu2, k_new, v_new, cu_new
