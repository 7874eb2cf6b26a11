"""GPU parity of the FlashBlock step through the C ABI against the fp64 oracle."""
import numpy as np
import pytest

import synth
from synth.device import tensor, to_device
from oracle.attention import attend, block_attention, lse_merge, prefix_attention, full_attention
from oracle import flashblock as OF
from tests.gpu_util import check_attn, check_lse, guarded, np_of, say, to_device_guarded

pytestmark = pytest.mark.gpu


def _alloc(fb, p, dev):
    """Step outputs, each between guard bands (checked after the test)."""
    import torch
    b, B, h, d = p.q.shape
    out_dt = torch.bfloat16 if p.dtype == "bf16" else torch.float32
    return dict(
        cache_a=guarded((b, B, h, d), torch.float32, 0.0, "cache_a"),
        cache_l=guarded((b, B, h), torch.float32, 0.0, "cache_l"),
        a_full=guarded((b, B, h, d), out_dt, 0.0, "a_full"),
        l_full=guarded((b, B, h), torch.float32, 0.0, "l_full"),
    )


def _shape(fb, p, dev, varlen=False, num_splits=0):
    code = fb.FB_BF16 if p.dtype == "bf16" else fb.FB_F32
    if varlen:
        return fb.make_shape(p.batch, p.h_q, p.h_kv, p.d, p.B, dtype=code, cu_seqlens_k=dev["cu"],
                             max_seqlen_k=int(p.seqlens.max()), num_splits=num_splits)
    assert len(set(p.seqlens.tolist())) == 1
    return fb.make_shape(p.batch, p.h_q, p.h_kv, p.d, p.B, dtype=code, seqlen_k=int(p.seqlens[0]),
                         num_splits=num_splits)


def _ws(fb, shape):
    import torch
    n = fb.workspace_size(shape)
    return guarded((max(n, 16),), torch.uint8, 0xFF, "workspace")   # poisoned, between guard bands


# ------------------------------------------------------------------------------ merge

@pytest.mark.parametrize("rows,d", [(1000, 128), (77, 64), (5, 200)])
def test_lse_merge_f32(gpu_lib, rows, d):
    import torch
    fb = gpu_lib
    g = np.random.default_rng(rows)
    ao, ai = g.normal(size=(rows, d)).astype(np.float32), g.normal(size=(rows, d)).astype(np.float32)
    lo, li = (g.normal(size=rows) * 8).astype(np.float32), (g.normal(size=rows) * 8).astype(np.float32)
    lo[::7] = -np.inf
    li[::11] = -np.inf
    li[::13] = lo[::13]
    lo[3] = li[3] = -np.inf
    t = lambda x: torch.from_numpy(x).cuda()
    af = guarded((rows, d), torch.float32, name="a_full")
    lf = guarded((rows,), torch.float32, name="l_full")
    fb.lse_merge(t(ao), t(lo), t(ai), t(li), af, lf)
    torch.cuda.synchronize()
    ea, el = lse_merge(ao, lo, ai, li)
    err = np.abs(np_of(af) - ea)
    assert (err <= 1e-6 + 1e-6 * np.abs(ea)).all(), err.max()
    check = np.isneginf(el)
    assert (np.isneginf(np_of(lf)) == check).all()
    assert (np.abs(np_of(lf)[~check] - el[~check]) <= 1e-6 * (1 + np.abs(el[~check]))).all()
    afb = guarded((rows, d), torch.bfloat16, name="a_full bf16")
    fb.lse_merge(t(ao), t(lo), t(ai), t(li), afb)
    torch.cuda.synchronize()
    assert np.allclose(np_of(afb), ea, rtol=1e-2, atol=1e-2)


# ---------------------------------------------------------------------- prefix / block

PREFIX_CASES = [
    # name, batch, h_q, h_kv, d, B, seqlens, dtype
    ("mha_d128_B32", 1, 4, 4, 128, 32, [1000], "bf16"),
    ("gqa4_d128_B32_varlen", 2, 8, 2, 128, 32, [700, 129], "bf16"),
    ("gqa4_d64_B8", 2, 8, 2, 64, 8, [300, 1], "bf16"),
    ("mha_B64", 1, 2, 2, 128, 64, [2500], "bf16"),
    ("mha_B5_ragged", 3, 3, 1, 128, 5, [33, 0, 517], "bf16"),
    ("rows_tail_B40_g4", 1, 4, 1, 128, 40, [640], "bf16"),
    # query groups of >= 256 rows (query-tiled kernel): ragged key tiles and query tiles
    ("rows300_mha", 1, 2, 2, 128, 300, [1000], "bf16"),
    ("rows400_gqa2", 1, 4, 2, 128, 200, [777], "bf16"),
    ("rows260_varlen_empty", 2, 2, 1, 128, 130, [0, 2100], "bf16"),
    ("rows33_first_tiled", 1, 1, 1, 128, 33, [1500], "bf16"),
    ("rows128_deep_edge", 1, 2, 2, 128, 128, [900], "bf16"),
    ("rows129_wide_edge", 1, 1, 1, 128, 129, [900], "bf16"),
    ("B1_mqa_g32", 2, 32, 1, 128, 1, [2000, 5], "bf16"),
    ("d64_rows64_generic", 1, 4, 1, 64, 16, [800], "bf16"),
    ("one_full_stream_chunk", 1, 2, 2, 128, 32, [5120], "bf16"),
    ("f32_d64", 2, 2, 2, 64, 4, [60, 77], "f32"),
    ("f32_d128_gqa", 1, 4, 2, 128, 7, [300], "f32"),
]


@pytest.mark.parametrize("case", PREFIX_CASES, ids=[c[0] for c in PREFIX_CASES])
def test_prefix_and_block_attn(gpu_lib, case):
    import torch
    fb = gpu_lib
    name, b, hq, hkv, d, B, lens, dt = case
    say(f"[prefix/block] {name}")
    p = synth.custom(7, b, hq, hkv, d, B, lens, dtype=dt, std=1.0)
    dev = to_device_guarded(p)
    shape = _shape(fb, p, dev, varlen=True)
    ws = _ws(fb, shape)
    a = guarded((b, B, hq, d), torch.float32, float("nan"), "a_out")
    l = guarded((b, B, hq), torch.float32, float("nan"), "l_out")
    fb.prefix_attn(shape, dev["q"], dev["k"], dev["v"], a, l, ws)
    torch.cuda.synchronize()
    ea, el = prefix_attention(p.q, p.k, p.v, p.cu, hkv, p.scale)
    check_attn(np_of(a), ea, dt, f"{name} A_out")
    check_lse(np_of(l), el, dt, f"{name} L_out")
    fb.block_attn(shape, dev["q"], dev["k_blk"], dev["v_blk"], a, l, ws)
    torch.cuda.synchronize()
    ea, el = block_attention(p.q, p.k_blk, p.v_blk, p.scale)
    check_attn(np_of(a), ea, dt, f"{name} A_in")
    check_lse(np_of(l), el, dt, f"{name} L_in")


# Groups of more than 128 rows run on the phase-shifted 8-wave kernel: one key tile, a full
# single tile, two tiles, ragged tails on both the key and the query side, empty waves in
# the last query tile, many splits, peaked logits (the lazy max is raised mid-chunk), and
# two heads of very different scale in one launch.
WIDE_CASES = [
    # name, batch, h_q, h_kv, B, seqlens, num_splits, q scale
    ("one_partial_tile", 1, 1, 1, 256, [40], 0, 1.0),
    ("one_full_tile", 1, 2, 2, 200, [64], 0, 1.0),
    ("two_tiles", 1, 1, 1, 257, [128], 0, 1.0),
    ("rows512_tail_keys", 1, 1, 1, 512, [1333], 0, 1.0),
    ("rows_tail_33", 2, 2, 2, 289, [700, 96], 0, 1.0),
    ("many_splits", 1, 2, 1, 150, [2000], 7, 1.0),
    ("peaked", 1, 2, 2, 300, [1500], 0, 4.0),
    ("gqa4_rows_per_wave_cross_heads", 1, 8, 2, 70, [900], 3, 1.0),
]


@pytest.mark.parametrize("case", WIDE_CASES, ids=[c[0] for c in WIDE_CASES])
def test_wide_groups_prefix_and_block(gpu_lib, case):
    import torch
    fb = gpu_lib
    name, b, hq, hkv, B, lens, ns, qs = case
    say(f"[wide groups] {name}")
    p = synth.custom(19, b, hq, hkv, 128, B, lens, std=1.0)
    p.q *= qs   # a power of two: the values stay bf16
    dev = to_device_guarded(p)
    shape = _shape(fb, p, dev, varlen=True, num_splits=ns)
    ws = _ws(fb, shape)
    a = guarded((b, B, hq, 128), torch.float32, float("nan"), "a_out")
    l = guarded((b, B, hq), torch.float32, float("nan"), "l_out")
    fb.prefix_attn(shape, dev["q"], dev["k"], dev["v"], a, l, ws)
    torch.cuda.synchronize()
    ea, el = prefix_attention(p.q, p.k, p.v, p.cu, hkv, p.scale)
    check_attn(np_of(a), ea, "bf16", f"{name} A_out")
    check_lse(np_of(l), el, "bf16", f"{name} L_out")
    fb.block_attn(shape, dev["q"], dev["k_blk"], dev["v_blk"], a, l, ws)
    torch.cuda.synchronize()
    ea, el = block_attention(p.q, p.k_blk, p.v_blk, p.scale)
    check_attn(np_of(a), ea, "bf16", f"{name} A_in")
    check_lse(np_of(l), el, "bf16", f"{name} L_in")


def test_prefix_peaked_softmax(gpu_lib):
    """Q, K ~ N(0, 1) at d = 128: logits of std ~1 make the softmax peaked, so errors in the
    max/sum bookkeeping show up."""
    import torch
    fb = gpu_lib
    p = synth.custom(11, 1, 4, 2, 128, 32, [3000], std=1.0)
    p.q *= 4.0   # sharper (values stay bf16: scaling by a power of two is exact)
    dev = to_device_guarded(p)
    shape = _shape(fb, p, dev)
    ws = _ws(fb, shape)
    a = guarded((1, 32, 4, 128), torch.float32, name="a_out")
    l = guarded((1, 32, 4), torch.float32, name="l_out")
    fb.prefix_attn(shape, dev["q"], dev["k"], dev["v"], a, l, ws)
    torch.cuda.synchronize()
    ea, el = prefix_attention(p.q, p.k, p.v, p.cu, 2, p.scale)
    check_attn(np_of(a), ea, "bf16", "peaked A_out")
    check_lse(np_of(l), el, "bf16", "peaked L_out")


@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_split_counts_agree(gpu_lib, dt):
    """1, 4 and 32 prefix chunks: each matches the oracle; with fp32 inputs they also agree
    with one another to 1e-5 (with bf16 inputs P is rounded against each chunk's own
    running max, so they agree only to the bf16 bound, which the oracle check covers)."""
    import torch
    fb = gpu_lib
    p = synth.custom(3, 1, 4, 4, 128, 32, [4096], dtype=dt, std=1.0)
    dev = to_device_guarded(p)
    ea, el = prefix_attention(p.q, p.k, p.v, p.cu, 4, p.scale)
    outs = []
    for ns in (1, 4, 32):
        shape = _shape(fb, p, dev, num_splits=ns)
        ws = _ws(fb, shape)
        a = guarded((1, 32, 4, 128), torch.float32, name=f"a_out splits {ns}")
        l = guarded((1, 32, 4), torch.float32, name=f"l_out splits {ns}")
        fb.prefix_attn(shape, dev["q"], dev["k"], dev["v"], a, l, ws)
        torch.cuda.synchronize()
        outs.append((np_of(a), np_of(l)))
        check_attn(outs[-1][0], ea, dt, f"splits={ns} A_out")
        check_lse(outs[-1][1], el, dt, f"splits={ns} L_out")
    if dt == "f32":
        for a, l in outs[1:]:
            assert np.allclose(a, outs[0][0], rtol=1e-5, atol=1e-6)
            assert np.allclose(l, outs[0][1], rtol=1e-6, atol=1e-6)


# ------------------------------------------------------------------------------- steps

def test_tiny_f32_two_steps(gpu_lib):
    """Tiny fp32 workload: fresh step (== unsplit attention), then a reuse step with the
    queries perturbed by N(0, 0.01^2)."""
    import torch
    fb = gpu_lib
    p = synth.tiny()
    dev = to_device_guarded(p)
    shape = _shape(fb, p, dev)
    ws = _ws(fb, shape)
    o = _alloc(fb, p, dev)
    zero = torch.zeros((1, 2), dtype=torch.uint8, device="cuda")
    fb.step(shape, dev["q"], dev["k"], dev["v"], dev["k_blk"], dev["v_blk"], zero, o["cache_a"], o["cache_l"],
            o["a_full"], o["l_full"], ws)
    torch.cuda.synchronize()
    ea, el, eca, ecl = OF.step(p.q, p.k, p.v, p.cu, p.k_blk, p.v_blk, np.zeros((1, 2), np.uint8), None, None, p.scale)
    fa, fl = full_attention(p.q, p.k, p.v, p.cu, p.k_blk, p.v_blk, p.scale)
    check_attn(np_of(o["a_full"]), fa, "f32", "tiny fresh A_full vs unsplit")
    check_lse(np_of(o["l_full"]), fl, "f32", "tiny fresh L_full vs unsplit")
    check_attn(np_of(o["cache_a"]), eca, "f32", "tiny cache A")
    q1 = tensor(p.extra["q_step1"], "f32")
    one = torch.ones((1, 2), dtype=torch.uint8, device="cuda")
    cache_before = o["cache_a"].clone()
    fb.step(shape, q1, dev["k"], dev["v"], dev["k_blk"], dev["v_blk"], one, o["cache_a"], o["cache_l"],
            o["a_full"], o["l_full"], ws)
    torch.cuda.synchronize()
    ra, rl, rca, rcl = OF.step(p.extra["q_step1"], p.k, p.v, p.cu, p.k_blk, p.v_blk, np.ones((1, 2), np.uint8),
                               np_of(cache_before).astype(np.float64), np_of(o["cache_l"]).astype(np.float64), p.scale)
    assert torch.equal(cache_before, o["cache_a"])
    check_attn(np_of(o["a_full"]), ra, "f32", "tiny reuse A_full")
    check_lse(np_of(o["l_full"]), rl, "f32", "tiny reuse L_full")


@pytest.mark.parametrize("block", [32, 1056], ids=["block32", "block1056_combine_decides_first"])
def test_reuse_equals_recompute_bitwise(gpu_lib, block):
    """Unchanged queries, KV and cache: the reuse step and the recompute step give
    bit-identical A_full, L_full and cache.  At block 1056 (16896 rows) the combine reads
    each row's decision before its loads; the threshold rule is checked there too."""
    import torch
    fb = gpu_lib
    say(f"[reuse bitwise] block {block}")
    p = synth.custom(5, 2, 8, 2, 128, block, [2000, 777])
    dev = to_device_guarded(p)
    shape = _shape(fb, p, dev, varlen=True)
    ws = _ws(fb, shape)
    o = _alloc(fb, p, dev)
    zero = torch.zeros((2, 8), dtype=torch.uint8, device="cuda")
    ones = torch.ones((2, 8), dtype=torch.uint8, device="cuda")
    args = lambda m: (shape, dev["q"], dev["k"], dev["v"], dev["k_blk"], dev["v_blk"], m, o["cache_a"],
                      o["cache_l"], o["a_full"], o["l_full"], ws)
    fb.step(*args(zero))
    torch.cuda.synchronize()
    a0, l0, c0, cl0 = (o[x].clone() for x in ("a_full", "l_full", "cache_a", "cache_l"))
    fb.step(*args(ones))
    torch.cuda.synchronize()
    a1, l1 = o["a_full"].clone(), o["l_full"].clone()
    assert torch.equal(o["cache_a"], c0) and torch.equal(o["cache_l"], cl0)
    fb.step(*args(zero))
    torch.cuda.synchronize()
    for x, y in ((a0, a1), (l0, l1), (o["a_full"], a0), (o["cache_a"], c0), (o["cache_l"], cl0)):
        assert torch.equal(x, y)
    mixed = torch.tensor([[0, 1] * 4, [1, 0] * 4], dtype=torch.uint8, device="cuda")
    fb.step(*args(mixed))
    torch.cuda.synchronize()
    assert torch.equal(o["a_full"], a0)
    # counts 9 and 0 with tau 4: sequence 0 recomputes, sequence 1 reuses
    m = torch.tensor([9, 0], dtype=torch.int32, device="cuda")
    fb.step_threshold(shape, dev["q"], dev["k"], dev["v"], dev["k_blk"], dev["v_blk"], m, 4, o["cache_a"],
                      o["cache_l"], o["a_full"], o["l_full"], ws)
    torch.cuda.synchronize()
    for x, y in ((o["a_full"], a0), (o["l_full"], l0), (o["cache_a"], c0), (o["cache_l"], cl0)):
        assert torch.equal(x, y)


MIXED_GROUP = [
    # name, h_q, h_kv, B, prefix lengths: G * B rows per (sequence, KV head) group
    ("streaming_rows32", 8, 2, 8, [900, 333]),        # 32 rows: streaming kernel
    ("tiled_rows64", 8, 2, 16, [700, 1500]),          # 64 rows: query-tiled, 4 waves
    ("wide_rows1200", 4, 1, 300, [640, 1100]),        # 1200 rows: query-tiled, 8 waves
]


@pytest.mark.parametrize("case", MIXED_GROUP, ids=[c[0] for c in MIXED_GROUP])
def test_mixed_reuse_inside_gqa_group(gpu_lib, case):
    """Each KV-head group holds both reusing and recomputing query heads, and the second
    step changes the queries and the block K/V.  Against the oracle chain (fresh step, then
    the mixed step on the oracle's own cache); the reused heads' cache rows must stay bit
    for bit what the first step wrote, the recomputed heads' rows must take the new prefix
    result."""
    import torch
    fb = gpu_lib
    name, hq, hkv, B, lens = case
    say(f"[mixed group] {name}")
    p = synth.custom(81, 2, hq, hkv, 128, B, lens, std=1.0)
    dev = to_device_guarded(p)
    shape = _shape(fb, p, dev, varlen=True)
    ws = _ws(fb, shape)
    o = _alloc(fb, p, dev)
    z = np.zeros((2, hq), np.uint8)
    fb.step(shape, dev["q"], dev["k"], dev["v"], dev["k_blk"], dev["v_blk"], torch.from_numpy(z).cuda(),
            o["cache_a"], o["cache_l"], o["a_full"], o["l_full"], ws)
    torch.cuda.synchronize()
    ea, el, ca, cl = OF.step(p.q, p.k, p.v, p.cu, p.k_blk, p.v_blk, z, None, None, p.scale)
    check_attn(np_of(o["a_full"]), ea, "bf16", f"{name} fresh A_full")
    check_attn(np_of(o["cache_a"]), ca, "bf16", f"{name} fresh cache")
    ga0, gl0 = np_of(o["cache_a"]).copy(), np_of(o["cache_l"]).copy()
    # every group mixes: sequence 0 reuses heads 1, 2 of each group of G, sequence 1 the others
    G = hq // hkv
    mask = np.zeros((2, hq), np.uint8)
    for h in range(hq):
        j = h % G
        mask[0, h] = 1 if j in (1, 2) else 0
        mask[1, h] = 1 - mask[0, h]
    for b in range(2):
        for g in range(hkv):
            grp = mask[b, g * G:(g + 1) * G]
            assert grp.any() and not grp.all(), (b, g, grp)
    g_ = synth.rng(82)
    q2 = synth.round_bf16(p.q + 0.3 * g_.standard_normal(p.q.shape, dtype=np.float32))
    kb2 = synth.round_bf16(p.k_blk + 0.3 * g_.standard_normal(p.k_blk.shape, dtype=np.float32))
    vb2 = synth.round_bf16(p.v_blk + 0.3 * g_.standard_normal(p.v_blk.shape, dtype=np.float32))
    fb.step(shape, tensor(q2), dev["k"], dev["v"], tensor(kb2), tensor(vb2), torch.from_numpy(mask).cuda(),
            o["cache_a"], o["cache_l"], o["a_full"], o["l_full"], ws)
    torch.cuda.synchronize()
    ea2, el2, ca2, cl2 = OF.step(q2, p.k, p.v, p.cu, kb2, vb2, mask, ca, cl, p.scale)
    check_attn(np_of(o["a_full"]), ea2, "bf16", f"{name} mixed A_full")
    check_lse(np_of(o["l_full"]), el2, "bf16", f"{name} mixed L_full")
    ga, gl = np_of(o["cache_a"]), np_of(o["cache_l"])
    check_attn(ga, ca2, "bf16", f"{name} mixed cache A_out")
    check_lse(gl, cl2, "bf16", f"{name} mixed cache L_out")
    for b in range(2):
        for h in range(hq):
            if mask[b, h]:
                assert np.array_equal(ga[b, :, h], ga0[b, :, h]) and np.array_equal(gl[b, :, h], gl0[b, :, h]), \
                    f"{name}: reused head ({b}, {h}) cache changed"
            else:
                assert not np.array_equal(ga[b, :, h], ga0[b, :, h]), f"{name}: head ({b}, {h}) was not recomputed"


def test_threshold_block_of_steps(gpu_lib):
    """A block of denoising steps at the dLLM shape (shorter prefix): threshold rule on the
    drawn M, queries and block K/V changing every step, compared step by step."""
    import torch
    fb = gpu_lib
    p = synth.dllm(n_prefix=4096)
    dev = to_device_guarded(p)
    shape = _shape(fb, p, dev)
    ws = _ws(fb, shape)
    o = _alloc(fb, p, dev)
    mask = torch.empty((1, 32), dtype=torch.uint8, device="cuda")
    g = synth.rng(100)
    q, kb, vb = p.q, p.k_blk, p.v_blk
    ca = cl = None
    for s in range(4):
        m_t = torch.from_numpy(p.extra["m_updated"][s]).cuda()
        fb.mask_threshold(m_t, p.extra["tau"], 32, mask)
        em = OF.mask_threshold(p.extra["m_updated"][s], p.extra["tau"], 32)
        fb.step(shape, tensor(q), dev["k"], dev["v"], tensor(kb), tensor(vb), mask, o["cache_a"], o["cache_l"],
                o["a_full"], o["l_full"], ws)
        torch.cuda.synchronize()
        assert (np_of(mask) == em).all()
        ea, el, ca, cl = OF.step(q, p.k, p.v, p.cu, kb, vb, em, ca, cl, p.scale)
        say(f"  step {s}: reuse={int(em[0, 0])}")
        check_attn(np_of(o["a_full"]), ea, "bf16", f"step {s} A_full")
        check_lse(np_of(o["l_full"]), el, "bf16", f"step {s} L_full")
        # the oracle carries its own cache from step to step (an all-oracle chain)
        check_attn(np_of(o["cache_a"]), ca, "bf16", f"step {s} cache A_out")
        check_lse(np_of(o["cache_l"]), cl, "bf16", f"step {s} cache L_out")
        # next step: a few block tokens change
        q = synth.round_bf16(q + 0.05 * g.standard_normal(q.shape, dtype=np.float32) / np.sqrt(128))
        kb = synth.round_bf16(kb + 0.05 * g.standard_normal(kb.shape, dtype=np.float32) / np.sqrt(128))


def test_dllm_full_size_fresh_step_sampled(gpu_lib):
    """The dLLM workload at full size (prefix 32768) in the bench's launch configuration,
    checked on a seeded sample of heads against the oracle computed head by head."""
    import torch
    fb = gpu_lib
    p = synth.dllm()
    dev = to_device_guarded(p)
    shape = _shape(fb, p, dev)
    ws = _ws(fb, shape)
    o = _alloc(fb, p, dev)
    fb.step(shape, dev["q"], dev["k"], dev["v"], dev["k_blk"], dev["v_blk"], None, o["cache_a"], o["cache_l"],
            o["a_full"], o["l_full"], ws)
    torch.cuda.synchronize()
    af, lf, ca = np_of(o["a_full"]), np_of(o["l_full"]), np_of(o["cache_a"])
    for h in synth.rng(1234).choice(32, size=6, replace=False):
        kk = np.concatenate([p.k[:, h], p.k_blk[0, :, h]])
        vv = np.concatenate([p.v[:, h], p.v_blk[0, :, h]])
        ea, el = attend(p.q[0, :, h], kk, vv, p.scale)
        eo, _ = attend(p.q[0, :, h], p.k[:, h], p.v[:, h], p.scale)
        check_attn(af[0, :, h], ea, "bf16", f"head {h} A_full")
        check_lse(lf[0, :, h], el, "bf16", f"head {h} L_full")
        check_attn(ca[0, :, h], eo, "bf16", f"head {h} A_out")


# -------------------------------------------------------------------- masks and cosine

def test_masks_and_cosine(gpu_lib):
    import torch
    fb = gpu_lib
    m = np.array([3, 4, 5, 0, 8, 1], dtype=np.int32)
    mask = guarded((6, 5), torch.uint8, name="threshold mask")
    fb.mask_threshold(torch.from_numpy(m).cuda(), 4, 5, mask)
    sim = np.array([[0.95, 0.9500001, 0.2, 1.0, -0.3, 0.96]], dtype=np.float32)
    ms = guarded((1, 6), torch.uint8, name="similarity mask")
    fb.mask_similarity(torch.from_numpy(sim).cuda(), 0.95, ms)
    g = np.random.default_rng(0)
    a0 = g.normal(size=(2, 9, 3, 128)).astype(np.float32)
    a1 = (a0 + 0.3 * g.normal(size=a0.shape)).astype(np.float32)
    a1[1, :, 2] = -a0[1, :, 2]
    a1[0, :, 1] = 0.0
    s = guarded((2, 3), torch.float32, name="cosine")
    fb.head_cosine(torch.from_numpy(a0).cuda(), torch.from_numpy(a1).cuda(), s)
    torch.cuda.synchronize()
    assert (np_of(mask) == OF.mask_threshold(m, 4, 5)).all()
    assert (np_of(ms) == OF.mask_similarity(sim, 0.95)).all()
    es = OF.head_cosine(a0, a1)
    assert np.allclose(np_of(s), es, rtol=1e-6, atol=1e-6)
    assert np_of(s)[1, 2] == pytest.approx(-1.0, abs=1e-6) and np_of(s)[0, 1] == 0.0


# ---------------------------------------------------------------- ragged and video shapes

def test_ragged_gqa_sampled(gpu_lib):
    """Batched ragged dLLM workload (GQA 32/8, prefixes in [8192, 65536], packed varlen,
    per-sequence threshold mask) at full size; sampled sequences against the oracle."""
    import torch
    fb = gpu_lib
    p = synth.ragged()
    dev = to_device_guarded(p)
    shape = _shape(fb, p, dev, varlen=True)
    ws = _ws(fb, shape)
    o = _alloc(fb, p, dev)
    fb.step(shape, dev["q"], dev["k"], dev["v"], dev["k_blk"], dev["v_blk"], None, o["cache_a"], o["cache_l"],
            o["a_full"], o["l_full"], ws)
    mask = torch.empty((p.batch, 32), dtype=torch.uint8, device="cuda")
    fb.mask_threshold(torch.from_numpy(p.extra["m_updated"]).cuda(), 4, 32, mask)
    q2 = synth.round_bf16(p.q * 0.5)
    fb.step(shape, tensor(q2), dev["k"], dev["v"], dev["k_blk"], dev["v_blk"], mask, o["cache_a"], o["cache_l"],
            o["a_full"], o["l_full"], ws)
    torch.cuda.synchronize()
    em = OF.mask_threshold(p.extra["m_updated"], 4, 32)
    af = np_of(o["a_full"])
    for b in synth.rng(77).choice(p.batch, size=3, replace=False):
        lo, hi = p.cu[b], p.cu[b + 1]
        for h in (0, 13, 31):
            g = h // 4
            qn = p.q if em[b, h] else q2
            eo, lo_ = attend(qn[b, :, h], p.k[lo:hi, g], p.v[lo:hi, g], p.scale)
            ei, li = attend(q2[b, :, h], p.k_blk[b, :, g], p.v_blk[b, :, g], p.scale)
            ea, _ = lse_merge(eo, lo_, ei, li)
            check_attn(af[b, :, h], ea, "bf16", f"seq {b} head {h} reuse={em[b, h]}")


def test_video_block_sampled(gpu_lib):
    """Video-block workload at full size (4680 block queries, prefix 32760, 12 heads) with
    the per-head similarity mask: every head reuses after a fresh step; a seeded sample of
    256 query rows is checked against the oracle for every head."""
    import torch
    fb = gpu_lib
    p = synth.video()
    dev = to_device_guarded(p)
    shape = _shape(fb, p, dev)
    ws = _ws(fb, shape)
    o = _alloc(fb, p, dev)
    fb.step(shape, dev["q"], dev["k"], dev["v"], dev["k_blk"], dev["v_blk"], None, o["cache_a"], o["cache_l"],
            o["a_full"], o["l_full"], ws)
    mask = torch.empty((1, 12), dtype=torch.uint8, device="cuda")
    fb.mask_similarity(torch.from_numpy(p.extra["sim"]).cuda(), p.extra["gamma"], mask)
    q2 = synth.round_bf16(p.q * 0.75)
    fb.step(shape, tensor(q2), dev["k"], dev["v"], dev["k_blk"], dev["v_blk"], mask, o["cache_a"], o["cache_l"],
            o["a_full"], o["l_full"], ws)
    torch.cuda.synchronize()
    em = OF.mask_similarity(p.extra["sim"], p.extra["gamma"])
    assert em.sum() == 7
    rows = np.sort(synth.rng(31).choice(p.B, size=256, replace=False))
    af = np_of(o["a_full"])
    for h in range(12):
        qn = p.q if em[0, h] else q2
        eo, lo_ = attend(qn[0, rows, h], p.k[:, h], p.v[:, h], p.scale)
        ei, li = attend(q2[0, rows, h], p.k_blk[0, :, h], p.v_blk[0, :, h], p.scale)
        ea, _ = lse_merge(eo, lo_, ei, li)
        check_attn(af[0, rows, h], ea, "bf16", f"video head {h} reuse={em[0, h]}")


def test_step_threshold_equals_mask_then_step(gpu_lib):
    """fb_step_threshold (rule evaluated inside the kernels) is bitwise identical to
    fb_mask_threshold followed by fb_step."""
    import torch
    fb = gpu_lib
    p = synth.custom(8, 3, 8, 2, 128, 32, [900, 64, 2000])
    dev = to_device_guarded(p)
    shape = _shape(fb, p, dev, varlen=True)
    ws = _ws(fb, shape)
    o1, o2 = _alloc(fb, p, dev), _alloc(fb, p, dev)
    fresh = torch.full((3,), 1 << 30, dtype=torch.int32, device="cuda")
    for o in (o1, o2):
        fb.step_threshold(shape, dev["q"], dev["k"], dev["v"], dev["k_blk"], dev["v_blk"], fresh, 4, o["cache_a"],
                          o["cache_l"], o["a_full"], o["l_full"], ws)
    m = torch.tensor([2, 7, 4], dtype=torch.int32, device="cuda")
    q2 = tensor(synth.round_bf16(p.q * 0.5))
    mask = torch.empty((3, 8), dtype=torch.uint8, device="cuda")
    fb.mask_threshold(m, 4, 8, mask)
    fb.step(shape, q2, dev["k"], dev["v"], dev["k_blk"], dev["v_blk"], mask, o1["cache_a"], o1["cache_l"],
            o1["a_full"], o1["l_full"], ws)
    fb.step_threshold(shape, q2, dev["k"], dev["v"], dev["k_blk"], dev["v_blk"], m, 4, o2["cache_a"], o2["cache_l"],
                      o2["a_full"], o2["l_full"], ws)
    torch.cuda.synchronize()
    assert np_of(mask)[:, 0].tolist() == [1, 0, 0]
    for k_ in ("a_full", "l_full", "cache_a", "cache_l"):
        assert torch.equal(o1[k_], o2[k_]), k_


def test_step_at_the_longest_swept_prefix(gpu_lib):
    """The dLLM step at the longest prefix the bench sweeps (819200 tokens, 32 heads, 13.4 GB
    of K/V in HBM): fresh, then reuse, on two sampled heads against the oracle."""
    import torch
    from synth.device import device_normal
    from oracle import flashblock as OF
    fb = gpu_lib
    n, H, d, B = 819200, 32, 128, 32
    std = 1.0 / np.sqrt(128.0)
    say("[longest prefix] draw")
    q = device_normal(71, (1, B, H, d), std)
    k = device_normal(72, (n, H, d), std)
    v = device_normal(73, (n, H, d), std)
    kb = device_normal(74, (1, B, H, d), std)
    vb = device_normal(75, (1, B, H, d), std)
    s = fb.make_shape(1, H, H, d, B, seqlen_k=n)
    ws = guarded((fb.workspace_size(s),), torch.uint8, name="workspace")
    ca = guarded((1, B, H, d), torch.float32, 0.0, "cache_a")
    cl = guarded((1, B, H), torch.float32, 0.0, "cache_l")
    af = guarded((1, B, H, d), torch.bfloat16, 0.0, "a_full")
    lf = guarded((1, B, H), torch.float32, 0.0, "l_full")
    say("[longest prefix] fresh step")
    fb.step(s, q, k, v, kb, vb, None, ca, cl, af, lf, ws)
    q2 = q + device_normal(76, (1, B, H, d), 0.01)
    af2 = guarded((1, B, H, d), torch.bfloat16, 0.0, "a_full reuse")
    lf2 = guarded((1, B, H), torch.float32, 0.0, "l_full reuse")
    fb.step(s, q2, k, v, kb, vb, torch.ones((1, H), dtype=torch.uint8, device="cuda"), ca, cl, af2, lf2, ws)
    torch.cuda.synchronize()
    heads = [5, 30]
    host = lambda t: t[..., heads, :].float().cpu().numpy().astype(np.float64)
    qh, kh, vh, kbh, vbh, q2h = host(q), host(k), host(v), host(kb), host(vb), host(q2)
    del k, v
    torch.cuda.empty_cache()
    say("[longest prefix] oracle")
    cu = np.array([0, n], np.int32)
    z = np.zeros((1, 2), np.uint8)
    ea, el, na, nl = OF.step(qh, kh, vh, cu, kbh, vbh, z, None, None, 1.0 / np.sqrt(d))
    check_attn(np_of(af)[:, :, heads], ea, "bf16", "longest fresh A_full")
    check_lse(np_of(lf)[:, :, heads], el, "bf16", "longest fresh L_full")
    check_attn(np_of(ca)[:, :, heads], na, "bf16", "longest cache")
    ea2, el2, _, _ = OF.step(q2h, kh, vh, cu, kbh, vbh, np.ones((1, 2), np.uint8), na, nl, 1.0 / np.sqrt(d))
    check_attn(np_of(af2)[:, :, heads], ea2, "bf16", "longest reuse A_full")
