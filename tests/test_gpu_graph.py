"""Steps captured into a HIP graph (stream capture) give the eager results bit for bit on
every replay, with eager work and synchronisations between the replays."""
import numpy as np
import pytest

import synth
from synth.device import to_device

pytestmark = pytest.mark.gpu


def _replays_match(fn, reset, outs, n=3):
    """fn: the step (the only work captured); reset: eager work that restores its inputs
    and poisons its outputs before every call and replay."""
    import torch
    reset()
    fn()
    torch.cuda.synchronize()
    ref = [o.clone() for o in outs]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    for i in range(n):
        reset()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for o, r in zip(outs, ref):
            assert torch.equal(o, r), f"replay {i} differs"
    del g


def test_step_graph_replays(gpu_lib):
    import torch
    fb = gpu_lib
    p = synth.custom(41, 2, 8, 2, 128, 32, [3000, 1200], std=1.0)
    dev = to_device(p)
    s = fb.make_shape(2, 8, 2, 128, 32, cu_seqlens_k=dev["cu"], max_seqlen_k=3000)
    ws = torch.empty(fb.workspace_size(s), dtype=torch.uint8, device="cuda")
    ca = torch.zeros((2, 32, 8, 128), device="cuda")
    cl = torch.zeros((2, 32, 8), device="cuda")
    af = torch.zeros((2, 32, 8, 128), dtype=torch.bfloat16, device="cuda")
    lf = torch.zeros((2, 32, 8), device="cuda")
    mask = torch.from_numpy(np.array([[0, 1] * 4, [1, 0] * 4], np.uint8)).cuda()
    fb.step(s, dev["q"], dev["k"], dev["v"], dev["k_blk"], dev["v_blk"], None, ca, cl, af, lf, ws)
    cache = (ca.clone(), cl.clone())

    def reset():
        ca.copy_(cache[0])
        cl.copy_(cache[1])
        af.fill_(float("nan"))
        lf.fill_(float("nan"))

    def run():
        fb.step(s, dev["q"], dev["k"], dev["v"], dev["k_blk"], dev["v_blk"], mask, ca, cl, af, lf, ws)
    _replays_match(run, reset, [af, lf, ca, cl])


def test_residual_step_graph_replays(gpu_lib):
    import torch
    fb = gpu_lib
    p = synth.custom(42, 1, 4, 4, 128, 64, [5000], std=1.0)
    dev = to_device(p)
    s = fb.make_shape(1, 4, 4, 128, 64, seqlen_k=5000)
    rs = fb.make_residual_shape(s, page_size=16, max_sel=64)
    sel = synth.page_selection(43, p.seqlens, 4, 16, 60, ("tail", "random"))
    pages, count = synth.pack_selection(sel, 64)
    sp, sc = torch.from_numpy(pages).cuda(), torch.from_numpy(count).cuda()
    ws = torch.empty(fb.residual_workspace_size(rs), dtype=torch.uint8, device="cuda")
    ca = torch.zeros((1, 64, 4, 128), device="cuda")
    cl = torch.zeros((1, 64, 4), device="cuda")
    af = torch.zeros((1, 64, 4, 128), dtype=torch.bfloat16, device="cuda")
    lf = torch.zeros((1, 64, 4), device="cuda")
    mask = torch.from_numpy(np.array([[1, 0, 1, 0]], np.uint8)).cuda()
    fb.residual_step(rs, dev["q"], dev["k"], dev["v"], dev["k_blk"], dev["v_blk"], sp, sc, None, ca, cl, af, lf, ws)
    cache = (ca.clone(), cl.clone())

    def reset():
        ca.copy_(cache[0])
        cl.copy_(cache[1])
        af.fill_(float("nan"))
        lf.fill_(float("nan"))

    def run():
        fb.residual_step(rs, dev["q"], dev["k"], dev["v"], dev["k_blk"], dev["v_blk"], sp, sc, mask, ca, cl, af, lf,
                         ws)
    _replays_match(run, reset, [af, lf, ca, cl])
