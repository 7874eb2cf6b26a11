"""fb_step_noalloc (the step for callers that cannot allocate: its partials live in the
library's static per-GPU array) against fb_step with a caller workspace, through the C
ABI: bit-identical outputs and cache on two calls in a row, the second with a smaller
input, and a reuse step; a shape larger than the array is refused with nothing written."""
import numpy as np
import pytest

import synth
from synth.device import tensor
from tests.gpu_util import guarded, np_of, say, to_device_guarded

pytestmark = pytest.mark.gpu


def _outs(p, name):
    import torch
    b, B, h, d = p.q.shape
    return dict(ca=guarded((b, B, h, d), torch.float32, 0.0, f"{name} cache_a"),
                cl=guarded((b, B, h), torch.float32, 0.0, f"{name} cache_l"),
                af=guarded((b, B, h, d), torch.bfloat16, 0.0, f"{name} a_full"),
                lf=guarded((b, B, h), torch.float32, 0.0, f"{name} l_full"))


def _shape(fb, p, dev):
    if p.batch == 1:
        return fb.make_shape(p.batch, p.h_q, p.h_kv, p.d, p.B, seqlen_k=int(p.seqlens[0]))
    return fb.make_shape(p.batch, p.h_q, p.h_kv, p.d, p.B, cu_seqlens_k=dev["cu"], max_seqlen_k=int(p.seqlens.max()))


def _same(x, y, what):
    assert np.array_equal(np_of(x).view(np.uint32), np_of(y).view(np.uint32)), what


def _compare(fb, p, dev, mask, q=None):
    """One fresh (or masked) step through both entry points on fresh output buffers."""
    import torch
    s = _shape(fb, p, dev)
    ws = guarded((fb.workspace_size(s),), torch.uint8, name="workspace")
    a, n = _outs(p, "fb_step"), _outs(p, "fb_step_noalloc")
    q = dev["q"] if q is None else q
    fb.step(s, q, dev["k"], dev["v"], dev["k_blk"], dev["v_blk"], mask, a["ca"], a["cl"], a["af"], a["lf"], ws)
    fb.step_noalloc(s, q, dev["k"], dev["v"], dev["k_blk"], dev["v_blk"], mask, n["ca"], n["cl"], n["af"], n["lf"])
    torch.cuda.synchronize()
    for key in ("ca", "cl", "af", "lf"):
        _same(a[key], n[key], f"{key} differs")
    assert np.isfinite(np_of(n["af"])).all()
    return a, n, s


def test_noalloc_step_matches_fb_step(gpu_lib):
    import torch
    fb = gpu_lib
    # call 1: the dLLM step at full size (prefix 32768, 32 heads, about 4 MiB of partials)
    say("[noalloc] dLLM full size")
    p = synth.dllm()
    dev = to_device_guarded(p)
    _compare(fb, p, dev, None)
    # call 2, smaller: GQA, two ragged sequences, then a reuse step on the same caches
    say("[noalloc] small ragged GQA, fresh then mixed reuse")
    p = synth.custom(91, 2, 8, 2, 128, 16, [1500, 311], std=1.0)
    dev = to_device_guarded(p)
    a, n, s = _compare(fb, p, dev, None)
    mask = torch.tensor([[0, 1] * 4, [1, 1, 0, 0] * 2], dtype=torch.uint8, device="cuda")
    q2 = tensor(synth.round_bf16(p.q * 0.5))
    ws = guarded((fb.workspace_size(s),), torch.uint8, name="workspace 2")
    fb.step(s, q2, dev["k"], dev["v"], dev["k_blk"], dev["v_blk"], mask, a["ca"], a["cl"], a["af"], a["lf"], ws)
    fb.step_noalloc(s, q2, dev["k"], dev["v"], dev["k_blk"], dev["v_blk"], mask, n["ca"], n["cl"], n["af"], n["lf"])
    torch.cuda.synchronize()
    for key in ("ca", "cl", "af", "lf"):
        _same(a[key], n[key], f"reuse step {key} differs")


def test_noalloc_refuses_a_shape_larger_than_its_array(gpu_lib):
    """The video block (4680 queries, 12 heads) needs about 84 MiB of partials: refused
    with FB_ERR_WORKSPACE before anything is enqueued."""
    import torch
    fb = gpu_lib
    s = fb.make_shape(1, 12, 12, 128, 4680, seqlen_k=32760)
    assert fb.workspace_size(s) > 64 << 20
    q = guarded((1, 4680, 12, 128), torch.bfloat16, 0.0, "q")
    kv = guarded((32760, 12, 128), torch.bfloat16, 0.0, "k")
    kb = guarded((1, 4680, 12, 128), torch.bfloat16, 0.0, "k_blk")
    ca = guarded((1, 4680, 12, 128), torch.float32, 7.0, "cache_a")
    cl = guarded((1, 4680, 12), torch.float32, 7.0, "cache_l")
    af = guarded((1, 4680, 12, 128), torch.bfloat16, 7.0, "a_full")
    with pytest.raises(fb.FlashBlockError) as e:
        fb.step_noalloc(s, q, kv, kv, kb, kb, None, ca, cl, af, None)
    assert e.value.status == 3
    torch.cuda.synchronize()
    assert (ca == 7.0).all() and (cl == 7.0).all() and (af == 7.0).all()
