"""GPU parity of the multi-branch prefix pass over packed variable-length queries
(fb_prefix_attn_varlen) through the C ABI against the fp64 oracle (oracle/varlen.py)."""
import numpy as np
import pytest

import synth
from synth.device import tensor
from oracle.varlen import prefix_attention_varlen
from tests.gpu_util import check_attn, check_lse, guarded, np_of, say

pytestmark = pytest.mark.gpu


def _run(fb, br, b_max):
    import torch
    code = fb.FB_BF16 if br["dtype"] == "bf16" else fb.FB_F32
    cu_k = torch.from_numpy(br["cu_k"]).cuda()
    cu_q = torch.from_numpy(br["cu_q"]).cuda()
    nb = len(br["blocks"])
    s = fb.make_shape(nb, br["h_q"], br["h_kv"], br["d"], b_max, dtype=code, cu_seqlens_k=cu_k,
                      max_seqlen_k=int(br["seqlens"].max()))
    tq = int(br["cu_q"][-1])
    vs = fb.make_varlen_shape(s, cu_q, tq)
    ws = guarded((max(fb.prefix_attn_varlen_workspace_size(vs), 16),), torch.uint8, name="varlen workspace")
    a = guarded((tq, br["h_q"], br["d"]), torch.float32, float("nan"), "a_out packed")
    l = guarded((tq, br["h_q"]), torch.float32, float("nan"), "l_out packed")
    k = tensor(br["k"], br["dtype"]) if br["k"].shape[0] else None
    v = tensor(br["v"], br["dtype"]) if br["v"].shape[0] else None
    fb.prefix_attn_varlen(vs, tensor(br["q"], br["dtype"]), k, v, a, l, ws)
    torch.cuda.synchronize()
    return np_of(a), np_of(l)


CASES = [
    # name, blocks, prefix lengths, h_q, h_kv, d, B_max, dtype
    ("stream_blocks_4_to_32", [4, 8, 16, 32], [300, 517, 93, 1000], 4, 4, 128, 32, "bf16"),
    ("tiled_blocks_to_128", [4, 128, 64, 0, 33], [700, 2000, 0, 50, 129], 2, 2, 128, 128, "bf16"),
    ("gqa4_stream", [8, 2, 5], [640, 1280, 77], 8, 2, 128, 8, "bf16"),
    # 2 query heads x 48 rows: a wave's 32 rows straddle the two heads, so a wave is idle
    # only where both heads' rows are padding (branch of 10: waves 0 and 1 work, 2 is idle)
    ("gqa2_tiled_heads_straddle", [40, 10, 48, 17], [500, 900, 300, 64], 4, 2, 128, 48, "bf16"),
    ("wide_256", [256, 100, 3], [900, 400, 1500], 1, 1, 128, 256, "bf16"),
    ("d64", [4, 16, 9], [200, 333, 64], 4, 2, 64, 16, "bf16"),
    ("f32", [3, 8, 1], [100, 40, 77], 4, 2, 32, 8, "f32"),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_prefix_attn_varlen(gpu_lib, case):
    name, blocks, lens, hq, hkv, d, b_max, dt = case
    say(f"[varlen] {name}")
    br = synth.branches(61, blocks, lens, hq, hkv, d, dtype=dt)
    a, l = _run(gpu_lib, br, b_max)
    ea, el = prefix_attention_varlen(br["q"], br["cu_q"], br["k"], br["v"], br["cu_k"], hkv, br["scale"])
    check_attn(a, ea, dt, f"{name} A_out")
    check_lse(l, el, dt, f"{name} L_out")


def test_prefix_attn_varlen_blockbatch_full_size(gpu_lib):
    """Six branches of one request with block sizes 4, 8, ..., 128 and their own prefixes of
    about 32k tokens (32 heads, d 128, bf16); sampled heads against the oracle."""
    blocks = [4, 8, 16, 32, 64, 128]
    lens = [32768 - 97 * i for i in range(6)]
    say("[varlen full] run")
    br = synth.branches(synth.SEED_RESIDUAL + 1, blocks, lens, 32, 32, 128, std=1.0 / np.sqrt(128.0))
    a, l = _run(gpu_lib, br, 128)
    heads = [0, 17, 31]
    sub = dict(br)
    sub["q"], sub["k"], sub["v"] = br["q"][:, heads], br["k"][:, heads], br["v"][:, heads]
    say("[varlen full] oracle")
    ea, el = prefix_attention_varlen(sub["q"], br["cu_q"], sub["k"], sub["v"], br["cu_k"], 3, br["scale"])
    check_attn(a[:, heads], ea, "bf16", "blockbatch A_out")
    check_lse(l[:, heads], el, "bf16", "blockbatch L_out")
