"""The measured-ceiling kernels (include/fb_ceiling.h) on the GPU: the streaming read
touches every 16-byte word of its buffer exactly once, with plain and with non-temporal
loads (the XOR of the workgroups' sink entries equals the XOR of the buffer, computed on the
host); the MFMA loop does all the multiply-adds it is counted for (its per-wave sums are
exact); the co-issue measurement runs the streams each mode names (the MFMA waves' sums are
exact, every vector chain ends at exactly 0) and nothing else."""
import numpy as np
import pytest

from tests.gpu_util import say

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("nontemporal", [False, True])
@pytest.mark.parametrize("nbytes,workgroups", [(16, 1), (4096, 3), (1_000_000 * 16, 7), (536_870_912, 4096),
                                                (536_870_912 + 48, 1024)])
def test_stream_read_reads_every_word_once(gpu_lib, nbytes, workgroups, nontemporal):
    import torch
    from cached_kv_prefix_amd import ceiling
    say(f"[ceiling] stream read {nbytes} B, {workgroups} workgroups, nontemporal {nontemporal}")
    g = torch.Generator(device="cuda")
    g.manual_seed(nbytes % 1000003)
    words = torch.randint(-(1 << 31), (1 << 31) - 1, (nbytes // 4,), dtype=torch.int32, device="cuda", generator=g)
    sink = torch.full((workgroups, 4), -1, dtype=torch.int32, device="cuda")
    ceiling.stream_read(words, nbytes, workgroups, sink, nontemporal=nontemporal)
    torch.cuda.synchronize()
    got = np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32), axis=0)
    want = np.bitwise_xor.reduce(words.cpu().numpy().view(np.uint32).reshape(-1, 4), axis=0)
    assert (got == want).all(), (got, want)


@pytest.mark.parametrize("workgroups,iters,a,b", [(1, 1, 1.0, 1.0), (5, 1000, 1.0, 1.0), (512, 262144, 1.0, 1.0),
                                                  (256, 4096, 0.5, -2.0)])
def test_mfma_loop_does_the_counted_work(gpu_lib, workgroups, iters, a, b):
    import torch
    from cached_kv_prefix_amd import ceiling
    say(f"[ceiling] mfma loop {workgroups} workgroups x {iters} iterations")
    sink = torch.full((workgroups * 4,), float("nan"), device="cuda")
    ceiling.mfma_loop(workgroups, iters, a, b, sink)
    torch.cuda.synchronize()
    want = 4 * 16 * iters * a * b
    assert (sink.cpu().numpy() == np.float32(want)).all(), sink[:8]


@pytest.mark.parametrize("mode", ["mfma", "valu", "pair", "interleaved"])
@pytest.mark.parametrize("valu_per_mfma", [2, 4, 8])
@pytest.mark.parametrize("workgroups,rounds", [(1, 1), (256, 2000), (3, 262144)])
def test_mfma_valu_runs_each_stream_it_names(gpu_lib, mode, valu_per_mfma, workgroups, rounds):
    import torch
    from cached_kv_prefix_amd import ceiling
    say(f"[ceiling] mfma/valu {mode} K={valu_per_mfma}, {workgroups} workgroups x {rounds} rounds")
    sink = torch.full((workgroups, 8), float("nan"), device="cuda")
    ceiling.mfma_valu(mode, valu_per_mfma, workgroups, rounds, sink)
    torch.cuda.synchronize()
    got = sink.cpu().numpy()
    for j, want in enumerate(ceiling.mfma_valu_expected(mode, rounds)):
        if want is None:
            assert np.isnan(got[:, j]).all(), (mode, j)
        else:
            assert (got[:, j] == np.float32(want)).all(), (mode, j, got[:4, j])
