"""Benchmark of the FlashBlock step on one MI355X.

Headline workload: dLLM-like step, batch 1, 32 heads (MHA), head_dim 128, block B = 32,
prefix 32768 tokens, bf16, Q/K/V ~ N(0,1)/sqrt(128).  One step = the reuse decision
(threshold rule on the drawn updated-token count) + fb_step (split-KV prefix pass, block
pass, chunk reduction, cache write and log-space merge).  The timed step is a fresh
(recompute) step: every prefix token is read.

Prints ONE JSON line.  `value` is the K/V bytes of the prefix read per second of step
time (inputs resident in HBM).  `roofline` is the attention kernel's algorithmic bytes
over its own average duration (HIP events recorded by the library on its stream around
that kernel); beside the published peak it carries the read rate a plain streaming kernel
reaches on this chip (`measured_peak`, `frac_of_measured`).  `cpu_baseline` is the fp64
oracle timed on the host cores on a bounded sample of the same step.  `extra` holds the reuse step, an 8-step block, and the other
workloads (ragged GQA, video block, LoSA sparse step).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, TFLOP/s
COUNTERS = os.path.join(ROOT, "profiles", "attn_stream_dllm_pmc.txt")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--only-main", action="store_true", help="headline workload only (for profiling)")
    ap.add_argument("--only-others", action="store_true",
                    help="ragged-GQA and LoSA sparse steps only, one JSON line of their times (for profiling)")
    ap.add_argument("--only-video", choices=["masked", "fresh"], default=None,
                    help="video-block steps only, masked (7 of 12 heads reuse) or all fresh, one JSON line of "
                         "their time (for profiling)")
    ap.add_argument("--video-splits", action="store_true",
                    help="video-block masked and all-fresh steps at forced prefix split counts (2, 5, 8, 16) and "
                         "at the plan's own, one JSON line (for the split-plan evidence)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle CPU baseline")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="run one device copy of this many MiB first (counter calibration)")
    return ap.parse_args()


class HipEvents:
    """HIP events created through the runtime, so that events the library records on its
    stream can be read back (torch.cuda.Event only tracks its own record() calls)."""
    def __init__(self, n):
        import ctypes as C
        self.C = C
        self.rt = C.CDLL("libamdhip64.so")
        self.rt.hipEventCreate.argtypes = [C.POINTER(C.c_void_p)]
        self.rt.hipEventElapsedTime.argtypes = [C.POINTER(C.c_float), C.c_void_p, C.c_void_p]
        self.rt.hipEventDestroy.argtypes = [C.c_void_p]
        self.ev = []
        for _ in range(n):
            pair = []
            for _ in range(2):
                e = C.c_void_p()
                assert self.rt.hipEventCreate(C.byref(e)) == 0
                pair.append(e)
            self.ev.append(tuple(pair))

    def ms(self):
        out = []
        for a, b in self.ev:
            x = self.C.c_float()
            assert self.rt.hipEventElapsedTime(self.C.byref(x), a, b) == 0
            out.append(x.value)
        return out

    def close(self):
        for a, b in self.ev:
            self.rt.hipEventDestroy(a)
            self.rt.hipEventDestroy(b)


def setup_step(fb, p, dev, varlen=False):
    import torch
    shape = (fb.make_shape(p.batch, p.h_q, p.h_kv, p.d, p.B, cu_seqlens_k=dev["cu"], max_seqlen_k=int(p.seqlens.max()))
             if varlen else fb.make_shape(p.batch, p.h_q, p.h_kv, p.d, p.B, seqlen_k=int(p.seqlens[0])))
    b, B, h, d = p.q.shape
    bufs = dict(
        ws=torch.empty(fb.workspace_size(shape), dtype=torch.uint8, device="cuda"),
        ca=torch.zeros((b, B, h, d), device="cuda"), cl=torch.zeros((b, B, h), device="cuda"),
        af=torch.zeros((b, B, h, d), dtype=torch.bfloat16, device="cuda"), lf=torch.zeros((b, B, h), device="cuda"),
        mask=torch.zeros((b, h), dtype=torch.uint8, device="cuda"),
    )
    return shape, bufs


def run_step(fb, shape, dev, bufs, mask_src=None, tau=4, trace=None, sim=None, gamma=0.95):
    """One step: the threshold rule (updated-token count per sequence, evaluated inside the
    step) or the similarity rule (per-head mask, then the step); no rule = recompute all."""
    if mask_src is not None:
        fb.step_threshold(shape, dev["q"], dev["k"], dev["v"], dev["k_blk"], dev["v_blk"], mask_src, tau,
                          bufs["ca"], bufs["cl"], bufs["af"], bufs["lf"], bufs["ws"], trace=trace)
        return
    if sim is not None:
        fb.mask_similarity(sim, gamma, bufs["mask"])
    fb.step(shape, dev["q"], dev["k"], dev["v"], dev["k_blk"], dev["v_blk"], bufs["mask"], bufs["ca"], bufs["cl"],
            bufs["af"], bufs["lf"], bufs["ws"], trace=trace)


def wall_time(fn, steps, warmup):
    """Warm up, then the wall time per call of `steps` calls back to back (synchronised on
    both sides)."""
    import torch
    for _ in range(warmup):
        fn(None)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        fn(None)
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) / steps


def time_steps(fn, steps, warmup):
    """Warm up, then time `steps` calls back to back (synchronised on both sides): the wall
    time per step.  A second pass of `steps` calls has the library record a HIP event pair
    around the attention kernel of every call (on its own stream); those give the kernel
    durations, and the recording stays out of the wall-time pass."""
    import torch
    import cached_kv_prefix_amd as fb
    for _ in range(warmup):
        fn(None)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        fn(None)
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) / steps
    ev = HipEvents(steps)
    tr = []
    for a, b in ev.ev:
        t = fb.FbTrace()
        t.attn_begin, t.attn_end = a.value, b.value
        tr.append(t)
    torch.cuda.synchronize()
    for i in range(steps):
        fn(tr[i])
    torch.cuda.synchronize()
    kern = ev.ms()
    ev.close()
    return wall, float(np.mean(kern)) / 1e3, kern


def graph_step_time(fn, steps, warmup=3):
    """One call of fn captured into a HIP graph (stream capture through torch.cuda.CUDAGraph),
    then `steps` replays back to back: the step time without the host's per-launch cost.
    The step itself enqueues no memset, so the graph holds kernel nodes only."""
    import torch
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn(None)
    torch.cuda.current_stream().wait_stream(side)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn(None)
    for _ in range(warmup):
        g.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        g.replay()
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) / steps
    del g
    return wall


def flushed_step_times(fn, n=100):
    """Per-step event timing after a 1 GiB read before each step (outside the events), so
    the 256 MB last-level cache holds none of the inputs.  A read, not a write: dirty
    lines left by a write would be written back during the timed step.  Returns the
    per-step times (s)."""
    import torch
    scratch = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
    sink = torch.empty((), dtype=torch.float32, device="cuda")
    out = []
    for _ in range(n):
        torch.sum(scratch, dim=0, out=sink)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        fn(None)
        b.record()
        torch.cuda.synchronize()
        out.append(a.elapsed_time(b) / 1e3)
    del scratch
    return out


STREAM_KERNEL = "fb::attn_stream_kernel<1, 40, false>"


# The sources the streaming kernel and its launch are built from: the kernel, the dispatch,
# the shared device helpers and descriptors, and the host split plan.
STREAM_SOURCES = ("fb_stream.hip", "fb_attn.hip", "fb_attn_common.hpp", "fb_device.hpp", "fb_internal.hpp",
                  "fb_api.hip")


def kernel_source_sha():
    """Fingerprint of the sources the headline attention launch depends on."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "cached_kv_prefix_amd", "csrc")
    for name in STREAM_SOURCES:
        h.update(name.encode())
        h.update(open(os.path.join(csrc, name), "rb").read())
    return h.hexdigest()


def counters_for(src_sha):
    """HBM traffic of the attention kernel from the committed rocprofv3 --pmc summary, if
    it was taken on the current kernel source."""
    if not os.path.exists(COUNTERS):
        return None
    kv = {}
    for line in open(COUNTERS):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    if kv.get("kernel_source_sha256") != src_sha:
        return None
    try:
        return float(kv["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def cpu_baseline(p):
    """The oracle (numpy fp64, as it stands) on a bounded sample of the headline step:
    the full prefix pass of a few heads plus their block pass and merge."""
    from oracle.attention import attend, lse_merge
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = len(os.sched_getaffinity(0))
    heads = [0, 1, 2, 3]
    t0 = time.perf_counter()
    reps = 0
    while True:
        for h in heads:
            ao, lo = attend(p.q[0, :, h], p.k[:, h], p.v[:, h], p.scale)
            ai, li = attend(p.q[0, :, h], p.k_blk[0, :, h], p.v_blk[0, :, h], p.scale)
            lse_merge(ao, lo, ai, li)
        reps += 1
        el = time.perf_counter() - t0
        if el > 10.0 or reps >= 20:
            break
    per_head = el / (reps * len(heads))
    step_s = per_head * p.h_q
    kv_bytes = p.k.shape[0] * p.h_kv * p.d * 2 * 2
    out = dict(value=kv_bytes / step_s / 1e9, unit="GB/s", cores=int(threads), kind="oracle",
               sample=f"{len(heads)} of {p.h_q} heads x {reps} reps (full 32768-token prefix + block + merge per "
                      f"head), scaled to the 32-head step: {step_s * 1e3:.1f} ms per step",
               step_ms=step_s * 1e3)
    # one BLAS thread: one head of the same step, scaled to the 32-head step; and the tiny fp32
    # two-step case (fresh + reuse) whole
    try:
        from threadpoolctl import threadpool_limits
        import synth
        from oracle.flashblock import step as oracle_step
        with threadpool_limits(limits=1):
            t0 = time.perf_counter()
            ao, lo = attend(p.q[0, :, 0], p.k[:, 0], p.v[:, 0], p.scale)
            ai, li = attend(p.q[0, :, 0], p.k_blk[0, :, 0], p.v_blk[0, :, 0], p.scale)
            lse_merge(ao, lo, ai, li)
            out["single_thread_step_ms"] = (time.perf_counter() - t0) * p.h_q * 1e3
            t = synth.tiny()
            t0 = time.perf_counter()
            z = np.zeros((1, t.h_q), np.uint8)
            _, _, ca, cl = oracle_step(t.q, t.k, t.v, t.cu, t.k_blk, t.v_blk, z, None, None, t.scale)
            oracle_step(t.extra["q_step1"], t.k, t.v, t.cu, t.k_blk, t.v_blk, 1 - z, ca, cl, t.scale)
            out["single_thread_tiny_two_steps_ms"] = (time.perf_counter() - t0) * 1e3
    except ImportError:
        pass
    return out


def cpu_baseline_others(probs):
    """The oracle (as it stands, all host BLAS threads) on bounded samples of the other
    workloads' steps, each scaled to its whole step:
      * video block, masked step (7 of 12 heads reuse): a seeded 256 of the 4680 block rows,
        every head (recomputing heads: prefix + block + merge; reusing heads: block + merge
        on stand-in cached rows), scaled by 4680 / 256;
      * ragged GQA, all-fresh step: 2 of the 8 sequences, every head, scaled by the total
        prefix length over theirs;
      * LoSA sparse step: the whole step (selection, sparse prefix for the active rows,
        block and merge for all 64 rows) on stand-in cached rows."""
    import synth
    from oracle import flashblock as OF
    from oracle import losa as OL
    out = {}
    p = probs.get("video")
    if p is not None:
        rows = np.sort(synth.rng(31).choice(p.B, size=256, replace=False))
        mask = OF.mask_similarity(p.extra["sim"], p.extra["gamma"])
        ca = np.zeros((1, 256, p.h_q, p.d))
        cl = np.zeros((1, 256, p.h_q))
        t0 = time.perf_counter()
        OF.step(p.q[:, rows], p.k, p.v, p.cu, p.k_blk, p.v_blk, mask, ca, cl, p.scale)
        step_s = (time.perf_counter() - t0) * p.B / 256
        n_fresh = int((mask == 0).sum())
        flop = 4.0 * p.B * p.B * p.d * p.h_q + n_fresh * 4.0 * p.B * int(p.seqlens[0]) * p.d
        out["video_block"] = dict(value=flop / step_s / 1e12, unit="TFLOP/s", step_ms=step_s * 1e3,
                                  sample="masked step on 256 of 4680 block rows x 12 heads, scaled to 4680 rows")
    p = probs.get("ragged")
    if p is not None:
        t0 = time.perf_counter()
        n_s = 0
        for b in (0, 1):
            lo, hi = int(p.cu[b]), int(p.cu[b + 1])
            z = np.zeros((1, p.h_q), np.uint8)
            OF.step(p.q[b:b + 1], p.k[lo:hi], p.v[lo:hi], np.array([0, hi - lo], np.int32), p.k_blk[b:b + 1],
                    p.v_blk[b:b + 1], z, None, None, p.scale)
            n_s += hi - lo
        step_s = (time.perf_counter() - t0) * float(p.seqlens.sum()) / n_s
        kv = float(p.seqlens.sum()) * p.h_kv * p.d * 4
        out["ragged_gqa"] = dict(value=kv / step_s / 1e9, unit="GB/s", step_ms=step_s * 1e3,
                                 sample=f"all-fresh step of sequences 0 and 1 ({n_s} of {int(p.seqlens.sum())} "
                                        f"prefix tokens), scaled to the 8 sequences")
    p = probs.get("losa")
    if p is not None:
        ca = np.zeros(p.q.shape)
        cl = np.zeros(p.q.shape[:3])
        t0 = time.perf_counter()
        OL.step(p.extra["q_cur"], p.extra["q_prev"], p.k, p.v, p.cu, p.k_blk, p.v_blk, ca, cl, 8, 16, 64, p.scale)
        step_s = time.perf_counter() - t0
        out["losa_sparse"] = dict(value=step_s * 1e3, unit="ms per sparse step", step_ms=step_s * 1e3,
                                  sample="the whole sparse step (131072-token prefix, 32 heads, B 64, |A| 8, "
                                         "top-64 of 8192 pages)")
    return out


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU only; --gpus must be 1"}))
        sys.exit(2)
    import torch
    import cached_kv_prefix_amd as fb
    import synth
    from synth.device import to_device, tensor
    fb.load()
    torch.cuda.init()

    if args.copy_probe_mib > 0:
        src = torch.ones(args.copy_probe_mib << 20, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    if args.only_others:
        print(json.dumps({"only_others": only_others(fb, args)}))
        return
    if args.only_video:
        print(json.dumps({"only_video": only_video(fb, args, args.only_video)}))
        return
    if args.video_splits:
        print(json.dumps({"video_splits": video_splits(fb, args)}))
        return

    # ---------------------------------------------------------------- headline workload
    p = synth.dllm()
    dev = to_device(p)
    shape, bufs = setup_step(fb, p, dev)
    m_all = torch.from_numpy(p.extra["m_updated"]).cuda()       # [8 steps, batch]
    m_fresh = m_all[0]                                           # step 0: recompute
    wall, attn_s, kern_ms = time_steps(lambda tr: run_step(fb, shape, dev, bufs, m_fresh, trace=tr),
                                       args.steps, args.warmup)
    kv_bytes = p.k.shape[0] * p.h_kv * p.d * 2 * 2               # K and V of the prefix
    attn_bytes = kv_bytes + p.q.size * 2 + p.k_blk.size * 2 * 2  # + Q + block K/V
    value = kv_bytes / wall / 1e9
    src_sha = kernel_source_sha()
    traffic = counters_for(src_sha)
    achieved = attn_bytes / attn_s / 1e9

    kq = np.percentile(np.asarray(kern_ms) * 1e3, [10, 50, 90])
    extra = {"step_us": wall * 1e6, "attn_kernel_us": attn_s * 1e6,
             "attn_kernel_us_p10_p50_p90": [float(x) for x in kq], "tokens_per_s": p.B / wall,
             "kv_bytes": kv_bytes, "attn_kernel_alg_bytes": attn_bytes,
             "step_frac_of_hbm_peak": value / HBM_PEAK_GBS}
    problems = {}
    if not args.only_main:
        # reuse step: every head reuses, only the block pass and the merge run
        one = torch.zeros_like(m_fresh)
        wall_r, _, _ = time_steps(lambda tr: run_step(fb, shape, dev, bufs, one, trace=tr), args.steps, 3)
        extra["reuse_step_us"] = wall_r * 1e6
        extra["reuse_step_graph_us"] = graph_step_time(lambda tr: run_step(fb, shape, dev, bufs, one, trace=tr),
                                                       args.steps) * 1e6
        extra["fresh_step_graph_us"] = graph_step_time(lambda tr: run_step(fb, shape, dev, bufs, m_fresh, trace=tr),
                                                       args.steps) * 1e6
        # an 8-step block with the drawn M (tau 4): mean step time
        def block(tr):
            for s in range(8):
                run_step(fb, shape, dev, bufs, m_all[s], trace=tr)
        wall_b, _, _ = time_steps(block, max(5, args.steps // 8), 2)
        fresh = int(1 + (p.extra["m_updated"][1:, 0] >= 4).sum())
        extra["block8_mean_step_us"] = wall_b / 8 * 1e6
        extra["block8_fresh_steps"] = fresh
        cold = np.asarray(flushed_step_times(lambda tr: run_step(fb, shape, dev, bufs, m_fresh))) * 1e6
        extra["cold_fresh_step_us"] = float(np.median(cold))
        extra["cold_fresh_step_us_p10_p50_p90"] = [float(x) for x in np.percentile(cold, [10, 50, 90])]
        ceil = measured_ceilings(kv_bytes)
        extra["ceilings"] = ceil
        extra["workloads"] = other_workloads(fb, args, keep=problems)
        vb = extra["workloads"]["video_block"]
        vb["masked_frac_of_measured_mfma"] = vb["masked_TFLOPs"] / ceil["mfma_bf16_TFLOPs"]
        vb["attn_kernel_all_fresh_frac_of_measured_mfma"] = (vb["attn_kernel_all_fresh_frac_mfma"] * MFMA_BF16_PEAK_TFLOPS
                                                            / ceil["mfma_bf16_TFLOPs"])
        extra["context_sweep"] = context_sweep(fb, args)
        extra["lifecycle"] = lifecycle_workload(fb, args)
    result = {
        "metric": "attn step µs & KV GB/s (B=32, 32k prefix, bf16); % of HBM/MFMA peak",
        "value": value, "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": wall * 1e3, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "dLLM fresh step: batch 1, 32 heads MHA, head_dim 128, block 32, prefix 32768, bf16, "
                               "Q/K/V ~ N(0,1)/sqrt(128)", "global_batch": 1, "seq_len": 32768, "block": 32,
                   "parallelism": "none (1 GPU)"},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": traffic,
                     "kernel": STREAM_KERNEL + " (split-KV prefix + block pass, one launch)"},
        "extra": extra,
    }
    if "ceilings" in extra:   # the same kernel against the read rate measured on this chip
        result["roofline"]["measured_peak"] = extra["ceilings"]["stream_read_GBps"]
        result["roofline"]["frac_of_measured"] = achieved / extra["ceilings"]["stream_read_GBps"]
    if not args.no_cpu:
        result["cpu_baseline"] = cpu_baseline(p)
        if problems:
            result["cpu_baseline"]["other_workloads"] = cpu_baseline_others(problems)
    print(json.dumps(result))


def measured_ceilings(nbytes: int):
    """The rates this chip reaches on the two resources the attention kernels are bound by,
    measured here beside the published peaks: a streaming read of `nbytes` with plain and with
    non-temporal loads (one launch at a time, each timed with events, as the attention kernel
    is), and a register-only bf16 MFMA loop on every CU (2 workgroups of 4 waves per CU,
    about 2 ms per launch).  Also how far MFMA work of one wave and vector work (exp and fma,
    4 per MFMA, the softmax mix) of another overlap on one SIMD."""
    import torch
    from cached_kv_prefix_amd import ceiling
    ceiling.load()
    buf = torch.empty(nbytes // 4, dtype=torch.int32, device="cuda")
    buf.fill_(0x01010101)
    wgs = 4096
    sink = torch.empty((wgs, 4), dtype=torch.int32, device="cuda")

    def read_us(nt):
        for _ in range(3):
            ceiling.stream_read(buf, nbytes, wgs, sink, nontemporal=nt)
        times = []
        for _ in range(20):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            ceiling.stream_read(buf, nbytes, wgs, sink, nontemporal=nt)
            e1.record()
            times.append((e0, e1))
        torch.cuda.synchronize()
        return float(np.mean([a.elapsed_time(b) for a, b in times])) * 1e3

    plain_us, nt_us = read_us(False), read_us(True)
    del buf, sink
    n_cu = torch.cuda.get_device_properties(0).multi_processor_count
    mwg, iters = 2 * n_cu, 16384
    msink = torch.empty(mwg * 4, device="cuda")
    ceiling.mfma_loop(mwg, 256, 1.0, 1.0, msink)
    rates = []
    for _ in range(5):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        ceiling.mfma_loop(mwg, iters, 1.0, 1.0, msink)
        e1.record()
        torch.cuda.synchronize()
        rates.append(ceiling.mfma_flops(mwg, iters) / (e0.elapsed_time(e1) * 1e-3) / 1e12)
    assert (msink.cpu().numpy() == np.float32(64 * iters)).all(), "MFMA loop result"
    coissue = mfma_valu_overlap(n_cu)
    best_us = min(plain_us, nt_us)
    return {"stream_read_GBps": nbytes / (best_us * 1e-6) / 1e9, "stream_read_us": best_us,
            "stream_read_plain_GBps": nbytes / (plain_us * 1e-6) / 1e9, "stream_read_plain_us": plain_us,
            "stream_read_nontemporal_GBps": nbytes / (nt_us * 1e-6) / 1e9, "stream_read_nontemporal_us": nt_us,
            "stream_read_bytes": nbytes,
            "mfma_bf16_TFLOPs": float(np.median(rates)), "mfma_workgroups": mwg,
            "mfma_valu_coissue": coissue,
            "probe": "libfb_ceiling.so: grid-stride 16-byte reads (4096 x 256 threads), plain and non-temporal, "
                     "the faster one taken as the read ceiling; 4 independent v_mfma_f32_32x32x16_bf16 chains per "
                     "wave; fbc_mfma_valu for the co-issue"}


def mfma_valu_overlap(n_cu: int, k: int = 4, rounds: int = 8192):
    """Launch times of fbc_mfma_valu's four modes, one workgroup per CU: the MFMA stream alone
    (one wave per SIMD), the vector stream alone, both side by side (two waves per SIMD) and
    both interleaved in one wave.  `overlap` = (t_mfma + t_valu - t_pair) / min(t_mfma, t_valu):
    1 when the shorter stream hides entirely under the longer, 0 when they add up."""
    import torch
    from cached_kv_prefix_amd import ceiling
    sink = torch.empty((n_cu, 8), device="cuda")
    out = {"valu_per_mfma": k, "rounds": rounds, "workgroups": n_cu}
    for mode in ("mfma", "valu", "pair", "interleaved"):
        ceiling.mfma_valu(mode, k, n_cu, 64, sink)
        ts = []
        for _ in range(5):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            ceiling.mfma_valu(mode, k, n_cu, rounds, sink)
            e1.record()
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1) * 1e3)
        got = sink.cpu().numpy()
        for j, want in enumerate(ceiling.mfma_valu_expected(mode, rounds)):
            if want is not None:
                assert (got[:, j] == np.float32(want)).all(), f"fbc_mfma_valu {mode} result"
        out[f"{mode}_us"] = float(np.median(ts))
    t_m, t_v, t_p = out["mfma_us"], out["valu_us"], out["pair_us"]
    out["overlap"] = (t_m + t_v - t_p) / min(t_m, t_v)
    return out


def sdpa_reference(dev, p, flop):
    """torch's scaled_dot_product_attention, flash backend only, on the all-fresh video
    computation (every block query over prefix + block keys, the bf16 inputs above), timed
    as a reference for what a library attention reaches on this shape.  Only the flash
    backend is allowed (no fallback to the math path).  None when it is not available."""
    import torch
    try:
        from torch.nn.attention import SDPBackend, sdpa_kernel
        q = dev["q"][0].transpose(0, 1).contiguous().unsqueeze(0)                       # [1, h, B, d]
        k = torch.cat([dev["k"], dev["k_blk"][0]], 0).transpose(0, 1).contiguous().unsqueeze(0)
        v = torch.cat([dev["v"], dev["v_blk"][0]], 0).transpose(0, 1).contiguous().unsqueeze(0)
        with sdpa_kernel([SDPBackend.FLASH_ATTENTION]):
            for _ in range(2):
                torch.nn.functional.scaled_dot_product_attention(q, k, v, scale=p.scale)
            ts = []
            for _ in range(5):
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record()
                torch.nn.functional.scaled_dot_product_attention(q, k, v, scale=p.scale)
                e1.record()
                torch.cuda.synchronize()
                ts.append(e0.elapsed_time(e1) * 1e3)
        del q, k, v
        us = float(np.median(ts))
        return {"us": us, "TFLOPs": flop / (us * 1e-6) / 1e12, "frac_mfma": flop / (us * 1e-6) / 1e12 / MFMA_BF16_PEAK_TFLOPS}
    except Exception as e:   # no flash kernel in this torch build
        return {"us": None, "error": type(e).__name__}


def context_sweep(fb, args, lengths=(102400, 204800, 409600, 819200)):
    """Prefix lengths 100k -> 800k on the dLLM step shape (32 heads, d 128, B 32, bf16):
    the always-fresh step and the mean step of an 8-step block under the threshold rule
    (tau 4, M drawn as in the dLLM workload).  The growth of each with the context, as a
    ratio, is the shape the FlashBlock pages claim (reuse roughly halves it).  Inputs are
    drawn on the device from a seeded generator (N(0,1)/sqrt(128), rounded to bf16); the
    kernels and split plans are the ones the parity tests cover."""
    import torch
    import synth
    gen = torch.Generator(device="cuda")
    gen.manual_seed(11)
    H, d, B = 32, 128, 32
    m_all = torch.from_numpy(synth.dllm().extra["m_updated"]).cuda()   # [8 steps, 1]
    out = []
    steps = max(5, args.steps // 5)
    for n in lengths:
        def draw(*shape):
            return (torch.randn(*shape, generator=gen, device="cuda") / np.sqrt(128.0)).to(torch.bfloat16)
        dev = dict(q=draw(1, B, H, d), k=draw(n, H, d), v=draw(n, H, d), k_blk=draw(1, B, H, d),
                   v_blk=draw(1, B, H, d))
        shape = fb.make_shape(1, H, H, d, B, seqlen_k=n)
        bufs = dict(ws=torch.empty(fb.workspace_size(shape), dtype=torch.uint8, device="cuda"),
                    ca=torch.zeros((1, B, H, d), device="cuda"), cl=torch.zeros((1, B, H), device="cuda"),
                    af=torch.zeros((1, B, H, d), dtype=torch.bfloat16, device="cuda"),
                    lf=torch.zeros((1, B, H), device="cuda"), mask=torch.zeros((1, H), dtype=torch.uint8, device="cuda"))
        fresh, _, _ = time_steps(lambda tr: run_step(fb, shape, dev, bufs, m_all[0], trace=tr), steps, 3)

        def block(tr):
            for s_ in range(8):
                run_step(fb, shape, dev, bufs, m_all[s_], trace=tr)
        blk, _, _ = time_steps(block, max(3, steps // 4), 1)
        out.append({"prefix": n, "fresh_step_us": fresh * 1e6, "block8_mean_step_us": blk / 8 * 1e6,
                    "fresh_kv_GBps": n * H * d * 4 / fresh / 1e9})
        del dev, bufs
        torch.cuda.empty_cache()
    f0, f1 = out[0]["fresh_step_us"], out[-1]["fresh_step_us"]
    b0, b1 = out[0]["block8_mean_step_us"], out[-1]["block8_mean_step_us"]
    return {"points": out, "fresh_growth_us": f1 - f0, "block8_growth_us": b1 - b0,
            "growth_ratio_block8_over_fresh": (b1 - b0) / (f1 - f0),
            "fresh_steps_per_block": int(1 + (synth.dllm().extra["m_updated"][1:, 0] >= 4).sum())}


def lifecycle_workload(fb, args, blocks=4, S=8):
    """Multi-block run on the dLLM step shape (32 heads, d 128, B 32): a prefix of 32768
    tokens grows by one block per block.  Per block: fb_block_run over S steps under the
    threshold rule (tau 4; M drawn as in the dLLM workload, one draw per block), the same
    steps under the per-head similarity rule (gamma 0.95: a head reuses from step 2 on when
    the cosine of its cached A_out before and after the previous step is above gamma), then
    fb_append_block in place.  Per-step queries drift by N(0, 0.01^2) around the block's
    queries and the block K/V by N(0, 0.05^2); inputs are drawn on the device from a seeded
    generator.  Reports the time per block and per step, and the reuse statistics of each
    rule (the masks each step used, and the per-head cosine of consecutive prefix outputs)."""
    import torch
    gen = torch.Generator(device="cuda")
    gen.manual_seed(13)
    H, d, B, N0 = 32, 128, 32, 32768
    g = np.random.Generator(np.random.PCG64(13))
    m_all = g.integers(0, 9, size=(blocks, S, 1)).astype(np.int32)

    def draw(*shape, std=1.0 / np.sqrt(128.0)):
        return (torch.randn(*shape, generator=gen, device="cuda") * std).to(torch.bfloat16)
    cap = N0 + blocks * B
    k = torch.empty((cap, H, d), dtype=torch.bfloat16, device="cuda")
    v = torch.empty_like(k)
    k[:N0] = draw(N0, H, d)
    v[:N0] = draw(N0, H, d)
    plans = {"threshold": fb.BlockPlan(S, fb.FB_RULE_THRESHOLD, 4, 0.0),
             "similarity": fb.BlockPlan(S, fb.FB_RULE_SIMILARITY, 0, 0.95)}
    per_rule = {r: [] for r in plans}
    for j in range(blocks):
        q0, kb0, vb0 = draw(1, B, H, d), draw(1, B, H, d), draw(1, B, H, d)
        q = torch.stack([q0 + draw(1, B, H, d, std=0.01) for _ in range(S)])
        kb = torch.stack([kb0 + draw(1, B, H, d, std=0.05) for _ in range(S)])
        vb = torch.stack([vb0 + draw(1, B, H, d, std=0.05) for _ in range(S)])
        n = N0 + j * B
        shape = fb.make_shape(1, H, H, d, B, seqlen_k=n)
        m = torch.from_numpy(m_all[j]).cuda()
        for rule, plan in plans.items():
            bufs = dict(ca=torch.zeros((1, B, H, d), device="cuda"), cl=torch.zeros((1, B, H), device="cuda"),
                        af=torch.empty((S, 1, B, H, d), dtype=torch.bfloat16, device="cuda"),
                        masks=torch.empty((S, 1, H), dtype=torch.uint8, device="cuda"),
                        sims=torch.empty((S, 1, H), device="cuda"),
                        ws=torch.empty(fb.block_workspace_size(shape), dtype=torch.uint8, device="cuda"))

            def run(tr):
                fb.block_run(shape, plan, q, k, v, kb, vb, m if rule == "threshold" else None, bufs["ca"],
                             bufs["cl"], bufs["af"], None, bufs["masks"], bufs["sims"], bufs["ws"])
            wall = wall_time(run, max(3, args.steps // 10), 1)
            masks = bufs["masks"].cpu().numpy()
            sims = bufs["sims"].cpu().numpy()[1:]
            per_rule[rule].append({"prefix": n, "block_us": wall * 1e6, "step_mean_us": wall / S * 1e6,
                                   "reused_head_steps": int(masks.sum()), "head_steps": int(masks.size),
                                   "sim_min": float(np.nanmin(sims)), "sim_mean": float(np.nanmean(sims))})
        fb.append_block(shape, k, v, kb[-1], vb[-1], k, v)   # in place: the block follows the prefix
    torch.cuda.synchronize()
    out = {"prefix_final": N0 + blocks * B}
    for rule, per_block in per_rule.items():
        reused = sum(b_["reused_head_steps"] for b_ in per_block)
        total = sum(b_["head_steps"] for b_ in per_block)
        out[rule] = {"blocks": per_block, "reuse_fraction": reused / total,
                     "step_mean_us": float(np.mean([b_["step_mean_us"] for b_ in per_block]))}
    # the threshold rule's figures at the top level, as before
    out["reuse_fraction"] = out["threshold"]["reuse_fraction"]
    out["step_mean_us"] = out["threshold"]["step_mean_us"]
    return out


def varlen_workload(fb, args):
    """Multi-branch prefix pass: six branches of one request with block sizes 4, 8, 16, 32,
    64, 128 (packed: 252 query rows) and their own prefixes of 32768 - 97 i tokens (32 heads
    MHA, d 128, bf16, N(0,1)/sqrt(128)); one fb_prefix_attn_varlen call per step."""
    import torch
    import synth
    from synth.device import tensor
    blocks = [4, 8, 16, 32, 64, 128]
    lens = [32768 - 97 * i for i in range(6)]
    br = synth.branches(synth.SEED_RESIDUAL + 1, blocks, lens, 32, 32, 128, std=1.0 / np.sqrt(128.0))
    cu_k = torch.from_numpy(br["cu_k"]).cuda()
    cu_q = torch.from_numpy(br["cu_q"]).cuda()
    s = fb.make_shape(6, 32, 32, 128, 128, cu_seqlens_k=cu_k, max_seqlen_k=max(lens))
    tq = int(br["cu_q"][-1])
    vs = fb.make_varlen_shape(s, cu_q, tq)
    ws = torch.empty(fb.prefix_attn_varlen_workspace_size(vs), dtype=torch.uint8, device="cuda")
    a = torch.empty((tq, 32, 128), device="cuda")
    l = torch.empty((tq, 32), device="cuda")
    q, k, v = tensor(br["q"]), tensor(br["k"]), tensor(br["v"])
    steps = max(5, args.steps // 5)
    w = wall_time(lambda tr: fb.prefix_attn_varlen(vs, q, k, v, a, l, ws), steps, 2)
    kv = float(sum(lens)) * 32 * 128 * 2 * 2
    return {"step_us": w * 1e6, "kv_bytes": kv, "kv_GBps": kv / w / 1e9, "frac_hbm": kv / w / 1e9 / HBM_PEAK_GBS,
            "branches": len(blocks), "query_rows": tq, "block_sizes": blocks}


def other_workloads(fb, args, keep=None):
    """The workloads beside the headline one; `keep` (a dict) receives their host problems,
    which the CPU baseline times the oracle on."""
    import torch
    import synth
    from synth.device import to_device, tensor
    out = {}
    keep = {} if keep is None else keep
    steps = max(5, args.steps // 5)
    # ragged GQA: per-sequence threshold mask from the drawn M
    p = synth.ragged()
    keep["ragged"] = p
    dev = to_device(p)
    shape, bufs = setup_step(fb, p, dev, varlen=True)
    fresh = torch.full((p.batch,), 1 << 30, dtype=torch.int32, device="cuda")
    w_f, a_f, _ = time_steps(lambda tr: run_step(fb, shape, dev, bufs, fresh, trace=tr), steps, 3)
    m = torch.from_numpy(p.extra["m_updated"]).cuda()
    w_m, _, _ = time_steps(lambda tr: run_step(fb, shape, dev, bufs, m, trace=tr), steps, 3)
    kv = int(p.seqlens.sum()) * p.h_kv * p.d * 4
    fresh_frac = float((p.extra["m_updated"] >= 4).mean())
    # The event pair around the attention launch is recorded in a second pass and also spans
    # the launch gap; a kernel time above the step's own wall time is not credible, so the
    # kernel fraction uses the smaller of the two (rocprofv3 durations are in profiles/).
    a_k = min(a_f, w_f)
    out["ragged_gqa"] = {"fresh_step_us": w_f * 1e6, "attn_kernel_us_events": a_f * 1e6, "attn_kernel_us": a_k * 1e6,
                         "kv_GBps": kv / w_f / 1e9, "frac_hbm_step": kv / w_f / 1e9 / HBM_PEAK_GBS,
                         "frac_hbm": kv / a_k / 1e9 / HBM_PEAK_GBS, "masked_step_us": w_m * 1e6,
                         "fresh_sequences": fresh_frac, "total_prefix_tokens": int(p.seqlens.sum())}
    del dev, bufs
    # video block: per-head similarity mask, 7 of 12 heads reuse
    p = synth.video()
    keep["video"] = p
    dev = to_device(p)
    shape, bufs = setup_step(fb, p, dev)
    sim = torch.from_numpy(p.extra["sim"]).cuda()
    w_all, a_all, _ = time_steps(lambda tr: run_step(fb, shape, dev, bufs, None, trace=tr), steps, 2)
    w_m, a_m, _ = time_steps(lambda tr: run_step(fb, shape, dev, bufs, None, sim=sim, trace=tr), steps, 2)
    nq, nb, npre, d = p.B, p.B, int(p.seqlens[0]), p.d
    flop_block = 4.0 * nq * nb * d * p.h_q
    flop_pre = 4.0 * nq * npre * d
    n_fresh = int((p.extra["sim"] <= np.float32(p.extra["gamma"])).sum())
    f_masked = flop_block + n_fresh * flop_pre
    f_all = flop_block + p.h_q * flop_pre
    a_all, a_m = min(a_all, w_all), min(a_m, w_m)   # event pairs include the launch gap; see ragged_gqa
    out["video_block"] = {"masked_step_us": w_m * 1e6, "masked_TFLOPs": f_masked / w_m / 1e12,
                          "masked_frac_mfma": f_masked / w_m / 1e12 / MFMA_BF16_PEAK_TFLOPS,
                          "masked_attn_kernel_us": a_m * 1e6,
                          "masked_attn_kernel_frac_mfma": f_masked / a_m / 1e12 / MFMA_BF16_PEAK_TFLOPS,
                          "all_fresh_step_us": w_all * 1e6, "all_fresh_TFLOPs": f_all / w_all / 1e12,
                          "attn_kernel_all_fresh_us": a_all * 1e6,
                          "attn_kernel_all_fresh_frac_mfma": f_all / a_all / 1e12 / MFMA_BF16_PEAK_TFLOPS,
                          "fresh_heads": n_fresh, "tokens_per_s": nq / w_m}
    out["video_block"]["torch_sdpa_flash_all_fresh"] = sdpa_reference(dev, p, f_all)
    del dev, bufs
    # LoSA sparse step
    p, dev, shape, bufs, ls, sparse, sel, cap = losa_setup(fb)
    keep["losa"] = p
    fresh = torch.full((1,), 1 << 30, dtype=torch.int32, device="cuda")
    w_d, _, _ = time_steps(lambda tr: run_step(fb, shape, dev, bufs, fresh, trace=tr), steps, 2)
    # a short step (about 0.1 ms): the full step count and more warm-up, as for the dLLM steps
    w_s, a_s, _ = time_steps(sparse, args.steps, 5)
    cnt = sel["count"].cpu().numpy()
    union_bytes = float(cnt.sum()) * 16 * p.d * 2 * 2
    meta_bytes = 2 * fb.losa_meta_bytes(ls)
    out["losa_sparse"] = {"sparse_step_us": w_s * 1e6, "attn_kernel_us": a_s * 1e6, "dense_step_us": w_d * 1e6,
                          "union_pages_mean": float(cnt.mean()), "density": float(cnt.mean()) / ls.max_pages,
                          "alg_bytes": meta_bytes + union_bytes,
                          "frac_hbm_step": (meta_bytes + union_bytes) / w_s / 1e9 / HBM_PEAK_GBS}
    out["sparse_residual"] = residual_workload(fb, p, dev, shape, sel, cap, steps, args.steps)
    del dev, bufs, sparse   # the step's closure holds the page metadata
    out["multi_branch_varlen"] = varlen_workload(fb, args)
    return out


def losa_setup(fb):
    """The LoSA workload (131072-token prefix, 32 heads, B 64, pages of 16, |A| 8, top-64):
    device inputs, page metadata, selection buffers, and the sparse step as a callable."""
    import torch
    import synth
    from synth.device import to_device, tensor
    p = synth.losa()
    dev = to_device(p)
    shape, bufs = setup_step(fb, p, dev)
    ls = fb.make_losa_shape(shape, page_size=16, topk=64, n_active=8)
    kmin = torch.empty(fb.losa_meta_bytes(ls) // 2, dtype=torch.bfloat16, device="cuda")
    kmax = torch.empty_like(kmin)
    fb.losa_page_meta(ls, dev["k"], kmin, kmax)
    qc, qp = tensor(p.extra["q_cur"]), tensor(p.extra["q_prev"])
    cap = fb.losa_union_capacity(ls)
    sel = dict(active=torch.empty((1, 8), dtype=torch.int32, device="cuda"),
               topk=torch.empty((1, 32, 8, 64), dtype=torch.int32, device="cuda"),
               union=torch.empty((1, 32, cap), dtype=torch.int32, device="cuda"),
               count=torch.empty((1, 32), dtype=torch.int32, device="cuda"),
               ws=torch.empty(fb.losa_workspace_size(ls), dtype=torch.uint8, device="cuda"))

    def sparse(tr):
        fb.losa_step(ls, qc, qp, dev["k"], dev["v"], dev["k_blk"], dev["v_blk"], kmin, kmax, bufs["ca"], bufs["cl"],
                     bufs["af"], bufs["lf"], sel["active"], sel["topk"], sel["union"], sel["count"], sel["ws"],
                     trace=tr)
    return p, dev, shape, bufs, ls, sparse, sel, cap


def only_others(fb, args):
    """Profiling mode: the ragged-GQA fresh step and the LoSA sparse step, `steps` times each
    after `warmup`, for counter runs on the kernels other than the dLLM step's."""
    import torch
    import synth
    from synth.device import to_device
    p = synth.ragged()
    dev = to_device(p)
    shape, bufs = setup_step(fb, p, dev, varlen=True)
    fresh = torch.full((p.batch,), 1 << 30, dtype=torch.int32, device="cuda")
    w_r = wall_time(lambda tr: run_step(fb, shape, dev, bufs, fresh), args.steps, args.warmup)
    del dev, bufs
    _, _, _, _, _, sparse, sel, _ = losa_setup(fb)
    w_s = wall_time(sparse, args.steps, args.warmup)
    return {"ragged_fresh_step_us": w_r * 1e6, "losa_sparse_step_us": w_s * 1e6,
            "union_pages": int(sel["count"].sum().item())}


def only_video(fb, args, which):
    """Profiling mode: `steps` video-block steps after `warmup`, either masked (the per-head
    similarity rule with the drawn similarities: 7 of 12 heads reuse) or all fresh."""
    import torch
    import synth
    from synth.device import to_device
    p = synth.video()
    dev = to_device(p)
    shape, bufs = setup_step(fb, p, dev)
    sim = torch.from_numpy(p.extra["sim"]).cuda() if which == "masked" else None
    w = wall_time(lambda tr: run_step(fb, shape, dev, bufs, None, sim=sim), args.steps, args.warmup)
    return {"which": which, "step_us": w * 1e6}


def video_splits(fb, args, counts=(0, 2, 5, 8, 16)):
    """The video-block masked step (7 of 12 heads reuse) and all-fresh step with the prefix
    pass forced to `counts` splits per head through fb_shape.num_splits (0 = the split plan's
    own choice), `steps` timed steps each after `warmup`: wall time per step and the event
    time of the attention kernel (the smaller of the two, as in other_workloads)."""
    import torch
    import synth
    from synth.device import to_device
    p = synth.video()
    dev = to_device(p)
    sim = torch.from_numpy(p.extra["sim"]).cuda()
    # untimed warm-up on the plan's own split count, so that the first row does not carry
    # the clock ramp of a cold GPU
    shape = fb.make_shape(p.batch, p.h_q, p.h_kv, p.d, p.B, seqlen_k=int(p.seqlens[0]))
    _, bufs = setup_step(fb, p, dev)
    wall_time(lambda tr: run_step(fb, shape, dev, bufs, None, sim=sim), 30, 5)
    del bufs
    rows = []
    for ns in counts:
        shape = fb.make_shape(p.batch, p.h_q, p.h_kv, p.d, p.B, seqlen_k=int(p.seqlens[0]), num_splits=ns)
        _, bufs = setup_step(fb, p, dev)
        bufs["ws"] = torch.empty(fb.workspace_size(shape), dtype=torch.uint8, device="cuda")
        w_m, a_m, _ = time_steps(lambda tr: run_step(fb, shape, dev, bufs, None, sim=sim, trace=tr), args.steps,
                                 args.warmup)
        bufs["mask"].zero_()
        w_f, a_f, _ = time_steps(lambda tr: run_step(fb, shape, dev, bufs, None, trace=tr), args.steps, args.warmup)
        rows.append({"num_splits": ns, "masked_step_us": w_m * 1e6, "masked_attn_us": min(a_m, w_m) * 1e6,
                     "fresh_step_us": w_f * 1e6, "fresh_attn_us": min(a_f, w_f) * 1e6,
                     "workspace_bytes": fb.workspace_size(shape)})
        del bufs
    return rows


def residual_workload(fb, p, dev, shape, sel, cap, steps, short_steps):
    """FlashBlock with a cached sparse residual on the LoSA workload's shape: the selection
    is the union the LoSA selection just produced (per KV head, about 500 of 8192 pages).
    A refresh step attends to the selection and to its complement (the whole prefix) and
    caches the residual; a reuse step reads the selected pages only."""
    import torch
    rs = fb.make_residual_shape(shape, page_size=16, max_sel=cap)
    b, B, h, d = p.q.shape
    bufs = dict(ws=torch.empty(fb.residual_workspace_size(rs), dtype=torch.uint8, device="cuda"),
                ca=torch.zeros((b, B, h, d), device="cuda"), cl=torch.zeros((b, B, h), device="cuda"),
                af=torch.zeros((b, B, h, d), dtype=torch.bfloat16, device="cuda"),
                lf=torch.zeros((b, B, h), device="cuda"))
    ones = torch.ones((b, h), dtype=torch.uint8, device="cuda")

    def step(mask):
        return lambda tr: fb.residual_step(rs, dev["q"], dev["k"], dev["v"], dev["k_blk"], dev["v_blk"], sel["union"],
                                           sel["count"], mask, bufs["ca"], bufs["cl"], bufs["af"], bufs["lf"],
                                           bufs["ws"], trace=tr)
    w_f, a_f, _ = time_steps(step(None), steps, 2)
    w_r, a_r, _ = time_steps(step(ones), short_steps, 5)   # a short step: more calls, more warm-up
    g_f = graph_step_time(step(None), steps)
    g_r = graph_step_time(step(ones), short_steps)
    cnt = sel["count"].cpu().numpy()
    sel_bytes = float(np.minimum(cnt * 16, p.seqlens[0]).sum()) * d * 2 * 2
    all_bytes = float(p.seqlens[0]) * p.h_kv * d * 2 * 2
    return {"refresh_step_us": w_f * 1e6, "refresh_attn_us": a_f * 1e6, "refresh_kv_GBps": all_bytes / w_f / 1e9,
            "refresh_attn_frac_hbm": all_bytes / a_f / 1e9 / HBM_PEAK_GBS,
            "reuse_step_us": w_r * 1e6, "reuse_attn_us": a_r * 1e6, "reuse_kv_GBps": sel_bytes / w_r / 1e9,
            "reuse_attn_frac_hbm": sel_bytes / a_r / 1e9 / HBM_PEAK_GBS,
            "refresh_step_graph_us": g_f * 1e6, "reuse_step_graph_us": g_r * 1e6,
            "selected_pages_mean": float(cnt.mean()), "selected_kv_bytes": sel_bytes, "prefix_kv_bytes": all_bytes}


if __name__ == "__main__":
    main()
