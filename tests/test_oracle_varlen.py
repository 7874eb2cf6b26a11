"""Pins for oracle/varlen.py (branches of different block sizes in one packed buffer)."""
import numpy as np

import synth
from oracle import attention as A
from oracle.varlen import prefix_attention_varlen


def _branches(seed, blocks, lens, hq=4, hkv=2, d=16):
    g = synth.rng(seed)
    q = g.standard_normal((sum(blocks), hq, d)).astype(np.float32)
    k = g.standard_normal((sum(lens), hkv, d)).astype(np.float32)
    v = g.standard_normal((sum(lens), hkv, d)).astype(np.float32)
    cu_q = np.concatenate([[0], np.cumsum(blocks)]).astype(np.int32)
    cu_k = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    return q, k, v, cu_q, cu_k


def test_equal_blocks_reduce_to_the_batched_prefix_pass():
    p = synth.custom(0, 3, 4, 2, 16, 5, [20, 7, 13], dtype="f32")
    q = p.q.reshape(-1, p.h_q, p.d)
    cu_q = np.arange(0, 3 * 5 + 1, 5, dtype=np.int32)
    a, l = prefix_attention_varlen(q, cu_q, p.k, p.v, p.cu, p.h_kv, p.scale)
    e, el = A.prefix_attention(p.q, p.k, p.v, p.cu, p.h_kv, p.scale)
    assert np.max(np.abs(a - e.reshape(a.shape))) <= 1e-14 and np.max(np.abs(l - el.reshape(l.shape))) <= 1e-14


def test_branches_are_independent_and_brute_force():
    blocks, lens = [4, 1, 0, 7], [9, 3, 5, 0]
    q, k, v, cu_q, cu_k = _branches(1, blocks, lens)
    a, l = prefix_attention_varlen(q, cu_q, k, v, cu_k, 2, 0.25)
    for b in range(4):
        for t in range(cu_q[b], cu_q[b + 1]):
            for h in range(4):
                g = h // 2
                ks, vs = k[cu_k[b]:cu_k[b + 1], g].astype(np.float64), v[cu_k[b]:cu_k[b + 1], g].astype(np.float64)
                if len(ks) == 0:
                    assert (a[t, h] == 0).all() and np.isneginf(l[t, h])
                    continue
                s = 0.25 * ks @ q[t, h].astype(np.float64)
                w = np.exp(s)                                 # small scores: no shift needed
                assert np.max(np.abs(a[t, h] - (w @ vs) / w.sum())) <= 1e-12
                assert abs(l[t, h] - np.log(w.sum())) <= 1e-12
    # reversing the branch order permutes the outputs and nothing else
    order = [3, 2, 1, 0]
    q2 = np.concatenate([q[cu_q[b]:cu_q[b + 1]] for b in order])
    k2 = np.concatenate([k[cu_k[b]:cu_k[b + 1]] for b in order])
    v2 = np.concatenate([v[cu_k[b]:cu_k[b + 1]] for b in order])
    cq2 = np.concatenate([[0], np.cumsum([blocks[b] for b in order])]).astype(np.int32)
    ck2 = np.concatenate([[0], np.cumsum([lens[b] for b in order])]).astype(np.int32)
    a2, _ = prefix_attention_varlen(q2, cq2, k2, v2, ck2, 2, 0.25)
    back = np.concatenate([a2[cq2[i]:cq2[i + 1]] for i in (3, 2, 1, 0)])
    assert np.array_equal(back, a)
