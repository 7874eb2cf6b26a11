"""Seeded synthetic inputs shared by the oracle-side tests, the GPU tests and the bench.

This module only draws and rounds random numbers; it holds none of the attention,
merge, reuse or selection arithmetic.  Every tensor is drawn with
``numpy.random.Generator(PCG64(seed))`` in a fixed order (Q, K, V, K_blk, V_blk,
then per-step draws) and rounded to bfloat16 (round-to-nearest-even) on the host,
so the oracle and the GPU path see exactly the same values.

Layouts (shared by every consumer):
  q        [batch, B, H_q, d]        block queries
  k, v     [sum_b N_b, H_kv, d]      packed variable-length prefix (growing KV cache)
  cu       [batch + 1] int32         prefix offsets into k/v
  k_blk    [batch, B, H_kv, d]       current block keys/values
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

SEED_TINY, SEED_DLLM, SEED_RAGGED, SEED_VIDEO, SEED_LOSA, SEED_RESIDUAL = 0, 1, 2, 3, 4, 5


def rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def round_bf16(x) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even); returns float32."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty_like(x)
    flat_in, flat_out = x.reshape(-1), out.reshape(-1)
    step = 1 << 24
    for s in range(0, flat_in.size, step):
        u = flat_in[s:s + step].view(np.uint32).astype(np.uint64)
        u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
        flat_out[s:s + step] = u.astype(np.uint32).view(np.float32)
    return out


def bf16_bits(x) -> np.ndarray:
    """uint16 bit patterns of values that are already bfloat16-representable."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    return (x.view(np.uint32) >> 16).astype(np.uint16)


def normal(g: np.random.Generator, shape, std: float = 1.0, bf16: bool = True) -> np.ndarray:
    x = g.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    return round_bf16(x) if bf16 else x


@dataclass
class Problem:
    """One seeded workload instance: shapes plus the drawn tensors (float32 arrays whose
    values are exactly representable in ``dtype``)."""
    name: str
    batch: int
    h_q: int
    h_kv: int
    d: int
    B: int
    seqlens: np.ndarray            # [batch] prefix lengths N_b
    dtype: str                     # "bf16" or "f32"
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    k_blk: np.ndarray
    v_blk: np.ndarray
    extra: dict = field(default_factory=dict)

    @property
    def cu(self) -> np.ndarray:
        return np.concatenate([[0], np.cumsum(self.seqlens)]).astype(np.int32)

    @property
    def scale(self) -> float:
        return 1.0 / float(np.sqrt(self.d))


def make_problem(name, seed, batch, h_q, h_kv, d, B, seqlens, dtype="bf16", std=1.0) -> Problem:
    """Draw Q, K, V, K_blk, V_blk in that order, N(0, std^2) each."""
    g = rng(seed)
    bf = dtype == "bf16"
    seqlens = np.asarray(seqlens, dtype=np.int64)
    total = int(seqlens.sum())
    q = normal(g, (batch, B, h_q, d), std, bf)
    k = normal(g, (total, h_kv, d), std, bf)
    v = normal(g, (total, h_kv, d), std, bf)
    kb = normal(g, (batch, B, h_kv, d), std, bf)
    vb = normal(g, (batch, B, h_kv, d), std, bf)
    p = Problem(name, batch, h_q, h_kv, d, B, seqlens.astype(np.int32), dtype, q, k, v, kb, vb)
    p.extra["gen"] = g
    return p


# ----------------------------------------------------------------------------------
# The five workloads (shapes, value distributions and per-step draws).
# ----------------------------------------------------------------------------------

def tiny(seed: int = SEED_TINY) -> Problem:
    """fp32: batch 1, 2 heads, d 64, B 4, prefix 60; Q/K/V ~ N(0,1).  Step 1 perturbs
    the queries by N(0, 0.01^2)."""
    p = make_problem("tiny_f32", seed, 1, 2, 2, 64, 4, [60], dtype="f32")
    g = p.extra.pop("gen")
    p.extra["q_step1"] = (p.q + 0.01 * g.standard_normal(p.q.shape, dtype=np.float32)).astype(np.float32)
    return p


def dllm(seed: int = SEED_DLLM, n_prefix: int = 32768, steps: int = 8) -> Problem:
    """bf16: batch 1, 32 heads MHA, d 128, B 32, prefix 32768; Q/K/V ~ N(0,1)/sqrt(128).
    Per block: ``steps`` denoising steps; M_s ~ U{0..8} updated tokens for s >= 1."""
    p = make_problem("dllm", seed, 1, 32, 32, 128, 32, [n_prefix], std=1.0 / np.sqrt(128.0))
    g = p.extra.pop("gen")
    m = g.integers(0, 9, size=(steps, p.batch)).astype(np.int32)
    m[0] = 1 << 30        # step 0 of a block has nothing cached: never below a threshold
    p.extra["m_updated"] = m
    p.extra["tau"] = 4
    return p


def ragged(seed: int = SEED_RAGGED, batch: int = 8, lo: int = 8192, hi: int = 65536) -> Problem:
    """bf16: batch 8, GQA 32 query / 8 KV heads, d 128, B 32; prefix lengths ~ U[lo, hi]
    packed variable-length; per-sequence M ~ U{0..8}, tau 4."""
    g0 = rng(seed)
    seqlens = g0.integers(lo, hi + 1, size=batch)
    p = make_problem("ragged", seed + 1000, batch, 32, 8, 128, 32, seqlens, std=1.0 / np.sqrt(128.0))
    g = p.extra.pop("gen")
    p.extra["m_updated"] = g.integers(0, 9, size=batch).astype(np.int32)
    p.extra["tau"] = 4
    return p


def video(seed: int = SEED_VIDEO, block: int = 4680, n_prefix: int = 32760, heads: int = 12) -> Problem:
    """bf16: batch 1, 12 heads, d 128, block 4680 (3 x 1560) queries, prefix 32760.
    Per-head similarity: a seeded permutation gives 7 heads U(0.951, 0.999) and the rest
    U(0.80, 0.949), so 7 of 12 heads reuse at gamma 0.95."""
    p = make_problem("video", seed, 1, heads, heads, 128, block, [n_prefix], std=1.0 / np.sqrt(128.0))
    g = p.extra.pop("gen")
    n_hi = (7 * heads + 11) // 12
    perm = g.permutation(heads)
    sim = np.empty(heads, dtype=np.float32)
    sim[perm[:n_hi]] = g.uniform(0.951, 0.999, size=n_hi).astype(np.float32)
    sim[perm[n_hi:]] = g.uniform(0.80, 0.949, size=heads - n_hi).astype(np.float32)
    p.extra["sim"] = sim.reshape(1, heads)
    p.extra["gamma"] = 0.95
    return p


def losa(seed: int = SEED_LOSA, n_prefix: int = 131072, B: int = 64, heads: int = 32,
         h_kv: int | None = None, n_active: int = 8, page: int = 16, topk: int = 64,
         sigma_active: float = 0.5, sigma_stable: float = 0.01) -> Problem:
    """bf16: batch 1, 32 heads, d 128, B 64, prefix 131072, page 16, |A| 8, top-64.
    Step t queries: ``n_active`` seeded tokens get Q += N(0, 0.5^2), the rest N(0, 0.01^2)."""
    h_kv = heads if h_kv is None else h_kv
    p = make_problem("losa", seed, 1, heads, h_kv, 128, B, [n_prefix], std=1.0 / np.sqrt(128.0))
    g = p.extra.pop("gen")
    moved = np.sort(g.permutation(B)[:n_active]).astype(np.int32)
    sig = np.full((p.batch, B, 1, 1), sigma_stable, dtype=np.float32)
    sig[:, moved] = sigma_active
    noise = g.standard_normal(size=p.q.shape, dtype=np.float32) * sig
    p.extra["q_prev"] = p.q
    p.extra["q_cur"] = round_bf16(p.q + noise)
    p.extra["moved"] = moved
    p.extra.update(n_active=n_active, page=page, topk=topk)
    return p


def custom(seed, batch, h_q, h_kv, d, B, seqlens, dtype="bf16", std=1.0) -> Problem:
    """Any shape, for parity sweeps: same draw order as the named workloads."""
    p = make_problem("custom", seed, batch, h_q, h_kv, d, B, seqlens, dtype=dtype, std=std)
    p.extra.pop("gen")
    return p


def page_selection(seed, seqlens, h_kv, page, n_sel, kinds=("random",)) -> list:
    """Per (sequence, KV head) a set of distinct prefix pages (page = ``page`` consecutive
    tokens), ascending.  Group j of the flattened (sequence, KV head) order takes kind
    ``kinds[j % len(kinds)]``: "empty"; "all" (every page); "random" (min(n_sel, pages)
    pages drawn without replacement); "tail" (as random, with the partial last page in)."""
    g = rng(seed)
    out, j = [], 0
    for n in np.asarray(seqlens, dtype=np.int64):
        P = int(-(-int(n) // page))
        row = []
        for _ in range(h_kv):
            kind = kinds[j % len(kinds)]
            j += 1
            if kind == "empty" or P == 0:
                row.append(np.zeros(0, np.int64))
            elif kind == "all":
                row.append(np.arange(P, dtype=np.int64))
            else:
                s = g.permutation(P)[:min(n_sel, P)]
                if kind == "tail" and P - 1 not in s:
                    s[-1] = P - 1
                row.append(np.sort(s).astype(np.int64))
        out.append(row)
    return out


def pack_selection(sel, max_sel, shuffle_seed=None):
    """[batch][h_kv][max_sel] int32 page lists padded with -1, and [batch][h_kv] counts.
    With ``shuffle_seed`` each list is permuted (the selection is a set; order is free)."""
    b, hk = len(sel), len(sel[0])
    pages = np.full((b, hk, max_sel), -1, dtype=np.int32)
    count = np.zeros((b, hk), dtype=np.int32)
    g = None if shuffle_seed is None else rng(shuffle_seed)
    for i in range(b):
        for h in range(hk):
            s = np.asarray(sel[i][h], dtype=np.int32)
            if g is not None:
                s = g.permutation(s)
            pages[i, h, :len(s)] = s
            count[i, h] = len(s)
    return pages, count


def branches(seed, blocks, seqlens, h_q, h_kv, d, dtype="bf16", std=1.0) -> dict:
    """Several branches of one request (the multi-branch pass): branch b has a block of
    blocks[b] query positions and its own prefix of seqlens[b] tokens.  Draw order: Q
    (packed [sum B_b, H_q, d]), K, V (packed [sum N_b, H_kv, d])."""
    g = rng(seed)
    bf = dtype == "bf16"
    blocks = np.asarray(blocks, dtype=np.int64)
    seqlens = np.asarray(seqlens, dtype=np.int64)
    q = normal(g, (int(blocks.sum()), h_q, d), std, bf)
    k = normal(g, (int(seqlens.sum()), h_kv, d), std, bf)
    v = normal(g, (int(seqlens.sum()), h_kv, d), std, bf)
    return dict(q=q, k=k, v=v, cu_q=np.concatenate([[0], np.cumsum(blocks)]).astype(np.int32),
                cu_k=np.concatenate([[0], np.cumsum(seqlens)]).astype(np.int32), blocks=blocks, seqlens=seqlens,
                h_q=h_q, h_kv=h_kv, d=d, dtype=dtype, scale=1.0 / float(np.sqrt(d)))
