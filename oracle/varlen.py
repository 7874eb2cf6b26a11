"""Prefix pass over several branches packed into one variable-length query buffer.

TEST INFRASTRUCTURE (oracle): plain fp64 CPU code; see oracle/attention.py for the import
rule and the source key.

Source: [BB] "Resumen Técnico: BlockBatch", "Optimización del Sistema": the query
positions of all active branches (each with its own block size and its own KV cache) are
packed into one variable-length buffer and processed in one pass; [FB-pt] §2 "Mecanismo
Central" for what the block-external pass of one branch computes.

Readings: branch b owns queries cu_q[b] .. cu_q[b+1]-1 of the packed buffer and prefix
tokens cu_k[b] .. cu_k[b+1]-1; its queries attend to its own prefix only.
"""
from __future__ import annotations

import numpy as np

from .attention import attend, _kv_head


def prefix_attention_varlen(q, cu_q, k, v, cu_k, h_kv: int, scale: float):
    """q [sum B_b, H_q, d] by cu_q; k, v [sum N_b, H_kv, d] by cu_k ->
    A [sum B_b, H_q, d], L [sum B_b, H_q]."""
    tq, h_q, d = q.shape
    a = np.zeros((tq, h_q, d))
    l = np.full((tq, h_q), -np.inf)
    for b in range(len(cu_q) - 1):
        q0, q1 = int(cu_q[b]), int(cu_q[b + 1])
        k0, k1 = int(cu_k[b]), int(cu_k[b + 1])
        if q1 == q0:
            continue
        for h in range(h_q):
            g = _kv_head(h, h_q, h_kv)
            a[q0:q1, h], l[q0:q1, h] = attend(q[q0:q1, h], k[k0:k1, g], v[k0:k1, g], scale)
    return a, l
