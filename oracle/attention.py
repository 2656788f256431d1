"""CPU oracle of the sparse-attention consumer (TEST INFRASTRUCTURE ONLY:
imported by ``tests/`` and ``bench.py``'s CPU-baseline leg, never by the GPU
library or its binding).

What it computes, from the pages "spec(MODEL-MM-QWEN4-EXP) ...": the model's
attention is plain GQA, 24 query heads over 2 KV heads with head_dim 256 (the
op-survey paragraph on QSA's twin), and its consumer attends to the raw tokens
the indexer selected at ratio-4 granularity (section "The component
deep-dives, and two corrections to the above").  Readings taken where the
pages are silent: softmax attention with scale 1/sqrt(head_dim) over exactly
the listed tokens (entries < 0 are padding; a row with none attends to nothing
and yields zeros); query head h reads KV head h // (q_heads / kv_heads); the
main KV cache is paged like the index cache, token t of a request at slot
t % page_size of page page_table[req][t // page_size], with K and V laid out
[page][slot][kv_head][head_dim].

Plain float64 arithmetic, one row and one head at a time; a matrix-vector
product and exp are the only library steps.
"""
from __future__ import annotations

import numpy as np


def sparse_attention(q, k_cache, v_cache, page_table, tokens, scale=None, row_req=None):
    """out[r, h, :] = sum_t softmax_t(scale * q[r,h].K[t]) V[t] over the
    tokens t listed in tokens[r] (entries < 0 skipped); float64 [rows, q_heads, d]."""
    rows, q_heads, d = q.shape
    page_size, kv_heads = k_cache.shape[1], k_cache.shape[2]
    assert q_heads % kv_heads == 0
    group = q_heads // kv_heads
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    out = np.zeros((rows, q_heads, d), dtype=np.float64)
    for r in range(rows):
        req = 0 if row_req is None else int(row_req[r])
        sel = np.asarray(tokens[r], dtype=np.int64)
        sel = sel[sel >= 0]
        if sel.size == 0:
            continue
        pages = page_table[req][sel // page_size]
        slots = sel % page_size
        K = k_cache[pages, slots].astype(np.float64)  # [n, kv_heads, d]
        V = v_cache[pages, slots].astype(np.float64)
        for h in range(q_heads):
            g = h // group
            s = (K[:, g, :] @ q[r, h].astype(np.float64)) * scale
            w = np.exp(s - s.max())
            w /= w.sum()
            out[r, h] = w @ V[:, g, :]
    return out
