"""CPU oracle of the compressed-key producer (TEST INFRASTRUCTURE ONLY:
imported by ``tests/`` and ``bench.py``'s CPU-baseline leg, never by the GPU
library or its binding).

What it computes, from the page "spec(MODEL-MM-QWEN4-EXP) ...", section "The
component deep-dives, and two corrections to the above": the indexer's side
cache stores one state per compress_ratio (4) tokens; a block is complete at
the token whose (position + 1) is a multiple of the ratio; the stored key is
a pooled key with RMSNorm applied to it and RoPE applied at the block-start
position.  The same section says the DeepSeek-V4 kernel's learned softmax pool
over eight tokens does not carry over, and the pages give no other pooling.

Readings taken where the pages are silent (each is a parameter here, so a
caller can pick another value):
  * pooling is the arithmetic mean of the block's ratio token keys;
  * RMSNorm is y_i = w_i * x_i / sqrt(mean_j x_j^2 + eps) over the key's 128
    values, with caller-given weights w and eps;
  * RoPE rotates the leading ``rope_dim`` values by angles p0 * base^(-2i/rope_dim),
    p0 = ratio * c for block c, pairing value i with i + rope_dim/2
    ("rotate-half") or value 2i with 2i+1 ("interleaved"); the pair (a, b)
    becomes (a cos - b sin, b cos + a sin);
  * compressed key c of request q lands in slot c % (page_size/ratio) of
    physical page page_table[q][c // (page_size/ratio)], the layout the scorer
    reads.

"Parity unpinned" as far as the pages go: they fix none of the readings above,
so the pins in tests/test_producer_oracle.py tie this code to the mathematics
of the readings (closed forms, invariances), not to values printed on a page.

Plain float64 arithmetic, one block at a time.
"""
from __future__ import annotations

import numpy as np


def mean_pool(keys):
    """Arithmetic mean over the block's token keys: [ratio, d] -> [d] float64."""
    keys = np.asarray(keys, dtype=np.float64)
    return keys.sum(axis=0) / keys.shape[0]


def rms_norm(x, w=None, eps=1e-6):
    """x / sqrt(mean(x^2) + eps), times the per-value weight w (1 if None)."""
    x = np.asarray(x, dtype=np.float64)
    y = x / np.sqrt(np.mean(x * x) + eps)
    if w is not None:
        y = y * np.asarray(w, dtype=np.float64)
    return y


def rope(x, p0, rope_dim=128, base=10000.0, interleaved=False):
    """Rotate the leading rope_dim values of x at position p0 (float64 copy)."""
    x = np.array(x, dtype=np.float64)
    half = rope_dim // 2
    for i in range(half):
        theta = float(p0) * float(base) ** (-2.0 * i / rope_dim)
        c, s = np.cos(theta), np.sin(theta)
        ia, ib = (2 * i, 2 * i + 1) if interleaved else (i, i + half)
        a, b = x[ia], x[ib]
        x[ia] = a * c - b * s
        x[ib] = b * c + a * s
    return x


def compress_block(keys, block, ratio=4, w=None, eps=1e-6, rope_dim=128, base=10000.0, interleaved=False):
    """Compressed key of block `block` from its `ratio` token keys, in token order."""
    keys = np.asarray(keys)
    assert keys.shape[0] == ratio
    return rope(rms_norm(mean_pool(keys), w, eps), ratio * block, rope_dim, base, interleaved)


def produce(history, page_table, page_size, ratio=4, w=None, eps=1e-6, rope_dim=128, base=10000.0,
            interleaved=False):
    """Every compressed key the producer has stored after seeing, for each
    request q, the raw token keys history[q] ([n_q, d], positions 0..n_q-1).

    Returns {(physical page, slot): float64 [d]} for each complete block
    (n_q // ratio blocks per request); incomplete blocks store nothing."""
    kpp = page_size // ratio
    stored = {}
    for q, keys in enumerate(history):
        keys = np.asarray(keys)
        for c in range(keys.shape[0] // ratio):
            page = int(page_table[q][c // kpp])
            stored[(page, c % kpp)] = compress_block(keys[ratio * c: ratio * (c + 1)], c, ratio, w, eps,
                                                     rope_dim, base, interleaved)
    return stored
