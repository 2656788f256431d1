"""Seeded synthetic inputs for the paged block-scoring indexer.

This module serves both the oracle and the GPU path (tests and bench) and holds
none of the method's arithmetic: it draws query vectors, a paged key cache, a
page table and per-row positions, and nothing else.  It never computes a score,
a visibility count or a selection.

Recipe (fixed draw order, NumPy PCG64 ``default_rng(seed)``):
  1. request contexts and per-request row counts,
  2. the page permutation (for permuted page pools),
  3. ``q``,
  4. ``kcache``, filled page by physical page,
  5. the outlier mask (decode workload).
fp16 values are ``standard_normal(float32)`` rounded to nearest-even fp16;
integer twins draw from ``integers(-2, 3)`` (values -2..2, exact in fp16).

The shapes follow the pages' kernel benchmark ("[Perf][Qwen4Exp] Admit the
cuBLAS QSA indexer and exact top-k on Turing", section "Test Plan": the last
1,616-row prefill chunk, 4 index heads, head dim 128, compress ratio 4, top-k
2,048) and the paged side cache of one key per 4 tokens in 64-token pages.
No public dataset is involved; these synthetic draws stand in for the
RMSNorm-ed, RoPE-d pooled keys of a real model, which would need trained
weights.
"""
from __future__ import annotations

import dataclasses
import hashlib

import numpy as np

HEADS = 4
HEAD_DIM = 128
COMPRESS_RATIO = 4
PAGE_SIZE = 64


@dataclasses.dataclass
class Workload:
    name: str
    q: np.ndarray            # float16 [rows, heads, head_dim]
    kcache: np.ndarray       # float16 [num_pages, page_size // cr, head_dim]
    page_table: np.ndarray   # int32   [num_reqs, pt_stride]
    row_req: np.ndarray      # int32   [rows]
    pos: np.ndarray          # int32   [rows]  absolute token position of each row
    ctx: np.ndarray          # int64   [num_reqs] tokens in each request's context
    compress_ratio: int
    page_size: int
    k: int
    seed: int

    @property
    def rows(self) -> int:
        return int(self.q.shape[0])

    @property
    def num_reqs(self) -> int:
        return int(self.page_table.shape[0])

    @property
    def num_pages(self) -> int:
        return int(self.kcache.shape[0])

    def digest(self) -> str:
        h = hashlib.sha256()
        for a in (self.q, self.kcache, self.page_table, self.row_req, self.pos):
            h.update(np.ascontiguousarray(a).tobytes())
        return h.hexdigest()


def _normal_f16(rng, shape, chunk_rows=None):
    """standard_normal(float32) rounded to fp16, drawn in a fixed chunking so
    that multi-GB caches never hold a full float32 copy."""
    shape = tuple(int(s) for s in shape)
    out = np.empty(shape, dtype=np.float16)
    if chunk_rows is None or shape[0] <= chunk_rows:
        out[...] = rng.standard_normal(shape, dtype=np.float32)
        return out
    for a in range(0, shape[0], chunk_rows):
        b = min(shape[0], a + chunk_rows)
        out[a:b] = rng.standard_normal((b - a,) + shape[1:], dtype=np.float32)
    return out


def _int_f16(rng, shape, chunk_rows=None):
    shape = tuple(int(s) for s in shape)
    out = np.empty(shape, dtype=np.float16)
    if chunk_rows is None or shape[0] <= chunk_rows:
        out[...] = rng.integers(-2, 3, size=shape, dtype=np.int8)
        return out
    for a in range(0, shape[0], chunk_rows):
        b = min(shape[0], a + chunk_rows)
        out[a:b] = rng.integers(-2, 3, size=(b - a,) + shape[1:], dtype=np.int8)
    return out


def build(name, rng, seed, ctxs, rows_per_req, *, permute_pages, integer=False,
          outlier_p=0.0, k=2048, compress_ratio=COMPRESS_RATIO, page_size=PAGE_SIZE,
          heads=HEADS, head_dim=HEAD_DIM, extra_pages=0):
    """Assemble a workload from per-request contexts and row counts.

    Request i owns ceil(ctx_i / page_size) pages; its rows are its last
    rows_i positions, ctx_i - rows_i .. ctx_i - 1 (a prefill chunk that ends
    the context; a decode row is the single last position).  Pages come from
    one pool, either contiguous per request or a seeded permutation of the
    pool.  ``extra_pages`` adds unreferenced pages to the pool.
    """
    ctxs = np.asarray(ctxs, dtype=np.int64)
    rows_per_req = np.asarray(rows_per_req, dtype=np.int64)
    assert ctxs.shape == rows_per_req.shape
    assert np.all(rows_per_req >= 0) and np.all(rows_per_req <= ctxs)
    keys_per_page = page_size // compress_ratio
    npages_req = (ctxs + page_size - 1) // page_size
    pool = int(npages_req.sum()) + int(extra_pages)
    # 2. page permutation
    phys = rng.permutation(pool).astype(np.int32) if permute_pages else np.arange(pool, dtype=np.int32)
    pt_stride = int(max(1, npages_req.max(initial=1)))
    page_table = np.zeros((len(ctxs), pt_stride), dtype=np.int32)
    off = 0
    for i, n in enumerate(npages_req):
        page_table[i, :n] = phys[off:off + n]
        off += int(n)
    row_req = np.repeat(np.arange(len(ctxs), dtype=np.int32), rows_per_req)
    pos = np.concatenate([np.arange(c - r, c, dtype=np.int64) for c, r in zip(ctxs, rows_per_req)]
                         + [np.zeros(0, np.int64)]).astype(np.int32)
    rows = int(rows_per_req.sum())
    draw = _int_f16 if integer else _normal_f16
    # 3. q
    q = draw(rng, (rows, heads, head_dim), chunk_rows=4096)
    # 4. kcache, page by physical page
    kcache = draw(rng, (pool, keys_per_page, head_dim), chunk_rows=8192)
    # 5. outliers: whole key vectors scaled by 8 (exact in fp16 for these magnitudes)
    if outlier_p > 0:
        mask = rng.random(pool * keys_per_page) < outlier_p
        flat = kcache.reshape(-1, head_dim)
        flat[mask] *= np.float16(8)
    return Workload(name=name, q=q, kcache=kcache, page_table=page_table, row_req=row_req,
                    pos=pos, ctx=ctxs, compress_ratio=compress_ratio, page_size=page_size,
                    k=k, seed=seed)


# ---------------------------------------------------------------------------
# the five measured workloads (and scaled-down variants of each for tests)

def tiny(seed=0, integer=False):
    """64 rows at positions 960..1023 of a 1,024-token request; top-k 64."""
    rng = np.random.default_rng(seed)
    return build("tiny", rng, seed, [1024], [64], permute_pages=False, integer=integer, k=64)


def kernel_shape(seed=1, integer=False, rows=1616, ctx=184_000):
    """The last ``rows``-row prefill chunk of one ``ctx``-token request
    (defaults: 1,616 rows of 184,000 tokens); contiguous pages; top-k 2,048."""
    rng = np.random.default_rng(seed)
    return build("kernel_shape", rng, seed, [ctx], [rows], permute_pages=False,
                 integer=integer, k=2048)


def tie_stress(seed=2, rows=512, ctx=32_768):
    """512 rows over a 32,768-token request, integer q and k in -2..2 so that
    fp32 sums are exact and ties pile up at the cutoff; top-k 2,048."""
    rng = np.random.default_rng(seed)
    return build("tie_stress", rng, seed, [ctx], [rows], permute_pages=False,
                 integer=True, k=2048)


def mixed(seed=3, integer=False, num_reqs=8, total_rows=1500, ctx_lo=4096, ctx_hi=131_072,
          max_rows=512):
    """8 requests, contexts ~ U{4,096..131,072}, prefill chunks of 1..512 rows
    rescaled to ~1,500 rows in total, pages a seeded permutation of one pool."""
    rng = np.random.default_rng(seed)
    ctxs = rng.integers(ctx_lo, ctx_hi + 1, size=num_reqs)
    raw = rng.integers(1, max_rows + 1, size=num_reqs)
    rows = np.clip(np.rint(raw * (total_rows / raw.sum())), 1, max_rows).astype(np.int64)
    rows = np.minimum(rows, ctxs)
    return build("mixed", rng, seed, ctxs, rows, permute_pages=True, integer=integer, k=2048)


def decode(seed=4, integer=False, num_reqs=256, ctx_lo=65_536, ctx_hi=184_000, outlier_p=0.01):
    """256 requests with one row each at its last position, contexts
    ~ U{65,536..184,000}, permuted pages, 1% of key vectors scaled by 8."""
    rng = np.random.default_rng(seed)
    ctxs = rng.integers(ctx_lo, ctx_hi + 1, size=num_reqs)
    rows = np.ones(num_reqs, dtype=np.int64)
    return build("decode", rng, seed, ctxs, rows, permute_pages=True, integer=integer,
                 outlier_p=outlier_p, k=2048)


def long_few(seed=5, integer=False, num_reqs=8, ctx=184_000, outlier_p=0.01):
    """A small batch of long requests: ``num_reqs`` requests of ``ctx``
    tokens with one row each at the last position (the decode row shape),
    permuted pages, 1% of key vectors scaled by 8; top-k 2,048."""
    rng = np.random.default_rng(seed)
    ctxs = np.full(num_reqs, ctx, dtype=np.int64)
    rows = np.ones(num_reqs, dtype=np.int64)
    return build(f"long_{num_reqs}", rng, seed, ctxs, rows, permute_pages=True, integer=integer,
                 outlier_p=outlier_p, k=2048)


def raw_token_keys(seed, lengths, page_size=PAGE_SIZE, compress_ratio=COMPRESS_RATIO, spare_pages=2):
    """Inputs of the compressed-key producer: each request's raw per-token
    index keys (fp16 [n_q, head_dim], standard normal), RMSNorm weights
    (float32 [head_dim], uniform in [0.5, 1.5)) and a page table over a
    permuted pool with room for every request's compressed keys, plus
    ``spare_pages`` pages that no request maps.  Draw order: keys request by
    request, weights, permutation."""
    rng = np.random.default_rng(seed)
    keys = [_normal_f16(rng, (int(n), HEAD_DIM), chunk_rows=1 << 16) for n in lengths]
    w = rng.uniform(0.5, 1.5, HEAD_DIM).astype(np.float32)
    kpp = page_size // compress_ratio
    per = max(1, max((int(n) // compress_ratio + kpp - 1) // kpp for n in lengths) if len(lengths) else 1)
    pool = len(lengths) * per + spare_pages
    pt = rng.permutation(pool)[:len(lengths) * per].astype(np.int32).reshape(len(lengths), per)
    return keys, w, pt, pool


# fp16 integers of large magnitude: multiples of 16 in [2^14, 2^15) and of 32
# in [2^15, 65504] are exact in fp16
_LARGE_INTS = np.array([16384, 20000, 24576, 30000, 32752, 32768, 40000, 49152, 65504], dtype=np.float32)
# head values of rows whose largest head sum sits at an edge: 65504 (the fp16
# maximum), 65520 (just past it), 131008 (twice it) and 131040 (just past
# that), and 4 * 65504 (the largest sum four fp16 values can reach)
_EDGE_HEADS = [(32752, 32752, 0, 0), (32752, 32768, 0, 0), (65504, 65504, 0, 0), (65504, 65504, 32, 0),
               (65504, 65504, 65504, 65504)]


def large_query(w, seed, frac=0.5):
    """A copy of workload ``w`` with large query values planted in a seeded
    subset of its rows, so that the per-dimension sum over the index heads
    leaves fp16's range (up to 4 * 65504).

    Integer workloads (q in -2..2) get integer values exact in fp16: in each
    chosen row, 1 to 3 dimensions where 2 to 4 heads take +-values from
    ``_LARGE_INTS``; rows 0..4 (and, negated, 5..9) carry the edge sums of
    ``_EDGE_HEADS`` in one dimension.  Every per-head dot then stays an
    integer below 2^21, so fp32 sums are exact in any order.  Gaussian
    workloads get whole rows scaled by 2^14 (exact in fp16) and clipped to
    +-65504.  Draw order: chosen rows, then per row its dimensions, heads,
    values and signs."""
    rng = np.random.default_rng(seed)
    q = w.q.copy()
    rows = q.shape[0]
    integer = bool(np.all(np.abs(w.q.astype(np.float32)) <= 2) and np.all(np.rint(w.q) == w.q))
    chosen = np.flatnonzero(rng.random(rows) < frac)
    if integer:
        for r in chosen:
            nd = int(rng.integers(1, 4))
            for d in rng.choice(q.shape[2], size=nd, replace=False):
                nh = int(rng.integers(2, 5))
                heads = rng.choice(q.shape[1], size=nh, replace=False)
                vals = rng.choice(_LARGE_INTS, size=nh) * rng.choice(np.array([-1.0, 1.0], np.float32), size=nh)
                q[r, heads, d] = vals.astype(np.float16)
        for i, hv in enumerate(_EDGE_HEADS):
            for sign, r in ((1.0, i), (-1.0, i + len(_EDGE_HEADS))):
                if r < rows:
                    q[r, :, 7] = (sign * np.array(hv, np.float32)).astype(np.float16)
    else:
        big = q[chosen].astype(np.float32) * np.float32(16384.0)
        q[chosen] = np.clip(big, -65504.0, 65504.0).astype(np.float16)
    return dataclasses.replace(w, name=w.name + "_largeq", q=q)


CONFIGS = {
    "tiny": tiny,
    "kernel_shape": kernel_shape,
    "tie_stress": tie_stress,
    "mixed": mixed,
    "decode": decode,
    # small batches of 184k-token requests (one or eight rows)
    "long_1": lambda **kw: long_few(num_reqs=1, **kw),
    "long_8": lambda **kw: long_few(num_reqs=8, **kw),
}


def make(name, **kw):
    return CONFIGS[name](**kw)
