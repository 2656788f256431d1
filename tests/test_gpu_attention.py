"""The sparse-attention consumer (qsa_sparse_attention) against its CPU
oracle (oracle/attention.py), element by element.

Tolerance, from the arithmetic: the inputs are fp16 and exact in the float64
oracle; the GPU accumulates the scores and P.V in fp32 (errors ~1e-6
relative) and evaluates exp in fp32, but feeds the softmax weights to the
P.V product rounded to fp16, a relative error of at most 2^-11 per weight,
while the normaliser sums the fp32 weights.  So each output element is off by
at most about 2^-11 * sum_t w_t |V_t| <= 2^-11 * max_t |V_t|; the test allows
2^-10 * max_t |V_t| of the row's selected values (per KV head) plus 1e-5.
"""
import numpy as np
import pytest
import torch

import workloads as W
from oracle import attention as OA
from paged_block_scoring_amd import qsa as Q

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def make_cache(seed, reqs, ctx, q_heads=24, kv_heads=2, d=256, page_size=64, rows=None):
    rng = np.random.default_rng(seed)
    pages_per = (ctx + page_size - 1) // page_size
    pool = reqs * pages_per + 3
    pt = rng.permutation(pool)[:reqs * pages_per].astype(np.int32).reshape(reqs, pages_per)
    k = rng.standard_normal((pool, page_size, kv_heads, d)).astype(np.float16)
    v = rng.standard_normal((pool, page_size, kv_heads, d)).astype(np.float16)
    rows = rows or reqs
    q = rng.standard_normal((rows, q_heads, d)).astype(np.float16)
    row_req = (np.arange(rows) % reqs).astype(np.int32)
    return rng, q, k, v, pt, row_req


def run(q, k, v, pt, tok, row_req):
    d = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(DEV)  # noqa: E731
    out = Q.qsa_sparse_attention(d(q), d(k), d(v), d(pt), d(tok), row_req=d(row_req))
    torch.cuda.synchronize()
    return out.cpu().numpy()


def check(q, k, v, pt, tok, row_req):
    got = run(q, k, v, pt, tok, row_req)
    ref = OA.sparse_attention(q, k, v, pt, tok, row_req=row_req)
    group = q.shape[1] // k.shape[2]
    worst = 0.0
    for r in range(q.shape[0]):
        sel = tok[r][tok[r] >= 0]
        if sel.size == 0:
            assert not got[r].any(), r
            continue
        vals = v[pt[row_req[r], sel // k.shape[1]], sel % k.shape[1]].astype(np.float64)  # [n, kv, d]
        for h in range(q.shape[1]):
            vmax = np.abs(vals[:, h // group]).max()
            err = np.abs(got[r, h] - ref[r, h]).max()
            worst = max(worst, err / vmax)
            assert err <= 2.0 ** -10 * vmax + 1e-5, (r, h, err, vmax)
    return worst


def test_attention_lists_of_every_shape():
    """Lists shorter than a chunk, several chunks with a ragged tail, two
    windows of 2,048 entries, padding in the middle and at the tail, an empty
    row, a single token, repeated entries."""
    rng, q, k, v, pt, rr = make_cache(11, reqs=3, ctx=5000, rows=9)
    kmax = 2100
    tok = np.full((9, kmax), -1, np.int32)
    tok[0, :1] = 4999
    tok[1, :63] = rng.choice(5000, 63, replace=False)
    tok[2, :200] = rng.choice(5000, 200, replace=False)
    tok[3, :kmax] = rng.choice(5000, kmax, replace=False)
    tok[4, :] = -1                                            # empty row
    tok[5, ::3] = rng.choice(5000, (kmax + 2) // 3, replace=False)  # padding in the middle
    tok[6, :2048] = np.arange(2048)                           # a whole prefix
    tok[7, :64] = 17                                          # one token listed 64 times
    tok[8, :130] = rng.choice(5000, 130, replace=False)
    check(q, k, v, pt, tok, rr)


def test_attention_gqa_group_sizes():
    for q_heads, kv_heads in ((24, 2), (16, 1), (8, 8), (32, 2)):
        rng, q, k, v, pt, rr = make_cache(12, reqs=2, ctx=3000, q_heads=q_heads, kv_heads=kv_heads, rows=4)
        tok = np.stack([rng.choice(3000, 700, replace=False) for _ in range(4)]).astype(np.int32)
        check(q, k, v, pt, tok, rr)


def test_attention_large_scores():
    """Scores far from zero (no overflow, the running max does its work)."""
    rng, q, k, v, pt, rr = make_cache(13, reqs=1, ctx=2000, rows=2)
    q *= np.float16(6)
    tok = np.stack([rng.choice(2000, 500, replace=False) for _ in range(2)]).astype(np.int32)
    check(q, k, v, pt, tok, rr)


def test_attention_split_lists():
    """Few rows split each list over several workgroups (a workspace holds the
    partial results): tokens only in the first or only in the last split,
    every split but one empty, an empty row, and scores far from zero in
    different splits."""
    rng, q, k, v, pt, rr = make_cache(15, reqs=2, ctx=6000, rows=5)
    kmax = 2048
    assert Q.qsa_sparse_attention_workspace_size(5, 24, 2, 256, kmax) > 0
    tok = np.full((5, kmax), -1, np.int32)
    tok[0, :5] = rng.choice(6000, 5, replace=False)             # first split only
    tok[1, kmax - 7:] = rng.choice(6000, 7, replace=False)      # last split only
    tok[2, ::500] = rng.choice(6000, len(range(0, kmax, 500)), replace=False)  # one token in a few splits
    tok[4, :] = rng.choice(6000, kmax, replace=False)           # every split full
    q[4] *= np.float16(5)                                       # large scores, maxima in different splits
    check(q, k, v, pt, tok, rr)


def test_attention_many_rows_no_split():
    """Enough (row, KV head) pairs to fill the device: one workgroup per pair,
    no workspace."""
    rows = 260
    assert Q.qsa_sparse_attention_workspace_size(rows, 24, 2, 256, 300) == 0
    rng, q, k, v, pt, rr = make_cache(16, reqs=4, ctx=3000, rows=rows)
    tok = np.stack([rng.choice(3000, 300, replace=False) for _ in range(rows)]).astype(np.int32)
    tok[7, 100:] = -1
    tok[8, :] = -1
    check(q, k, v, pt, tok, rr)


def test_attention_after_the_indexer():
    """End to end on a reduced kernel shape (80 rows of a 184k context): the
    indexer's token selection feeds the consumer."""
    w = W.kernel_shape(rows=80)
    dq = lambda a: torch.from_numpy(a).to(DEV)  # noqa: E731
    import oracle
    mv = max(oracle.visible_keys(int(p), w.compress_ratio) for p in w.pos)
    tok = Q.qsa_select_paged_tokens(dq(w.q), dq(w.kcache), dq(w.page_table), dq(w.pos), w.compress_ratio, w.k,
                                    max_visible=mv, row_req=dq(w.row_req))
    torch.cuda.synchronize()
    tok = tok.cpu().numpy()
    rng = np.random.default_rng(14)
    q = rng.standard_normal((w.rows, 24, 256)).astype(np.float16)
    # the main cache shares the index cache's page table (64-token pages)
    k = rng.standard_normal((w.num_pages, 64, 2, 256)).astype(np.float16)
    v = rng.standard_normal((w.num_pages, 64, 2, 256)).astype(np.float16)
    worst = check(q, k, v, w.page_table, tok, w.row_req)
    print(f"attention after the indexer: rows={w.rows} worst error / max|V| = {worst:.2e}")
