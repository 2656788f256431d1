"""The three steps chained on the GPU: the compressed-key producer builds the
side cache from raw token keys (one prefill call per request, then decode
calls), the indexer selects tokens from that cache, and the sparse-attention
consumer attends over the selection.  Each step is checked against its own
oracle on the GPU output of the step before it, to that step's bar:
  * producer: every stored key within half an fp16 ulp of the oracle's value
    plus 4e-6 of the key's largest value (the bar of the producer's own tests);
  * indexer: scores within 1e-3 relative of the oracle's on the same cache,
    and the selection bit-exact with the oracle's selector run on the GPU's
    own scores;
  * consumer: within 2^-10 of the largest selected value plus 1e-5 of the
    oracle's float64 attention over the same selection."""
import numpy as np
import pytest
import torch

import oracle as O
import workloads as W
from oracle import attention as OA
from oracle import producer as OP
from paged_block_scoring_amd import qsa as Q

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
D = 128


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def test_produce_select_attend():
    cr, page_size, k = 4, 64, 512
    prefill = [6000, 3001]
    steps = 3
    total = [n + steps for n in prefill]
    keys, w, pt, pool = W.raw_token_keys(21, total, page_size, cr)
    kpp = page_size // cr

    # producer: one prefill call holding both requests, then decode calls
    kc = torch.zeros((pool, kpp, D), dtype=torch.float16, device=DEV)
    state = torch.zeros((len(total), cr, D), dtype=torch.float16, device=DEV)
    calls = [[(0, 0, prefill[0]), (1, 0, prefill[1])]]
    calls += [[(1, prefill[1] + s, prefill[1] + s + 1), (0, prefill[0] + s, prefill[0] + s + 1)] for s in range(steps)]
    for call in calls:
        k_tok = np.concatenate([keys[q][a:b] for q, a, b in call])
        req = np.concatenate([np.full(b - a, q, np.int32) for q, a, b in call])
        pos = np.concatenate([np.arange(a, b, dtype=np.int32) for q, a, b in call])
        Q.qsa_compress_keys(dev(k_tok), dev(pos), state, kc, dev(pt), cr, tok_req=dev(req), norm_w=dev(w))
    torch.cuda.synchronize()
    cache = kc.cpu().numpy()
    stored = OP.produce(keys, pt, page_size, cr, w)
    assert len(stored) == sum(n // cr for n in total)
    for (page, slot), ref in stored.items():
        got = cache[page, slot].astype(np.float64)
        e = np.floor(np.log2(np.maximum(np.abs(ref), 2.0 ** -14)))
        tol = 0.5 * 2.0 ** (e - 10) + 4e-6 * np.abs(ref).max() + 2.0 ** -25
        assert np.all(np.abs(got - ref) <= tol), (page, slot)

    # indexer: the last rows of each request, over the cache the producer built
    rng = np.random.default_rng(22)
    rows_per = [63, 24]
    pos = np.concatenate([np.arange(t - n, t, dtype=np.int32) for t, n in zip(total, rows_per)])
    row_req = np.concatenate([np.full(n, q, np.int32) for q, n in enumerate(rows_per)])
    rows = len(pos)
    q = rng.standard_normal((rows, 4, D)).astype(np.float16)
    d_q, d_pt, d_pos, d_rr = dev(q), dev(pt), dev(pos), dev(row_req)
    V = np.array([O.visible_keys(int(p), cr) for p in pos], np.int32)
    scores = Q.qsa_score_paged(d_q, kc, d_pt, d_pos, cr, max_visible=int(V.max()), row_req=d_rr)
    tok = Q.qsa_select_paged_tokens(d_q, kc, d_pt, d_pos, cr, k, max_visible=int(V.max()), row_req=d_rr)
    torch.cuda.synchronize()
    gs, tok = scores.cpu().numpy(), tok.cpu().numpy()
    ref = O.score_paged(q, cache, pt, pos, cr, row_req=row_req)
    for r in range(rows):
        a, b = gs[r, :V[r]].astype(np.float64), ref[r, :V[r]].astype(np.float64)
        assert np.all(np.abs(a - b) <= 1e-3 * np.maximum(np.abs(b), 1.0)), r
    blocks = O.select_rows(gs, V, k // cr)
    want = np.where(blocks[:, :, None] >= 0, blocks[:, :, None] * cr + np.arange(cr), -1).reshape(rows, k)
    assert np.array_equal(tok, want.astype(np.int32))

    # consumer: 24 query heads over 2 KV heads, a main cache on the same pages
    qa = rng.standard_normal((rows, 24, 256)).astype(np.float16)
    kv_k = rng.standard_normal((pool, page_size, 2, 256)).astype(np.float16)
    kv_v = rng.standard_normal((pool, page_size, 2, 256)).astype(np.float16)
    out = Q.qsa_sparse_attention(dev(qa), dev(kv_k), dev(kv_v), d_pt, dev(tok), row_req=d_rr)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    exp = OA.sparse_attention(qa, kv_k, kv_v, pt, tok, row_req=row_req)
    for r in range(rows):
        sel = tok[r][tok[r] >= 0]
        vals = kv_v[pt[row_req[r], sel // page_size], sel % page_size].astype(np.float64)
        for h in range(24):
            vmax = np.abs(vals[:, h // 12]).max()
            assert np.abs(got[r, h] - exp[r, h]).max() <= 2.0 ** -10 * vmax + 1e-5, (r, h)
