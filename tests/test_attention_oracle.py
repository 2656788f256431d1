"""Pins of the sparse-attention consumer's CPU oracle (oracle/attention.py):
closed forms and invariances that the softmax-attention definition fixes,
each chosen so that a plausible mistake (scale, head mapping, page or slot
arithmetic, padding, the softmax axis, overflow without the max shift) fails
one of them."""
import math

import numpy as np

from oracle.attention import sparse_attention


def _case(seed, rows=3, q_heads=24, kv_heads=2, d=256, page_size=64, pages=6, reqs=2):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((rows, q_heads, d)).astype(np.float16)
    k = rng.standard_normal((pages * reqs, page_size, kv_heads, d)).astype(np.float16)
    v = rng.standard_normal((pages * reqs, page_size, kv_heads, d)).astype(np.float16)
    pt = rng.permutation(pages * reqs).astype(np.int32).reshape(reqs, pages)
    row_req = (np.arange(rows) % reqs).astype(np.int32)
    return q, k, v, pt, row_req


def test_single_token_is_its_value():
    q, k, v, pt, rr = _case(1)
    tok = np.array([[200, -1, -1], [5, -1, -1], [383, -1, -1]], np.int32)
    out = sparse_attention(q, k, v, pt, tok, row_req=rr)
    for r in range(3):
        t = tok[r, 0]
        page, slot = pt[rr[r], t // 64], t % 64
        for h in range(24):
            assert np.array_equal(out[r, h], v[page, slot, h // 12].astype(np.float64))


def test_zero_query_averages_values():
    q, k, v, pt, rr = _case(2)
    q[:] = 0
    tok = np.array([[1, 2, 300, 64], [0, 63, -1, -1], [10, 11, 12, 13]], np.int32)
    out = sparse_attention(q, k, v, pt, tok, row_req=rr)
    for r in range(3):
        sel = tok[r][tok[r] >= 0]
        vals = v[pt[rr[r], sel // 64], sel % 64].astype(np.float64)  # [n, kv, d]
        for h in range(24):
            assert np.allclose(out[r, h], vals[:, h // 12].mean(axis=0), rtol=0, atol=1e-12)


def test_two_tokens_closed_form_with_scale():
    # q = a e0, K1 = b1 e0, K2 = b2 e0: the scores are a*b*scale exactly, the
    # weights sigma(s1 - s2) and its complement
    d, page_size = 256, 64
    q = np.zeros((1, 24, d), np.float16)
    k = np.zeros((2, page_size, 2, d), np.float16)
    v = np.random.default_rng(3).standard_normal((2, page_size, 2, d)).astype(np.float16)
    q[0, :, 0] = 4.0
    k[1, 3, :, 0] = 2.0     # token 64 + 3 = 67 (page 1)
    k[0, 9, :, 0] = -1.5    # token 9 (page 0)
    pt = np.array([[0, 1]], np.int32)
    out = sparse_attention(q, k, v, pt, np.array([[67, 9]], np.int32))
    s1, s2 = 4.0 * 2.0 / 16.0, 4.0 * -1.5 / 16.0
    w1 = 1.0 / (1.0 + math.exp(s2 - s1))
    for h in range(24):
        g = h // 12
        exp = w1 * v[1, 3, g].astype(np.float64) + (1 - w1) * v[0, 9, g].astype(np.float64)
        assert np.allclose(out[0, h], exp, rtol=0, atol=1e-12)


def test_large_scores_do_not_overflow():
    q, k, v, pt, rr = _case(4, rows=1)
    q[:] = np.float16(60)
    k[:] = np.float16(60)  # scores of 60*60*256/16 = 57,600: exp overflows without the max shift
    out = sparse_attention(q, k, v, pt, np.array([[1, 2, 3]], np.int32), row_req=rr[:1])
    assert np.all(np.isfinite(out))


def test_heads_map_to_kv_head_by_group():
    q, k, v, pt, rr = _case(5, rows=1)
    q[0, :] = q[0, 0]  # every query head the same vector
    out = sparse_attention(q, k, v, pt, np.array([[7, 70, 130, 250]], np.int32), row_req=rr[:1])
    assert np.array_equal(out[0, 0], out[0, 11])      # heads 0..11 read KV head 0
    assert np.array_equal(out[0, 12], out[0, 23])     # heads 12..23 read KV head 1
    assert not np.allclose(out[0, 11], out[0, 12])


def test_invariances_padding_order_pages():
    q, k, v, pt, rr = _case(6)
    tok = np.array([[3, 70, 128, 300, 5], [64, 65, 66, 0, 1], [383, 200, 100, 50, 25]], np.int32)
    base = sparse_attention(q, k, v, pt, tok, row_req=rr)
    # padding anywhere is ignored
    padded = np.full((3, 9), -1, np.int32)
    padded[:, ::2] = tok
    assert np.array_equal(sparse_attention(q, k, v, pt, padded, row_req=rr), base)
    # the order of the list does not matter
    perm = tok[:, ::-1].copy()
    assert np.allclose(sparse_attention(q, k, v, pt, perm, row_req=rr), base, rtol=0, atol=1e-12)
    # relabelled physical pages
    rng = np.random.default_rng(7)
    relabel = rng.permutation(k.shape[0])
    k2, v2 = np.empty_like(k), np.empty_like(v)
    k2[relabel], v2[relabel] = k, v
    pt2 = relabel[pt].astype(np.int32)
    assert np.array_equal(sparse_attention(q, k2, v2, pt2, tok, row_req=rr), base)


def test_empty_row_is_zero():
    q, k, v, pt, rr = _case(8, rows=2)
    out = sparse_attention(q, k, v, pt, np.array([[-1, -1], [4, -1]], np.int32), row_req=rr)
    assert not out[0].any()
    assert out[1].any()
