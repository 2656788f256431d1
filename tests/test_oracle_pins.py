"""Pins of the CPU oracle against things other than itself.

Each test checks the oracle against a fact the pages or the mathematics fix:
the IEEE binary16 format (NumPy's converter), the causal visibility rule by
brute force, exact integer arithmetic (int64 matmul), the textbook fp32
summation error bound against a float64 recomputation, a library sort
(np.lexsort) for the exact lexicographic top-k, closed forms, metamorphic
relations, and a hand-derived golden fixture.  Sources: the Qwen3.8-Flash-Next
spec PR (section "The component deep-dives, and two corrections to the above")
and the Turing QSA indexer PR (sections "Purpose", "Test Plan", "Path
coverage", "Test Result").
"""
import numpy as np
import pytest

import workloads as W
from conftest import golden_arrays, load_golden

U = 2.0 ** -24


def gamma(n):
    return n * U / (1 - n * U)


# ---------------------------------------------------------------- fp16 input

def test_half_to_float_all_bit_patterns(oracle_mod):
    bits = np.arange(65536, dtype=np.uint32)
    ref = bits.astype(np.uint16).view(np.float16).astype(np.float32)
    got = np.array([oracle_mod.half_to_float(int(b)) for b in bits], dtype=np.float32)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan].view(np.uint32), ref[~nan].view(np.uint32))


# ---------------------------------------------------------------- visibility

@pytest.mark.parametrize("cr", [1, 2, 3, 4, 8])
def test_visibility_brute_force(oracle_mod, cr):
    """Key j covers tokens cr*j..cr*j+cr-1 and exists once position cr*j+cr-1
    has been seen; count the complete keys by brute force."""
    for pos in range(-1, 4096):
        brute = sum(1 for j in range(0, 4096) if cr * j + cr - 1 <= pos)
        assert oracle_mod.visible_keys(pos, cr) == brute, (pos, cr)


def test_visibility_through_full_path(oracle_mod):
    """The number of non-padding tokens is cr * min(kb, V) with V the brute
    force count, through the whole oracle path."""
    rng = np.random.default_rng(11)
    ctx = 300
    w = W.build("vis", rng, 11, [ctx], [ctx], permute_pages=True, k=4 * 200)
    out = oracle_mod.select_paged_tokens(w.q, w.kcache, w.page_table, w.pos, 4, w.k)
    for r, p in enumerate(w.pos):
        V = sum(1 for j in range(ctx) if 4 * j + 3 <= p)
        assert int((out[r] >= 0).sum()) == 4 * min(200, V)
        assert np.all(out[r][4 * min(200, V):] == -1)


# ---------------------------------------------------------------- scores

def dense_keys(w, req):
    """Logical keys of request `req` gathered through the page table (numpy)."""
    kpp = w.kcache.shape[1]
    n = w.page_table.shape[1]
    return w.kcache[w.page_table[req, :n]].reshape(n * kpp, -1)


def _int_workload(seed, ctxs, rows):
    rng = np.random.default_rng(seed)
    return W.build("int", rng, seed, ctxs, rows, permute_pages=True, integer=True, k=64,
                   extra_pages=3)


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_integer_scores_exact_int64(oracle_mod, seed):
    """Integer inputs in -2..2: every fp32 partial sum is an integer below
    2^24, so the oracle's fp32 score equals the exact int64 dot product."""
    w = _int_workload(seed, [260, 97, 130], [5, 3, 4])
    s = oracle_mod.score_paged(w.q, w.kcache, w.page_table, w.pos, 4, row_req=w.row_req)
    for r in range(w.rows):
        req = int(w.row_req[r])
        V = (int(w.pos[r]) + 1) // 4
        K = dense_keys(w, req)[:V].astype(np.int64)
        qi = w.q[r].astype(np.int64)                 # [H, D]
        ref = (K @ qi.T).sum(axis=1)                 # exact integer sum over heads
        assert np.array_equal(s[r, :V], ref.astype(np.float32)), r
        assert np.all(np.isnan(s[r, V:]))


def test_large_integer_query_scores_exact_int64(oracle_mod):
    """Integer queries with planted values up to 65504 whose sum over the
    heads reaches 4 * 65504 in a dimension: every per-head dot is an integer
    below 2^21 and their sum below 2^24, so the oracle's fp32 score is the
    exact int64 dot product (the large-magnitude parity cases rely on it)."""
    w = W.large_query(_int_workload(3, [260, 97, 130], [12, 3, 9]), seed=5)
    u = np.abs(w.q.astype(np.int64).sum(axis=1)).max(axis=1)
    assert u.max() == 4 * 65504 and np.any((u > 65504) & (u <= 2 * 65504))
    s = oracle_mod.score_paged(w.q, w.kcache, w.page_table, w.pos, 4, row_req=w.row_req)
    for r in range(w.rows):
        V = (int(w.pos[r]) + 1) // 4
        K = dense_keys(w, int(w.row_req[r]))[:V].astype(np.int64)
        heads = K @ w.q[r].astype(np.int64).T
        assert np.abs(heads).max(initial=0) < 2 ** 21 and np.abs(heads.sum(axis=1)).max(initial=0) < 2 ** 24
        assert np.array_equal(s[r, :V], heads.sum(axis=1).astype(np.float32)), r


@pytest.mark.parametrize("seed", [0, 1])
def test_integer_scores_relu_exact(oracle_mod, seed):
    """relu form: sum over heads of relu(integer dot) is an exact integer; the
    oracle's result is that integer times the fp32 scale within two roundings
    of the exact value integer / sqrt(128)."""
    w = _int_workload(seed, [200, 120], [4, 6])
    s = oracle_mod.score_paged(w.q, w.kcache, w.page_table, w.pos, 4, row_req=w.row_req,
                               flags=oracle_mod.SCORE_RELU)
    for r in range(w.rows):
        V = (int(w.pos[r]) + 1) // 4
        K = dense_keys(w, int(w.row_req[r]))[:V].astype(np.int64)
        heads = K @ w.q[r].astype(np.int64).T
        isum = np.maximum(heads, 0).sum(axis=1).astype(np.float64)
        exact = isum / np.sqrt(128.0)
        err = np.abs(s[r, :V].astype(np.float64) - exact)
        assert np.all(err <= 3 * U * np.abs(exact)), r


def test_scale_constant_is_nearest_fp32(oracle_mod):
    """A single nonzero head dot of 1 isolates the scale: it must be the fp32
    value nearest 1/sqrt(128)."""
    q = np.zeros((1, 4, 128), np.float16)
    q[0, 0, 0] = 1
    kc = np.zeros((1, 16, 128), np.float16)
    kc[0, :, 0] = 1
    s = oracle_mod.score_paged(q, kc, np.zeros((1, 1), np.int32), np.array([63], np.int32), 4,
                               flags=oracle_mod.SCORE_RELU)
    x = 1.0 / np.sqrt(128.0)
    cands = np.array([np.float32(x), np.nextafter(np.float32(x), np.float32(0)),
                      np.nextafter(np.float32(x), np.float32(1))], dtype=np.float32)
    nearest = cands[np.argmin(np.abs(cands.astype(np.float64) - x))]
    assert s[0, 0] == nearest


@pytest.mark.parametrize("relu", [False, True])
def test_gaussian_scores_within_fp32_bound(oracle_mod, relu):
    """N(0,1) inputs: the oracle's fp32 score lies within the textbook bound
    gamma_n * sum|terms| of a float64 dense recomputation (n = 128 + 4
    additions), plus the two roundings of the scale in the relu form."""
    rng = np.random.default_rng(5)
    w = W.build("g", rng, 5, [700, 333], [6, 5], permute_pages=True, k=64)
    flags = oracle_mod.SCORE_RELU if relu else 0
    s = oracle_mod.score_paged(w.q, w.kcache, w.page_table, w.pos, 4, row_req=w.row_req, flags=flags)
    for r in range(w.rows):
        V = (int(w.pos[r]) + 1) // 4
        K = dense_keys(w, int(w.row_req[r]))[:V].astype(np.float64)
        qd = w.q[r].astype(np.float64)
        heads = K @ qd.T                             # [V, H] float64
        absterms = np.abs(K) @ np.abs(qd).T
        if relu:
            ref = np.maximum(heads, 0).sum(axis=1) / np.sqrt(128.0)
            bound = gamma(132) * absterms.sum(axis=1) / np.sqrt(128.0) + 3 * U * np.abs(ref)
        else:
            ref = heads.sum(axis=1)
            bound = gamma(132) * absterms.sum(axis=1)
        err = np.abs(s[r, :V].astype(np.float64) - ref)
        assert np.all(err <= bound), (r, float((err - bound).max()))


# ---------------------------------------------------------------- selection

def lexsort_topk(scores, V, k):
    idx = np.arange(V)
    order = np.lexsort((idx, -scores[:V].astype(np.float64)))
    sel = order[:k]
    return np.concatenate([sel, -np.ones(k - len(sel), dtype=np.int64)])


def test_select_rows_vs_lexsort_brute_force(oracle_mod):
    rng = np.random.default_rng(7)
    for trial in range(300):
        V = int(rng.integers(0, 301))
        k = int(rng.integers(1, 65))
        ld = V + int(rng.integers(0, 5)) + 1
        mode = trial % 3
        if mode == 0:       # heavy ties
            sc = rng.integers(-3, 4, size=ld).astype(np.float32)
        elif mode == 1:     # continuous
            sc = rng.standard_normal(ld).astype(np.float32)
        else:               # signed zeros and few values
            sc = rng.choice(np.array([-0.0, 0.0, 1.0, -1.0], np.float32), size=ld)
        out = oracle_mod.select_rows(sc[None, :], np.array([V], np.int32), k)
        assert np.array_equal(out[0], lexsort_topk(sc, V, k)), trial


def test_select_invariants(oracle_mod):
    """Min selected >= max unselected; among cutoff ties the selected indices
    all lie below the unselected ones (the exact-selector requirement of the
    Turing PR's "Purpose" and the failing invariant of its "Test Result")."""
    rng = np.random.default_rng(9)
    V, k = 20_000, 512
    sc = rng.integers(-40, 41, size=V).astype(np.float32)
    out = oracle_mod.select_rows(sc[None, :], np.array([V], np.int32), k)[0]
    sel = np.zeros(V, bool)
    sel[out] = True
    assert sc[sel].min() >= sc[~sel].max()
    cut = sc[sel].min()
    assert np.where(sel & (sc == cut))[0].max() < np.where(~sel & (sc == cut))[0].min()
    # rank order: scores non-increasing, indices ascending within equal scores
    s = sc[out]
    assert np.all(np.diff(s) <= 0)
    same = np.diff(s) == 0
    assert np.all(np.diff(out)[same] > 0)


def test_signed_zero_ties(oracle_mod):
    sc = np.array([[0.0, -0.0, 1.0, -0.0, 0.0]], np.float32)
    sc[0, 0] = -0.0
    out = oracle_mod.select_rows(sc, np.array([5], np.int32), 5)
    assert out.tolist() == [[2, 0, 1, 3, 4]]


def test_all_equal_closed_form(oracle_mod):
    """All scores equal: the lowest indices win, so blocks 0..kb-1, i.e.
    tokens 0..k-1."""
    q = np.zeros((3, 4, 128), np.float16)
    kc = np.zeros((8, 16, 128), np.float16)
    pt = np.arange(8, dtype=np.int32)[None, :]
    pos = np.array([511, 200, 40], np.int32)
    out = oracle_mod.select_paged_tokens(q, kc, pt, pos, 4, 64)
    assert np.array_equal(out[0], np.arange(64))
    assert np.array_equal(out[1], np.arange(64))
    # V = 10 keys < kb = 16 blocks: 40 tokens then padding
    assert np.array_equal(out[2], np.concatenate([np.arange(40), -np.ones(24, int)]))


def test_known_permutation_ranks(oracle_mod):
    """key j = c_j * e0 and q = e0 on head 0: score_j = c_j exactly, so the
    rank is argsort of -c."""
    rng = np.random.default_rng(3)
    V = 256
    c = rng.permutation(V).astype(np.float16) - 128
    kc = np.zeros((16, 16, 128), np.float16)
    kc.reshape(-1, 128)[:V, 0] = c
    q = np.zeros((1, 4, 128), np.float16)
    q[0, 0, 0] = 1
    out = oracle_mod.select_paged_tokens(q, kc, np.arange(16, dtype=np.int32)[None], np.array([1023], np.int32),
                                         4, 4 * 32, flags=oracle_mod.OUT_KEYS)
    assert np.array_equal(out[0][:32], np.argsort(-c.astype(np.float64), kind="stable")[:32])


# ---------------------------------------------------------------- golden

def test_golden_paged_ties_expand(oracle_mod):
    g = load_golden("paged_ties_expand.json")
    q, kc, pt, pos = golden_arrays(g)
    cr = g["compress_ratio"]
    out = oracle_mod.select_paged_tokens(q, kc, pt, pos, cr, g["k"])
    assert out.tolist() == g["expected_tokens"]
    out = oracle_mod.select_paged_tokens(q, kc, pt, pos, cr, g["k"], flags=oracle_mod.SCORE_RELU)
    assert out.tolist() == g["expected_tokens_relu"]
    out = oracle_mod.select_paged_tokens(q, kc, pt, pos, cr, g["k_keys"], flags=oracle_mod.OUT_KEYS)
    assert out.tolist() == g["expected_keys"]
    s = oracle_mod.score_paged(q, kc, pt, pos, cr)
    assert s[0, :16].tolist() == g["expected_scores_row0_first16"]


# ---------------------------------------------------------------- metamorphic

def test_page_relabelling_invariance(oracle_mod):
    """Moving pages to other physical slots (and updating the page table)
    leaves every output unchanged; contiguous and permuted pools agree."""
    rng = np.random.default_rng(21)
    w = W.build("m", rng, 21, [900, 500], [7, 9], permute_pages=False, k=128)
    perm = rng.permutation(w.num_pages)
    kc2 = np.empty_like(w.kcache)
    kc2[perm] = w.kcache
    pt2 = perm[w.page_table].astype(np.int32)
    for flags in (0, oracle_mod.SCORE_RELU):
        a = oracle_mod.select_paged_tokens(w.q, w.kcache, w.page_table, w.pos, 4, w.k, row_req=w.row_req, flags=flags)
        b = oracle_mod.select_paged_tokens(w.q, kc2, pt2, w.pos, 4, w.k, row_req=w.row_req, flags=flags)
        assert np.array_equal(a, b)


def test_request_split_and_row_permutation(oracle_mod):
    """Each row's output depends only on its own request: scoring requests
    together or one at a time, and in any row order, gives the same rows."""
    rng = np.random.default_rng(22)
    w = W.build("m", rng, 22, [640, 300, 1000], [5, 4, 6], permute_pages=True, k=256)
    both = oracle_mod.select_paged_tokens(w.q, w.kcache, w.page_table, w.pos, 4, w.k, row_req=w.row_req)
    for req in range(w.num_reqs):
        m = w.row_req == req
        alone = oracle_mod.select_paged_tokens(w.q[m], w.kcache, w.page_table[req:req + 1], w.pos[m], 4, w.k)
        assert np.array_equal(alone, both[m])
    perm = rng.permutation(w.rows)
    shuf = oracle_mod.select_paged_tokens(w.q[perm], w.kcache, w.page_table, w.pos[perm], 4, w.k,
                                          row_req=w.row_req[perm])
    assert np.array_equal(shuf, both[perm])


def test_full_path_equals_score_then_select(oracle_mod):
    rng = np.random.default_rng(23)
    w = W.build("m", rng, 23, [2000], [12], permute_pages=True, k=256)
    s = oracle_mod.score_paged(w.q, w.kcache, w.page_table, w.pos, 4)
    V = np.array([(int(p) + 1) // 4 for p in w.pos], np.int32)
    blocks = oracle_mod.select_rows(np.nan_to_num(s, nan=0.0), V, 64)
    toks = np.where(blocks[:, :, None] >= 0, blocks[:, :, None] * 4 + np.arange(4), -1).reshape(w.rows, -1)
    full = oracle_mod.select_paged_tokens(w.q, w.kcache, w.page_table, w.pos, 4, w.k)
    assert np.array_equal(full, toks)


# ---------------------------------------------------------------- generator

def test_generator_deterministic():
    a, b = W.tiny(), W.tiny()
    assert a.digest() == b.digest()
    assert W.tiny(seed=5).digest() != a.digest()
    m1, m2 = W.mixed(), W.mixed()
    assert m1.digest() == m2.digest()
    assert m1.rows == int(np.sum(np.bincount(m1.row_req)))


def test_generator_shapes():
    w = W.kernel_shape(rows=16)
    assert w.pos.tolist() == list(range(184_000 - 16, 184_000))
    assert w.page_table.shape == (1, 2875)
    t = W.tiny()
    assert t.pos.min() == 960 and t.pos.max() == 1023 and t.k == 64
    ts = W.tie_stress(rows=8)
    assert set(np.unique(ts.q.astype(np.float32))) <= {-2.0, -1.0, 0.0, 1.0, 2.0}
