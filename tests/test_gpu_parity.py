"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Bar (from the indexer's definition): integer-valued inputs are exact in fp32
whatever the summation order, so scores and indices must be bit-exact with
the oracle; on Gaussian inputs each score must lie within 1e-3 * max(|ref|, 1)
of the oracle's, and the selection the GPU makes on its own scores must be
bit-exact with the oracle's selector applied to those same scores.  Sources:
"[Perf][Qwen4Exp] Admit the cuBLAS QSA indexer and exact top-k on Turing",
sections "Purpose" (exact lexicographic selector) and "Test Plan" (selected
token sets identical in all rows); "spec(MODEL-MM-QWEN4-EXP) ...", section
"The component deep-dives, and two corrections to the above".
"""
import contextlib
import sys

import numpy as np
import pytest
import torch

import workloads as W
from paged_block_scoring_amd import qsa as Q

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
RELU = Q.QSA_SCORE_RELU
KEYS = Q.QSA_OUT_KEYS


PATHS = ["two_pass", "fused", "fused_fallback", "fused_redo", "stream"]


ARM_BITS = {"two_pass": Q.QSA_DEBUG_FORCE_TWO_PASS, "fused": Q.QSA_DEBUG_FORCE_FUSED,
            "fused_fallback": Q.QSA_DEBUG_FORCE_FALLBACK, "fused_redo": Q.QSA_DEBUG_FORCE_REDO,
            "stream": Q.QSA_DEBUG_FORCE_STREAM}
SCORER_BITS = {"tiles": Q.QSA_DEBUG_FORCE_TILES, "groups": Q.QSA_DEBUG_FORCE_GROUPS}


@contextlib.contextmanager
def _forced(group, bit):
    """Replace the override bits of one group (arms or scorers) for the block."""
    old = Q.qsa_debug_forced()
    Q.qsa_debug_force((old & ~sum(group.values())) | bit)
    try:
        yield
    finally:
        Q.qsa_debug_force(old)


def force_path(name):
    """Drive one execution arm deliberately; "fused_fallback" makes every row
    of the fused arm take its exact recompute path, "fused_redo" every row's
    final select its second pass; None leaves the choice to the library."""
    return _forced(ARM_BITS, 0 if name is None else ARM_BITS[name])


def note(*a):
    print(*a, file=sys.stderr, flush=True)


def to_dev(w):
    return dict(q=torch.from_numpy(w.q).to(DEV), kcache=torch.from_numpy(w.kcache).to(DEV),
                page_table=torch.from_numpy(w.page_table).to(DEV), pos=torch.from_numpy(w.pos).to(DEV),
                row_req=torch.from_numpy(w.row_req).to(DEV))


def visible(oracle_mod, w):
    return np.array([oracle_mod.visible_keys(int(p), w.compress_ratio) for p in w.pos], np.int32)


def max_visible(w):
    """The caller's bound on every row's visible key count (the oracle's rule)."""
    import oracle
    return max([oracle.visible_keys(int(p), w.compress_ratio) for p in w.pos], default=0)


def gpu_scores(d, w, flags):
    s = Q.qsa_score_paged(d["q"], d["kcache"], d["page_table"], d["pos"], w.compress_ratio,
                          max_visible=max_visible(w), row_req=d["row_req"], flags=flags & RELU)
    torch.cuda.synchronize()
    return s.cpu().numpy()


def gpu_select(d, w, flags, k=None):
    out = Q.qsa_select_paged_tokens(d["q"], d["kcache"], d["page_table"], d["pos"], w.compress_ratio,
                                    k or w.k, max_visible=max_visible(w), row_req=d["row_req"], flags=flags)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def expand(blocks, cr):
    rows, kb = blocks.shape
    t = np.where(blocks[:, :, None] >= 0, blocks[:, :, None] * cr + np.arange(cr), -1)
    return t.reshape(rows, kb * cr).astype(np.int32)


def expected_from_scores(oracle_mod, scores, V, k, cr, flags):
    kb = k if flags & KEYS else k // cr
    blocks = oracle_mod.select_rows(scores, V, kb)
    return blocks if flags & KEYS else expand(blocks, cr)


def assert_scores(gs, ref, V, exact, rows=None, floors=None):
    """floors[r] replaces the 1 of max(|ref|, 1) for rows whose query is the
    N(0,1) draw scaled by a power of two c: scaling q by c scales every score
    (and both sides' rounding errors) by c exactly, so the bar moves with it."""
    rows = range(len(V)) if rows is None else rows
    worst = 0.0
    for i, r in enumerate(rows):
        a = gs[r, :V[r]].astype(np.float64)
        b = ref[i, :V[r]].astype(np.float64)
        if exact:
            assert np.array_equal(a, b), f"row {r}: first mismatch at {np.argmax(a != b)}"
        else:
            floor = 1.0 if floors is None else float(floors[r])
            err = np.abs(a - b) / np.maximum(np.abs(b), floor)
            worst = max(worst, float(err.max(initial=0.0)))
            assert np.all(err <= 1e-3), f"row {r}: max rel err {err.max()}"
    return worst


def full_parity(oracle_mod, w, flags, integer, paths=(None,), floors=None):
    """Scores element by element, the GPU selection on its own scores, and
    (integer inputs) the whole path against the oracle, for each forced arm."""
    d = to_dev(w)
    V = visible(oracle_mod, w)
    gs = gpu_scores(d, w, flags)
    ref = oracle_mod.score_paged(w.q, w.kcache, w.page_table, w.pos, w.compress_ratio, row_req=w.row_req,
                                 flags=flags & RELU)
    worst = assert_scores(gs, ref, V, exact=integer, floors=floors)
    exp = expected_from_scores(oracle_mod, gs, V, w.k, w.compress_ratio, flags)
    full = None
    if integer:
        full = oracle_mod.select_paged_tokens(w.q, w.kcache, w.page_table, w.pos, w.compress_ratio, w.k,
                                              row_req=w.row_req, flags=flags)
    out = None
    for path in paths:
        with force_path(path):
            out = gpu_select(d, w, flags)
            ran = Q.qsa_last_path()
        if path is not None:
            assert ran == ("fused" if path.startswith("fused") else path)
        assert np.array_equal(out, exp), f"{w.name} path={path}: selection differs from oracle_select(GPU scores)"
        if full is not None:
            assert np.array_equal(out, full), f"{w.name} path={path}: differs from the oracle end to end"
    note(f"{w.name}: rows={w.rows} sumV={int(V.sum())} flags={flags} max_rel_err={worst:.2e}")
    return out


# ------------------------------------------------------------ small, whole

@pytest.mark.parametrize("flags", [0, RELU, KEYS, RELU | KEYS])
@pytest.mark.parametrize("integer", [False, True])
def test_tiny(oracle_mod, flags, integer):
    full_parity(oracle_mod, W.tiny(integer=integer), flags, integer, paths=PATHS)


REDUCED = {
    # 80 rows: one full 64-row tile plus a ragged 16-row tail; 46,000 keys
    # span 45 key chunks and end mid-chunk.
    "kernel_shape_80": lambda integer: W.kernel_shape(rows=80, integer=integer),
    "tie_stress_96": lambda integer: W.tie_stress(rows=96),
    "mixed_small": lambda integer: W.mixed(total_rows=100, max_rows=40, ctx_hi=40_000, integer=integer),
    "decode_small": lambda integer: W.decode(num_reqs=12, integer=integer),
    # three requests of 40 rows: 64-row tiles straddle request boundaries
    "three_reqs_40": lambda integer: W.build("three_reqs_40", np.random.default_rng(31), 31,
                                             [9000, 5003, 12345], [40, 40, 40], permute_pages=True,
                                             integer=integer, k=2048),
}


@pytest.mark.parametrize("flags", [0, RELU])
@pytest.mark.parametrize("integer", [False, True])
@pytest.mark.parametrize("name", sorted(REDUCED))
def test_reduced(oracle_mod, name, integer, flags):
    if name == "tie_stress_96" and not integer:
        pytest.skip("the tie-stress workload is integer-valued by definition")
    w = REDUCED[name](integer)
    full_parity(oracle_mod, w, flags, integer or name == "tie_stress_96", paths=PATHS)


def force_scorer(name):
    """Pick the scorer behind qsa_score_paged and the two-pass arm: "tiles"
    (rows of a tile share staged keys) or "groups" (each wave streams the keys
    of a small row window)."""
    return _forced(SCORER_BITS, SCORER_BITS[name])


@pytest.mark.parametrize("flags", [0, RELU])
@pytest.mark.parametrize("name", ["kernel_shape_80", "mixed_small", "decode_small", "three_reqs_40"])
def test_scorers_bit_identical(oracle_mod, name, flags):
    """Both scorers run the same MFMA chain on the same operands, so their
    scores must agree to the bit (windows of 32 / 8 rows here straddle request
    boundaries and end in ragged tails)."""
    w = REDUCED[name](False)
    d = to_dev(w)
    V = visible(oracle_mod, w)
    with force_scorer("tiles"):
        a = gpu_scores(d, w, flags)
    with force_scorer("groups"):
        b = gpu_scores(d, w, flags)
    for r in range(w.rows):
        assert np.array_equal(a[r, :V[r]].view(np.uint32), b[r, :V[r]].view(np.uint32)), f"row {r}"
    exp = expected_from_scores(oracle_mod, a, V, w.k, w.compress_ratio, flags)
    for scorer in ("groups", "tiles"):  # (the tiled scorer shares out each tile's own keys here)
        with force_scorer(scorer), force_path("two_pass"):
            out = gpu_select(d, w, flags)
        assert np.array_equal(out, exp), scorer


LARGE_Q = ["kernel_shape_80", "mixed_small", "decode_small", "three_reqs_40"]


@pytest.mark.parametrize("integer", [True, False])
@pytest.mark.parametrize("name", LARGE_Q)
def test_large_query(oracle_mod, name, integer):
    """Query rows whose sum over the index heads leaves fp16's range in some
    dimension (up to 4 * 65504, with rows at 65504, 65520, 131008, 131040 and
    262016 exactly): the default form's folded head sum must still give the
    oracle's scores -- bit-exact on the integer twin, within the tolerance on
    Gaussian rows scaled by 2^14 (its floor scaled by 2^14 too) -- and the
    same selection, in every arm."""
    w = W.large_query(REDUCED[name](integer), seed=77)
    floors = np.where(np.abs(w.q.astype(np.float32)).max(axis=(1, 2)) > 64.0, 16384.0, 1.0)
    for flags in (0, KEYS) + ((RELU,) if integer else ()):
        full_parity(oracle_mod, w, flags, integer, paths=PATHS, floors=None if integer else floors)


@pytest.mark.parametrize("name", LARGE_Q)
def test_large_query_scorers(oracle_mod, name):
    """The same large integer rows through both scorers: bit-identical scores,
    exact against the oracle, and the two-pass selection on the windowed
    scorer's output equal to the oracle's end to end."""
    w = W.large_query(REDUCED[name](True), seed=78)
    d = to_dev(w)
    V = visible(oracle_mod, w)
    ref = oracle_mod.score_paged(w.q, w.kcache, w.page_table, w.pos, w.compress_ratio, row_req=w.row_req)
    for scorer in ("tiles", "groups"):
        with force_scorer(scorer):
            gs = gpu_scores(d, w, 0)
        assert_scores(gs, ref, V, exact=True)
    full = oracle_mod.select_paged_tokens(w.q, w.kcache, w.page_table, w.pos, w.compress_ratio, w.k,
                                          row_req=w.row_req)
    with force_scorer("groups"), force_path("two_pass"):
        assert np.array_equal(gpu_select(d, w, 0), full)


GEOMETRIES = [
    # (compress_ratio, page_size): keys per page 16 (the benchmark), 24 (not a
    # power of two), 8, 1 (a page per key) and 64 (a stage spans half a page)
    (4, 64), (2, 48), (8, 64), (1, 4), (4, 256),
]


@pytest.mark.parametrize("cr,page_size", GEOMETRIES)
def test_geometries(oracle_mod, cr, page_size):
    """Other compress ratios and page sizes through every arm and both
    scorers: integer inputs, so scores and selections are bit-exact with the
    oracle; three requests of different lengths on a permuted page pool, k a
    multiple of cr, one request with fewer visible keys than k / cr."""
    rng = np.random.default_rng(60 + cr)
    k = 64 * cr
    w = W.build(f"geom_{cr}_{page_size}", rng, 60 + cr, [7000, 9 * cr, 3001], [40, 5, 37], permute_pages=True,
                integer=True, k=k, compress_ratio=cr, page_size=page_size, extra_pages=2)
    full_parity(oracle_mod, w, 0, True, paths=PATHS)
    full_parity(oracle_mod, w, KEYS, True, paths=("two_pass",))
    with force_scorer("groups"):
        full_parity(oracle_mod, w, 0, True, paths=("two_pass",))


def test_out_keys_reduced(oracle_mod):
    w = W.kernel_shape(rows=40, ctx=30_000)
    d = to_dev(w)
    V = visible(oracle_mod, w)
    gs = gpu_scores(d, w, 0)
    for path in PATHS:
        for k in (1, 7, 512, 2048, Q.QSA_MAX_SELECT):
            with force_path(path):
                out = gpu_select(d, w, KEYS, k=k)
            assert np.array_equal(out, expected_from_scores(oracle_mod, gs, V, k, 4, KEYS)), (path, k)


@pytest.mark.parametrize("flags", [0, RELU])
def test_interleaved_requests(oracle_mod, flags):
    """Rows of different requests in any order (not grouped by request), both
    score forms."""
    rng = np.random.default_rng(41)
    w = W.build("interleaved", rng, 41, [3000, 7000, 500, 12000], [30, 20, 5, 25], permute_pages=True,
                integer=True, k=256)
    perm = rng.permutation(w.rows)
    w.q, w.pos, w.row_req = np.ascontiguousarray(w.q[perm]), w.pos[perm].copy(), w.row_req[perm].copy()
    full_parity(oracle_mod, w, flags, True, paths=PATHS)


def test_edges(oracle_mod):
    """V = 0 rows, V below / equal / above the block budget, k = cr, a
    partial last page, rows = 1."""
    rng = np.random.default_rng(42)
    ctx = 64 * 7 + 13
    w = W.build("edges", rng, 42, [ctx], [1], permute_pages=True, integer=True, k=4 * 32)
    w.pos = np.array([ctx - 1], np.int32)
    cases = [0, 1, 2, 3, 4, 126, 127, 128, 129, 130, 131, 255, ctx - 1]
    w.q = np.repeat(w.q, len(cases), axis=0)
    w.pos = np.array(cases, np.int32)
    w.row_req = np.zeros(len(cases), np.int32)
    full_parity(oracle_mod, w, 0, True, paths=PATHS)
    for path in PATHS:
        for k in (4, 8):
            with force_path(path):
                out = gpu_select(to_dev(w), w, 0, k=k)
            exp = oracle_mod.select_paged_tokens(w.q, w.kcache, w.page_table, w.pos, 4, k)
            assert np.array_equal(out, exp), (path, k)
    one = W.build("one", rng, 43, [5000], [1], permute_pages=False, integer=True, k=2048)
    full_parity(oracle_mod, one, 0, True, paths=PATHS)


@pytest.mark.parametrize("flags", [0, RELU])
def test_tiles_without_keys(oracle_mod, flags):
    """Several requests (the scorer then shares each tile's own visible keys
    among its workgroups): a whole 128-row tile whose rows see no key at all,
    a tile mixing such rows with rows of a long context, and a short and a long
    request side by side; every arm, both score forms, integer inputs, end to
    end."""
    rng = np.random.default_rng(44)
    w = W.build("tiles", rng, 44, [20000, 300, 9000, 40], [128, 200, 70, 30], permute_pages=True, integer=True,
                k=2048)
    w.pos = w.pos.copy()
    w.pos[128:328] = np.arange(200) % 3          # request 1: positions 0..2, no visible key
    full_parity(oracle_mod, w, flags, True, paths=PATHS)


@pytest.mark.parametrize("flags", [0, RELU, KEYS])
@pytest.mark.parametrize("name", ["decode_small", "kernel_shape_80", "mixed_small"])
def test_stream_select_flag(oracle_mod, name, flags):
    """QSA_STREAM_SELECT (the caller's request for the streaming arm) takes
    that arm and returns the default arm's selection; a forced arm still wins."""
    w = REDUCED[name](False)
    d = to_dev(w)
    base = gpu_select(d, w, flags)
    out = gpu_select(d, w, flags | Q.QSA_STREAM_SELECT)
    assert Q.qsa_last_path() == "stream"
    assert np.array_equal(out, base)
    with force_path("two_pass"):
        again = gpu_select(d, w, flags | Q.QSA_STREAM_SELECT)
        assert Q.qsa_last_path() == "two_pass"
    assert np.array_equal(again, base)


def test_stream_merge_beyond_registers(oracle_mod):
    """Streaming arm: rows whose chunk lists exceed the merge's registers
    (kb = 4,096 with QSA_OUT_KEYS and more than six 8,192-key chunks, so the
    merge cuts the lists down in LDS), beside a row whose last chunk is
    shorter than kb; integer inputs (many ties), compared with the oracle's
    selector on the GPU's own scores, and end to end for one case."""
    rng = np.random.default_rng(91)
    # 100,000, 60,000 (two rows) and 8,250 visible keys
    w = W.build("stream_long", rng, 91, [400_000, 240_000, 33_000], [1, 2, 1], permute_pages=True, integer=True,
                k=4096)
    d = to_dev(w)
    V = visible(oracle_mod, w)
    gs = gpu_scores(d, w, 0)
    for flags, k in ((KEYS, 4096), (0, 4096), (KEYS, 1000)):
        with force_path("stream"):
            out = gpu_select(d, w, flags, k=k)
        assert Q.qsa_last_path() == "stream"
        assert np.array_equal(out, expected_from_scores(oracle_mod, gs, V, k, w.compress_ratio, flags)), (flags, k)
    full = oracle_mod.select_paged_tokens(w.q, w.kcache, w.page_table, w.pos, w.compress_ratio, 4096,
                                          row_req=w.row_req, flags=KEYS)
    with force_path("stream"):
        assert np.array_equal(gpu_select(d, w, KEYS, k=4096), full)


@pytest.mark.parametrize("name,path", [("kernel_shape_80", "fused"), ("decode_small", "two_pass"),
                                       ("mixed_small", "fused_fallback"), ("decode_small", "stream")])
def test_graph_capture(oracle_mod, name, path):
    """The whole call captured in a HIP graph (the pages name graph capture as a
    failure site of their cooperative selector): every replay, with eager work
    and synchronisations between replays, equals the eager result."""
    w = REDUCED[name](False)
    d = to_dev(w)
    mv = int(visible(oracle_mod, w).max())
    with force_path(path):  # the workspace query follows the forced arm
        need = Q.qsa_select_paged_tokens_workspace_size(w.rows, w.num_reqs, mv, w.compress_ratio, w.k)
        ws = torch.empty(max(need, 1), dtype=torch.uint8, device=DEV)
        call = lambda out: Q.qsa_select_paged_tokens(d["q"], d["kcache"], d["page_table"], d["pos"],  # noqa: E731
                                                     w.compress_ratio, w.k, row_req=d["row_req"],
                                                     max_visible=mv, out=out, workspace=ws)
        eager = torch.empty((w.rows, w.k), dtype=torch.int32, device=DEV)
        call(eager)
        torch.cuda.synchronize()
        exp = eager.cpu().numpy()
        out = torch.empty_like(eager)
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            call(out)
        torch.cuda.current_stream().wait_stream(side)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            call(out)
        for i in range(4):
            out.fill_(-7)
            g.replay()
            torch.cuda.synchronize()
            assert np.array_equal(out.cpu().numpy(), exp), (name, path, i)
            call(eager)  # eager work on the same workspace between replays
            torch.cuda.synchronize()
            assert np.array_equal(eager.cpu().numpy(), exp), (name, path, i)


def test_golden_fixture_on_gpu():
    from conftest import golden_arrays, load_golden
    g = load_golden("paged_ties_expand.json")
    q, kc, pt, pos = golden_arrays(g)
    d = dict(q=torch.from_numpy(q).to(DEV), kcache=torch.from_numpy(kc).to(DEV),
             page_table=torch.from_numpy(pt).to(DEV), pos=torch.from_numpy(pos).to(DEV))
    cr = g["compress_ratio"]
    import oracle
    mv = max(oracle.visible_keys(int(p), cr) for p in pos)
    sel = lambda k, flags=0: Q.qsa_select_paged_tokens(d["q"], d["kcache"], d["page_table"], d["pos"], cr, k,  # noqa: E731
                                                       max_visible=mv, flags=flags)
    assert sel(g["k"]).cpu().numpy().tolist() == g["expected_tokens"]
    assert sel(g["k"], RELU).cpu().numpy().tolist() == g["expected_tokens_relu"]
    assert sel(g["k_keys"], KEYS).cpu().numpy().tolist() == g["expected_keys"]
    s = Q.qsa_score_paged(d["q"], d["kcache"], d["page_table"], d["pos"], cr, max_visible=mv)
    assert s[0, :16].cpu().numpy().tolist() == g["expected_scores_row0_first16"]


@pytest.mark.parametrize("path", ["two_pass", "fused"])
def test_determinism(path):
    w = W.kernel_shape(rows=130, ctx=60_000)
    d = to_dev(w)
    with force_path(path):
        outs = [gpu_select(d, w, 0) for _ in range(3)]
    side = torch.cuda.Stream()
    with force_path(path), torch.cuda.stream(side):
        o = Q.qsa_select_paged_tokens(d["q"], d["kcache"], d["page_table"], d["pos"], 4, w.k,
                                      max_visible=max_visible(w), row_req=d["row_req"])
    side.synchronize()
    outs.append(o.cpu().numpy())
    for o in outs[1:]:
        assert np.array_equal(o, outs[0])
    assert Q.qsa_last_path() != ""


# ------------------------------------------------------------ selector alone

def run_topk(scores_np, V, k, max_visible=None):
    s = torch.from_numpy(scores_np).to(DEV)
    vis = torch.from_numpy(np.asarray(V, np.int32)).to(DEV)
    out = Q.qsa_topk_rows(s, k, visible=vis, max_visible=max_visible)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def test_topk_rows_random_with_ties(oracle_mod):
    rng = np.random.default_rng(51)
    # (also 512-key rows with k above V, one-key rows, and k = 1)
    for trial, (rows, ld, k) in enumerate([(37, 300, 17), (16, 5000, 512), (9, 20_000, 2048),
                                           (5, 9000, Q.QSA_MAX_SELECT), (64, 70, 64), (48, 512, 600),
                                           (7, 1, 3), (40, 512, 1)]):
        kind = trial % 3
        if kind == 0:
            sc = rng.integers(-3, 4, size=(rows, ld)).astype(np.float32)
        elif kind == 1:
            sc = rng.standard_normal((rows, ld)).astype(np.float32)
        else:
            sc = rng.choice(np.array([-0.0, 0.0, 1.5, -2.0, 7.0], np.float32), size=(rows, ld))
        V = rng.integers(0, ld + 1, size=rows).astype(np.int32)
        V[0] = ld
        out = run_topk(sc, V, k, max_visible=ld)
        assert np.array_equal(out, oracle_mod.select_rows(sc, V, k)), (rows, ld, k)


def test_topk_rows_stress_row(oracle_mod):
    """A row of 106,861 scores with k = 2,048: the stress shape of the Turing
    PR's "Test Result"; no selected value may be below an unselected one."""
    rng = np.random.default_rng(52)
    n, k = 106_861, 2048
    sc = (rng.standard_normal((1, n)) * 100).astype(np.float32)
    sc[0, rng.integers(0, n, 5000)] = 3.0        # a block of exact ties near the middle
    out = run_topk(sc, [n], k)[0]
    assert np.array_equal(out, oracle_mod.select_rows(sc, np.array([n], np.int32), k)[0])
    sel = np.zeros(n, bool)
    sel[out] = True
    assert sc[0, sel].min() >= sc[0, ~sel].max()


def test_topk_rows_all_equal(oracle_mod):
    """More copies of the cutoff key than fit in LDS: the index-ordered path."""
    n, k = 50_000, Q.QSA_MAX_SELECT
    sc = np.full((2, n), 0.25, np.float32)
    sc[1, 7] = 1.0
    sc[1, 40_000] = 1.0
    out = run_topk(sc, [n, n], k)
    assert np.array_equal(out[0], np.arange(k))
    assert np.array_equal(out, oracle_mod.select_rows(sc, np.array([n, n], np.int32), k))


@pytest.mark.parametrize("kind", ["gauss", "ints", "few_values"])
def test_topk_rows_few_long(oracle_mod, kind):
    """A few long rows: lengths at, around and between multiples of the
    workgroup's 512 threads, rows shorter than k, an empty row, and tie-heavy
    scores (crowded histogram bins)."""
    rng = np.random.default_rng({"gauss": 61, "ints": 62, "few_values": 63}[kind])
    rows, ld = 9, 60_000
    if kind == "gauss":
        sc = rng.standard_normal((rows, ld)).astype(np.float32)
    elif kind == "ints":
        sc = rng.integers(-3, 4, size=(rows, ld)).astype(np.float32)
    else:
        sc = rng.choice(np.array([-0.0, 0.0, 1.5, 7.0], np.float32), size=(rows, ld))
    V = np.array([ld, 4096, 4097, 8192, 12_345, 300, 0, 59_999, 20_000], np.int32)
    for k in (512, 1024, 37):
        out = run_topk(sc, V, k, max_visible=ld)
        assert np.array_equal(out, oracle_mod.select_rows(sc, V, k)), (kind, k)


def test_topk_rows_repeated_calls(oracle_mod):
    """Rows of 16k..40k scores (the sampled-bound path, whose survivors are
    stored at per-thread places and read by other waves after a barrier),
    256 rows so that every compute unit holds one: twenty calls in a row, each
    equal to the oracle's selection."""
    rng = np.random.default_rng(54)
    rows, ld, k = 256, 40_000, 2048
    sc = rng.standard_normal((rows, ld)).astype(np.float32)
    sc[:, rng.integers(0, ld, 300)] = 2.25          # ties near the cut of most rows
    V = rng.integers(16_000, ld + 1, size=rows).astype(np.int32)
    exp = oracle_mod.select_rows(sc, V, k)
    s = torch.from_numpy(sc).to(DEV)
    vis = torch.from_numpy(V).to(DEV)
    for it in range(20):
        out = Q.qsa_topk_rows(s, k, visible=vis, max_visible=ld)
        torch.cuda.synchronize()
        assert np.array_equal(out.cpu().numpy(), exp), f"call {it}"


def test_topk_rows_visible_none(oracle_mod):
    rng = np.random.default_rng(53)
    sc = rng.standard_normal((7, 6000)).astype(np.float32)
    s = torch.from_numpy(sc).to(DEV)
    out = Q.qsa_topk_rows(s, 100).cpu().numpy()
    assert np.array_equal(out, oracle_mod.select_rows(sc, np.full(7, 6000, np.int32), 100))


# ------------------------------------------------------------ full sizes

def sampled_parity(oracle_mod, w, flags, integer, sample_rows, paths=(None,)):
    """Full-size launch (the configuration the benchmark times): the oracle
    scores a sample of rows one by one; the GPU selection over every row is
    checked against the oracle's selector on the GPU's own scores."""
    d = to_dev(w)
    V = visible(oracle_mod, w)
    gs = gpu_scores(d, w, flags)
    rows = sorted(set(int(r) for r in sample_rows))
    ref = oracle_mod.score_paged(w.q[rows], w.kcache, w.page_table, w.pos[rows], w.compress_ratio,
                                 row_req=w.row_req[rows], flags=flags & RELU)
    worst = assert_scores(gs, ref, V, exact=integer, rows=rows)
    exp = expected_from_scores(oracle_mod, gs, V, w.k, w.compress_ratio, flags)
    out = None
    for path in paths:
        with force_path(path):
            out = gpu_select(d, w, flags)
        assert np.array_equal(out, exp), f"{w.name} full, path={path}"
    note(f"{w.name} full: rows={w.rows} sumV={int(V.sum())} sampled={len(rows)} max_rel_err={worst:.2e}")
    return out


def _spread(n_rows, n, seed):
    """n distinct rows spread over the batch (seeded), with both ends."""
    rng = np.random.default_rng(seed)
    return sorted(set([0, n_rows - 1] + list(rng.choice(n_rows, size=min(n, n_rows), replace=False))))


@pytest.mark.parametrize("flags", [0, RELU])
def test_full_kernel_shape(oracle_mod, flags):
    """The benchmark's kernel shape in both score forms: 64 sampled rows
    (with the tile edges) scored by the oracle; every row's selection checked
    in the fused arm, the two-pass arm and the fused arm's exact recompute
    path."""
    w = W.kernel_shape()
    rows = sorted(set(_spread(w.rows, 56, 5) + [63, 64, 127, 128, 1535, 1536, 1599, 1600]))
    sampled_parity(oracle_mod, w, flags, False, rows, paths=(None, "two_pass", "fused_fallback", "fused_redo", "stream"))


def test_full_tie_stress(oracle_mod):
    w = W.tie_stress()
    d = to_dev(w)
    full = oracle_mod.select_paged_tokens(w.q, w.kcache, w.page_table, w.pos, 4, w.k)
    for path in (None, "two_pass", "fused", "stream"):
        with force_path(path):
            out = gpu_select(d, w, 0)
        assert np.array_equal(out, full), path


@pytest.mark.parametrize("flags", [0, RELU])
def test_full_mixed(oracle_mod, flags):
    """Mixed batch in both score forms: each request's first and last row
    and 32 more sampled rows; every row's selection in both arms."""
    w = W.mixed()
    starts = np.concatenate([[0], np.cumsum(np.bincount(w.row_req))])
    sample = sorted(set(list(starts[:-1]) + list(starts[1:] - 1) + _spread(w.rows, 32, 6)))
    sampled_parity(oracle_mod, w, flags, False, sample, paths=(None, "two_pass", "fused", "stream"))


@pytest.mark.parametrize("name", ["long_1", "long_8"])
def test_full_long_few(oracle_mod, name):
    """One and eight 184k-token requests with one row each."""
    w = W.make(name)
    sampled_parity(oracle_mod, w, 0, False, [0, w.rows - 1], paths=(None, "fused", "stream"))


@pytest.mark.slow
@pytest.mark.parametrize("flags", [0, RELU])
def test_full_decode(oracle_mod, flags):
    """Decode batch in both score forms: every row's scores against the
    oracle, and every row's selection in both arms."""
    w = W.decode()
    sampled_parity(oracle_mod, w, flags, False, list(range(w.rows)), paths=(None, "fused", "stream"))
