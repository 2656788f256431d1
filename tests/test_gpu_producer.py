"""The compressed-key producer (qsa_compress_keys) against its CPU oracle
(oracle/producer.py): a sequence of calls (prefill chunks that end inside a
block, decode steps of several requests in one call, mixed calls) builds the
side cache, which must then hold the oracle's key in every slot of a
finished block and be untouched everywhere else.

Tolerance, from the arithmetic: the token keys are fp16 and exact in the
float64 oracle; the GPU pools, normalises and rotates in fp32 (rotation
angles reduced modulo 2 pi in fp64 first), an error of a few fp32 ulps of
the key's largest value M, then rounds once to fp16.  Each stored value is
therefore within half an fp16 ulp of the oracle's value plus 4e-6 * M (plus
half the fp16 subnormal spacing).  A wrong pair, sign, angle or slot gives
errors of order M.
"""
import numpy as np
import pytest
import torch

import workloads as W
from oracle import producer as OP
from paged_block_scoring_amd import qsa as Q

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
D = 128
SENTINEL = 0x7C01  # an fp16 NaN pattern the producer never writes


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def ulp16(x):
    ax = np.abs(x)
    e = np.floor(np.log2(np.maximum(ax, 2.0 ** -14)))
    return 2.0 ** (e - 10)


def run_calls(calls, keys, w, pt, pool, cr, page_size, *, rope_dim, base, interleaved, eps, seed=0,
              pos_offset=0):
    """Runs each call (a list of (request, start, end) token runs) through the
    producer; returns the side cache as float16 numpy."""
    kpp = page_size // cr
    kc = torch.full((pool, kpp, D), SENTINEL, dtype=torch.int16, device=DEV).view(torch.float16)
    state = None
    if cr > 1:
        garbage = np.random.default_rng(seed + 99).standard_normal((pt.shape[0], cr, D)).astype(np.float16)
        state = dev(garbage)
    w_d = dev(w) if w is not None else None
    pt_d = dev(pt)
    for call in calls:
        k_tok = np.concatenate([keys[q][a:b] for q, a, b in call]) if call else np.zeros((0, D), np.float16)
        req = np.concatenate([np.full(b - a, q, np.int32) for q, a, b in call]) if call else np.zeros(0, np.int32)
        pos = np.concatenate([np.arange(a, b, dtype=np.int64) + pos_offset for q, a, b in call]).astype(np.int32) \
            if call else np.zeros(0, np.int32)
        print(f"producer call: {len(call)} runs, {k_tok.shape[0]} tokens", flush=True)
        Q.qsa_compress_keys(dev(k_tok), dev(pos), state, kc, pt_d, cr, tok_req=dev(req), norm_w=w_d, eps=eps,
                            rope_dim=rope_dim, rope_base=base, interleaved=interleaved)
    torch.cuda.synchronize()
    return kc.cpu().numpy()


def check(kc, stored, sample=None):
    """Every oracle slot within the tolerance; with sample=None, every other
    slot still holds the sentinel."""
    bits = kc.view(np.uint16)
    if sample is None:
        untouched = np.ones(bits.shape[:2], dtype=bool)
        for page, slot in stored:
            untouched[page, slot] = False
        assert np.all(bits[untouched] == SENTINEL), "the producer wrote a slot of an unfinished block"
    items = list(stored.items()) if sample is None else [(k, stored[k]) for k in sample]
    worst = 0.0
    for (page, slot), ref in items:
        got = kc[page, slot].astype(np.float64)
        M = np.abs(ref).max()
        tol = 0.5 * ulp16(ref) + 4e-6 * M + 2.0 ** -25
        err = np.abs(got - ref)
        assert np.all(err <= tol), ((page, slot), float(err.max()), int(np.argmax(err - tol)))
        worst = max(worst, float((err / ulp16(ref)).max()))
    return worst


def scenario_calls():
    # five requests; runs end inside blocks, decode steps of several requests
    # per call (not in request order), and a long final chunk
    calls = [[(0, 0, 131), (1, 0, 7)],
             [(0, 131, 133), (2, 0, 64), (3, 0, 3)],
             [(1, 7, 150), (4, 0, 997)]]
    for s in range(9):
        step = [(4, 997 + s, 998 + s)] if 997 + s < 1000 else []
        step += [(0, 133 + s, 134 + s), (1, 150 + s, 151 + s)]
        calls.append(step)
    calls.append([(0, 142, 300)])
    consumed = [300, 159, 64, 3, 1000]
    return calls, consumed


@pytest.mark.parametrize("cr,page_size,rope_dim,interleaved,eps,with_w", [
    (4, 64, 128, False, 1e-6, True),
    (4, 64, 64, True, 1e-6, True),
    (4, 16, 16, False, 1e-5, False),
    (8, 64, 128, True, 1e-6, True),
    (2, 64, 0, False, 1e-6, True),
])
def test_call_sequence(cr, page_size, rope_dim, interleaved, eps, with_w):
    calls, consumed = scenario_calls()
    keys, w, pt, pool = W.raw_token_keys(11, consumed, page_size, cr)
    w = w if with_w else None
    kc = run_calls(calls, keys, w, pt, pool, cr, page_size, rope_dim=rope_dim, base=10000.0,
                   interleaved=interleaved, eps=eps)
    hist = [keys[q][:n] for q, n in enumerate(consumed)]
    stored = OP.produce(hist, pt, page_size, cr, w, eps, rope_dim, 10000.0, interleaved)
    assert len(stored) == sum(n // cr for n in consumed)
    worst = check(kc, stored)
    print(f"worst error {worst:.3f} fp16 ulp over {len(stored)} keys")


def test_ratio_one_needs_no_state():
    consumed = [50, 21]
    keys, w, pt, pool = W.raw_token_keys(12, consumed, 64, 1)
    calls = [[(0, 0, 40), (1, 0, 20)], [(1, 20, 21), (0, 40, 41)], [(0, 41, 50)]]
    kc = run_calls(calls, keys, w, pt, pool, 1, 64, rope_dim=128, base=500000.0, interleaved=False, eps=1e-6)
    stored = OP.produce(keys, pt, 64, 1, w, 1e-6, 128, 500000.0, False)
    check(kc, stored)


def test_ignored_tokens_and_short_page_table():
    # tokens of an unknown request or at a negative position write nothing;
    # blocks past the page table's width are dropped, the rest are stored
    cr, page_size = 4, 64                                      # 16 keys per page
    keys, w, pt, pool = W.raw_token_keys(13, [100, 8], page_size, cr)
    pt = np.ascontiguousarray(pt[:, :1])                       # one logical page: blocks 0..15
    junk = np.random.default_rng(5).standard_normal((3, D)).astype(np.float16)
    k_tok = np.concatenate([keys[0], keys[1], junk])
    req = np.array([0] * 100 + [1] * 8 + [-1, 2, 1], np.int32)
    pos = np.array(list(range(100)) + list(range(8)) + [3, 7, -1], np.int32)
    kc = torch.full((pool, page_size // cr, D), SENTINEL, dtype=torch.int16, device=DEV).view(torch.float16)
    state = torch.zeros((2, cr, D), dtype=torch.float16, device=DEV)
    Q.qsa_compress_keys(dev(k_tok), dev(pos), state, kc, dev(pt), cr, tok_req=dev(req), norm_w=dev(w))
    torch.cuda.synchronize()
    stored = OP.produce([keys[0][:64], keys[1]], pt, page_size, cr, w)
    check(kc.cpu().numpy(), stored)


def test_positions_near_int32_max():
    # a run starting at a block boundary just below 2^31: rotation angles up
    # to 2e9 radians must keep their accuracy
    cr, kpp = 4, 1 << 14
    page_size = cr * kpp
    p0 = (1 << 31) - 256
    n = 250                                                    # last position 2^31 - 7
    rng = np.random.default_rng(14)
    keys = rng.standard_normal((n, D)).astype(np.float16)
    w = rng.uniform(0.5, 1.5, D).astype(np.float32)
    c0 = p0 // cr
    lp = c0 // kpp
    pt = np.zeros((1, lp + 2), np.int32)
    pt[0, lp] = 1
    pt[0, lp + 1] = 2
    kc = run_calls([[(0, 0, n)]], [keys], w, pt, 3, cr, page_size, rope_dim=128, base=10000.0,
                   interleaved=False, eps=1e-6, pos_offset=p0)
    stored = {}
    for i in range(n // cr):
        c = c0 + i
        stored[(int(pt[0, c // kpp]), c % kpp)] = OP.compress_block(keys[cr * i: cr * i + cr], c, cr, w, 1e-6, 128)
    worst = check(kc, stored)
    print(f"worst error {worst:.3f} fp16 ulp at positions near 2^31")


def test_full_prompt_184k_then_decode():
    # one 184,003-token prompt in one call (46,000 blocks, 3 tokens left
    # open), then the decode token that finishes block 46,000 from the
    # staging state; checked on a sample of blocks and by counting writes
    n = 184_003
    cr, page_size = 4, 64
    keys, w, pt, pool = W.raw_token_keys(15, [n + 1], page_size, cr)
    kc = run_calls([[(0, 0, n)], [(0, n, n + 1)]], keys, w, pt, pool, cr, page_size, rope_dim=128,
                   base=10000.0, interleaved=False, eps=1e-6)
    kpp = page_size // cr
    written = int(np.any(kc.view(np.uint16) != SENTINEL, axis=2).sum())
    assert written == (n + 1) // cr
    rng = np.random.default_rng(16)
    blocks = sorted(set(rng.choice((n + 1) // cr, 400, replace=False).tolist()) | {0, 45_999, 46_000})
    stored = {}
    for c in blocks:
        stored[(int(pt[0, c // kpp]), c % kpp)] = OP.compress_block(keys[0][cr * c: cr * c + cr], c, cr, w)
    check(kc, stored, sample=list(stored))
