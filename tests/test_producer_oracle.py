"""Pins of the compressed-key producer's CPU oracle (oracle/producer.py)
against closed forms and invariances of its readings: mean pooling, RMSNorm,
RoPE at the block-start position, and the slot a block lands in.  The pages fix
none of these numerically (parity unpinned with respect to the pages); each
test below fails for a plausible slip in the oracle (a wrong rotation sign, a
frequency exponent off by a factor, block end instead of block start, a pair
mismatch, a dropped eps or weight, a wrong slot)."""
import numpy as np
import pytest

from oracle import producer as P

D = 128


def _rng(seed=0):
    return np.random.default_rng(seed)


def test_rotation_sign_and_block_start():
    # Only pair (0, 1) rotates, at frequency 1, so the angle is the position
    # itself: block 1 of ratio 4 starts at token 4 (not 7, its last token).
    keys = np.zeros((4, D))
    keys[:, 0] = 0.5
    out = P.compress_block(keys, block=1, ratio=4, eps=0.0, rope_dim=2)
    norm = np.sqrt(D)  # e0 normalised to rms 1 over 128 values
    want = np.zeros(D)
    want[0], want[1] = norm * np.cos(4.0), norm * np.sin(4.0)
    np.testing.assert_allclose(out, want, rtol=0, atol=1e-12)
    # e1 turns the same way: (0, 1) -> (-sin, cos).
    x = np.zeros(D)
    x[1] = 1.0
    y = P.rope(x, 4, rope_dim=2)
    np.testing.assert_allclose(y[:2], [-np.sin(4.0), np.cos(4.0)], atol=1e-15)


@pytest.mark.parametrize("interleaved", [False, True])
def test_frequency_exponent(interleaved):
    # rope_dim 4, base 100: pair 0 at frequency 1, pair 1 at 100^(-2/4) = 0.1.
    # At p0 = 10 the second pair turns by exactly 1 radian.
    ia, ib = (2, 3) if interleaved else (1, 3)
    x = np.zeros(D)
    x[ia] = 1.0
    y = P.rope(x, 10, rope_dim=4, base=100.0, interleaved=interleaved)
    want = np.zeros(D)
    want[ia], want[ib] = np.cos(1.0), np.sin(1.0)
    np.testing.assert_allclose(y, want, atol=1e-15)
    # pair 0 at frequency 1: angle 10
    ja, jb = (0, 1) if interleaved else (0, 2)
    x = np.zeros(D)
    x[ja] = 1.0
    y = P.rope(x, 10, rope_dim=4, base=100.0, interleaved=interleaved)
    assert y[ja] == pytest.approx(np.cos(10.0), abs=1e-15)
    assert y[jb] == pytest.approx(np.sin(10.0), abs=1e-15)


@pytest.mark.parametrize("interleaved", [False, True])
@pytest.mark.parametrize("rope_dim", [16, 64, 128])
def test_rope_relative_position_and_norm(interleaved, rope_dim):
    rng = _rng(1)
    a, b = rng.standard_normal(D), rng.standard_normal(D)
    p, s = 37, 1_000
    kw = dict(rope_dim=rope_dim, base=10000.0, interleaved=interleaved)
    d1 = P.rope(a, p + s, **kw) @ P.rope(b, s, **kw)
    d0 = P.rope(a, p, **kw) @ P.rope(b, 0, **kw)
    assert d1 == pytest.approx(d0, rel=1e-10, abs=1e-10)
    # position 0 is the identity; every position keeps the norm and leaves
    # the values past rope_dim alone
    np.testing.assert_array_equal(P.rope(a, 0, **kw), a)
    y = P.rope(a, 184_003, **kw)
    assert np.linalg.norm(y) == pytest.approx(np.linalg.norm(a), rel=1e-12)
    np.testing.assert_array_equal(y[rope_dim:], a[rope_dim:])


def test_rotate_half_and_interleaved_are_one_permutation_apart():
    rng = _rng(2)
    rd, half = 64, 32
    xh = rng.standard_normal(D)
    perm = np.arange(D)
    perm[0:rd:2] = np.arange(half)         # interleaved slot 2i holds rotate-half value i
    perm[1:rd:2] = np.arange(half, rd)     # slot 2i+1 holds value i + half
    xi = xh[perm]
    yh = P.rope(xh, 1234, rope_dim=rd, interleaved=False)
    yi = P.rope(xi, 1234, rope_dim=rd, interleaved=True)
    np.testing.assert_allclose(yi, yh[perm], atol=1e-12)


def test_rms_norm_properties():
    rng = _rng(3)
    x = rng.standard_normal(D) * 3.0
    y = P.rms_norm(x, eps=0.0)
    assert np.mean(y * y) == pytest.approx(1.0, rel=1e-13)
    np.testing.assert_allclose(P.rms_norm(7.5 * x, eps=0.0), y, rtol=1e-13)
    ms = np.mean(x * x)
    eps = 0.25
    assert np.mean(P.rms_norm(x, eps=eps) ** 2) == pytest.approx(ms / (ms + eps), rel=1e-13)
    w = rng.uniform(0.5, 1.5, D)
    np.testing.assert_allclose(P.rms_norm(x, w, eps=eps), w * P.rms_norm(x, eps=eps), rtol=1e-14)


def test_mean_pool_properties():
    rng = _rng(4)
    k = rng.standard_normal(D)
    np.testing.assert_allclose(P.mean_pool(np.stack([k] * 4)), k, rtol=1e-15)
    keys = rng.standard_normal((4, D))
    np.testing.assert_allclose(P.mean_pool(keys[::-1]), P.mean_pool(keys), rtol=0, atol=1e-14)
    # the mean of a constant shift moves by that shift
    np.testing.assert_allclose(P.mean_pool(keys + 2.0), P.mean_pool(keys) + 2.0, rtol=0, atol=1e-14)
    # the mean lies inside the range of the tokens, value by value
    m = P.mean_pool(keys)
    assert np.all(m <= keys.max(axis=0) + 1e-15) and np.all(m >= keys.min(axis=0) - 1e-15)


def test_produce_places_complete_blocks_only():
    rng = _rng(5)
    ratio, page_size = 4, 8          # two compressed keys per page
    page_table = np.array([[5, 2, 9], [7, 1, 3]])
    hist = [rng.standard_normal((10, D)), rng.standard_normal((3, D))]
    stored = P.produce(hist, page_table, page_size, ratio)
    # request 0: tokens 0..9 complete blocks 0 and 1 (closing at positions 3
    # and 7), both on its first logical page (physical 5); block 2 is open.
    # request 1 has no complete block.
    assert sorted(stored) == [(5, 0), (5, 1)]
    np.testing.assert_array_equal(stored[(5, 1)], P.compress_block(hist[0][4:8], 1, ratio))
    # a third page-worth: 20 tokens -> blocks 0..4, block 2 on logical page 1
    hist = [rng.standard_normal((20, D)), np.zeros((0, D))]
    stored = P.produce(hist, page_table, page_size, ratio)
    assert sorted(stored) == [(2, 0), (2, 1), (5, 0), (5, 1), (9, 0)]
