"""Host model of the row-tiled scorer's work split: which page-table entries
a launch reads.

The kernel cuts every tile's logical keys into 8 XCD stripes padded to whole
32-key stages and hands each workgroup an equal run of (tile, key) positions,
processed as pieces of at most 2,048 keys; each piece builds a slot table
from the page table.  The public contract is that a request's page-table
entries at or beyond ceil(V / keys_per_page) of its longest row are never
read.  This model follows the single-request split of the launcher and
kernel (the multi-request split bounds each piece by its tile's visible
count) and checks the largest page-table index read for every workload and
for the strides the sampling pass uses.  CPU only.
"""
import numpy as np
import pytest

import workloads as W

XCDS, STEP, PIECE, TILE = 8, 32, 2048, 128


def ceil_div(a, b):
    return -(-a // b)


def largest_page_read(rows, max_visible, stride, kpp, cus=256, clamp=True):
    lmax = ceil_div(max_visible, stride)
    tiles = ceil_div(rows, TILE)
    stripe = ceil_div(ceil_div(lmax, XCDS), STEP) * STEP
    positions = tiles * stripe
    per_xcd = (cus // XCDS) * 2
    seg = ceil_div(ceil_div(positions, per_xcd), STEP) * STEP
    seg = max(seg, 64)
    per_xcd = ceil_div(positions, seg)
    worst = -1
    for xcd in range(XCDS):
        xk0 = xcd * stripe
        span = min(stripe, ceil_div(lmax - xk0, STEP) * STEP)
        if span <= 0:
            continue
        total = tiles * span
        for loc in range(per_xcd):
            p, pend = loc * seg, min(loc * seg + seg, total)
            while p < pend:
                tile = p // span
                off = p - tile * span
                n = min(span - off, pend - p, PIECE)
                c0 = xk0 + off
                end = min(c0 + n, lmax) if clamp else c0 + n
                if end > c0:
                    worst = max(worst, ((end - 1) * stride) // kpp)
                p += n
    return worst


def sampling_strides(max_visible):
    """The sampling pass's stride: 16, doubled until a row has at most 4,096 samples."""
    s = 16
    while ceil_div(max_visible, s) > 4096:
        s *= 2
    return s


CASES = {
    "tiny": lambda: W.tiny(),
    "kernel_shape_1616": lambda: W.kernel_shape(),
    "tie_stress": lambda: W.tie_stress(),
    "kernel_shape_80": lambda: W.kernel_shape(rows=80),
    "kernel_shape_130_60k": lambda: W.kernel_shape(rows=130, ctx=60_000),
}


@pytest.mark.parametrize("name", sorted(CASES))
def test_no_page_table_read_past_the_visible_pages(name):
    import oracle
    w = CASES[name]()
    kpp = w.page_size // w.compress_ratio
    mv = max(oracle.visible_keys(int(p), w.compress_ratio) for p in w.pos)
    bound = ceil_div(mv, kpp)            # entries 0 .. bound-1 may be read
    for stride in (1, sampling_strides(mv)):
        assert largest_page_read(w.rows, mv, stride, kpp) < bound, (name, stride)


def test_model_sees_the_unclamped_stage_padding():
    """Without the clamp to the last visible key, the stage-padded stripe end
    reaches past the table at the kernel shape (46,000 keys: stripes of 5,760
    keys, the last one padded): the model is sharp enough to catch that."""
    assert largest_page_read(1616, 46000, 1, 16, clamp=False) >= ceil_div(46000, 16)
    assert largest_page_read(1616, 46000, 16, 16, clamp=False) >= ceil_div(46000, 16)


# ---------------------------------------------------------------------------
# The balanced split used with several requests (TileShares in
# score_rows.hpp): each tile's own visible keys cut into 8 stripes padded to
# whole stages, this XCD's stripe of every tile laid end to end, the XCD's
# workgroups sharing that total evenly.  The default-form kernel uses it with
# 128-row tiles, 32-key stages and 2,048-key pieces; the relu-form kernel with
# 64-row tiles, 64-key stages and 1,024-key pieces.

def tile_counts(w, tile):
    """Largest visible-key count of each tile's rows (0 for rows past the end)."""
    import oracle
    v = np.array([oracle.visible_keys(int(p), w.compress_ratio) for p in w.pos], dtype=np.int64)
    tiles = ceil_div(w.rows, tile)
    pad = np.zeros(tiles * tile, dtype=np.int64)
    pad[:w.rows] = v
    return pad.reshape(tiles, tile).max(axis=1)


def balanced_pieces(tile_v, stride, step, piece, per):
    """Every piece (xcd, workgroup, tile, first key, length) of the balanced
    split, following the kernel's begin/piece steps."""
    def share(t, xcd):
        lv = ceil_div(int(tile_v[t]), stride)
        st = ceil_div(ceil_div(lv, XCDS), step) * step
        u = min(max(lv - xcd * st, 0), st)
        return ceil_div(u, step) * step, st

    out = []
    tiles = len(tile_v)
    for xcd in range(XCDS):
        shares = [share(t, xcd) for t in range(tiles)]
        total = sum(u for u, _ in shares)
        seg = max(step, ceil_div(ceil_div(total, per), step) * step)
        starts = np.concatenate([[0], np.cumsum([u for u, _ in shares])])
        for loc in range(per):
            p, pend = loc * seg, min(loc * seg + seg, total)
            if p >= pend:
                continue
            # the tile whose share holds p: exactly one tile with u > 0 qualifies
            hits = [t for t in range(tiles) if shares[t][0] > 0 and starts[t] <= p < starts[t] + shares[t][0]]
            assert len(hits) == 1
            t = hits[0]
            pbase, (ucur, st) = starts[t], shares[t]
            while p < pend:
                while p >= pbase + ucur:
                    pbase += ucur
                    t += 1
                    ucur, st = shares[t]
                off = p - pbase
                n = min(ucur - off, pend - p, piece)
                out.append((xcd, loc, t, xcd * st + off, n))
                p += n
    return out


@pytest.mark.parametrize("tile,step,piece", [(128, 32, 2048), (64, 64, 1024)])
@pytest.mark.parametrize("name", ["mixed", "three_reqs", "empty_tiles"])
def test_balanced_split_covers_every_visible_key_once(name, tile, step, piece):
    """Every visible logical key of every tile lies in exactly one piece, pieces
    start on stage boundaries and stay within their tile's stage-padded stripe,
    and no workgroup gets more than one stage above an even share."""
    rng = np.random.default_rng(7)
    if name == "mixed":
        w = W.mixed()
    elif name == "three_reqs":
        w = W.build("three", rng, 7, [5000, 300, 70000], [100, 150, 90], permute_pages=True, k=256)
    else:  # whole tiles of rows that see no key, between long ones
        w = W.build("empty", rng, 7, [20000, 300, 9000], [200, 260, 70], permute_pages=True, k=256)
        w.pos = w.pos.copy()
        w.pos[200:460] = np.arange(260) % 3
    tv = tile_counts(w, tile)
    per = (256 // XCDS) * 2
    for stride in (1, 16):
        pieces = balanced_pieces(tv, stride, step, piece, per)
        covered = {}
        work = {}
        for xcd, loc, t, c0, n in pieces:
            assert c0 % step == 0 and 0 < n <= piece, (xcd, loc, t, c0, n)
            lv = ceil_div(int(tv[t]), stride)
            st = ceil_div(ceil_div(lv, XCDS), step) * step
            assert xcd * st <= c0 and c0 + n <= (xcd + 1) * st, (xcd, t, c0, n, st)
            for j in range(c0, min(c0 + n, lv)):
                covered[(t, j)] = covered.get((t, j), 0) + 1
            work[(xcd, loc)] = work.get((xcd, loc), 0) + n
        for t in range(len(tv)):
            lv = ceil_div(int(tv[t]), stride)
            assert all(covered.get((t, j), 0) == 1 for j in range(lv)), (name, stride, t)
        for xcd in range(XCDS):
            loads = [n for (x, _), n in work.items() if x == xcd]
            if loads:
                mean = sum(loads) / per
                assert max(loads) <= mean + 2 * step, (name, stride, xcd, max(loads), mean)
