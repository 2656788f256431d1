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
