"""Pins for the oracle's token orders (cuboid tiling) and window r* on them (CPU only).

The storage order is checked against hand-worked fixtures, against the
frame-major order in the cases where both agree, and against its structural
properties (a bijection; every full block an exact ct x ch x cw box, stored
frame-major).  Window r* on a cuboid order is checked against hand-worked
values and against the closed form for two boxes, which does not go through
token coordinates at all.
"""

import json
import os

import numpy as np
import pytest

from oracle import layout as ol
from oracle import masks as om

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _load():
    with open(os.path.join(GOLDEN, "cuboid_layout_hand_cases.json")) as f:
        return json.load(f)


CASES = _load()


@pytest.mark.parametrize("case", CASES["orders"], ids=lambda c: c["name"])
def test_order_hand_cases(case):
    o = ol.cuboid_order(case["T"], case["H"], case["W"], case["cuboid"])
    assert o.tolist() == case["order"]


@pytest.mark.parametrize("case", CASES["rstar"], ids=lambda c: c["name"])
def test_rstar_hand_cases(case):
    o = ol.cuboid_order(case["T"], case["H"], case["W"], case["cuboid"])
    rs = om.window_rstar_bruteforce(case["T"], case["H"], case["W"], case["block"], case["t_window"], order=o)
    rs = np.where(rs >= om.RSTAR_INF, -1, rs)
    assert rs.tolist() == case["rstar"]


GRIDS = [
    (21, 30, 52, (4, 4, 4)), (21, 30, 52, (1, 8, 8)), (21, 30, 52, (2, 4, 8)), (21, 30, 52, (1, 4, 16)),
    (41, 45, 80, (2, 8, 8)), (41, 45, 80, (1, 8, 16)), (5, 10, 14, (2, 4, 8)), (3, 7, 5, (2, 2, 2)),
    (4, 6, 9, (3, 2, 2)), (2, 3, 3, (4, 4, 4)),
]


@pytest.mark.parametrize("grid", GRIDS, ids=str)
def test_order_is_a_permutation(grid):
    T, H, W, cub = grid
    o = ol.cuboid_order(T, H, W, cub)
    assert o.size == T * H * W
    np.testing.assert_array_equal(np.sort(o), np.arange(T * H * W))


@pytest.mark.parametrize("grid", GRIDS, ids=str)
def test_full_blocks_are_boxes(grid):
    """Each of the first F blocks is one full cuboid, aligned to the cuboid grid, stored frame-major."""
    T, H, W, (ct, ch, cw) = grid
    blk = ct * ch * cw
    o = ol.cuboid_order(T, H, W, (ct, ch, cw))
    F = (T // ct) * (H // ch) * (W // cw)
    t, y, x = ol.slot_coords(T, H, W, o)
    prev = None
    for j in range(F):
        s = slice(j * blk, (j + 1) * blk)
        tj, yj, xj = t[s], y[s], x[s]
        t0, y0, x0 = tj.min(), yj.min(), xj.min()
        assert (t0 % ct, y0 % ch, x0 % cw) == (0, 0, 0)
        dt, dy, dx = np.meshgrid(np.arange(ct), np.arange(ch), np.arange(cw), indexing="ij")
        np.testing.assert_array_equal(tj, t0 + dt.reshape(-1))
        np.testing.assert_array_equal(yj, y0 + dy.reshape(-1))
        np.testing.assert_array_equal(xj, x0 + dx.reshape(-1))
        key = (t0 // ct, y0 // ch, x0 // cw)
        assert prev is None or key > prev  # lexicographic cuboid order
        prev = key
    # every later slot belongs to a partial cuboid
    tail = slice(F * blk, None)
    a, b, c = t[tail] // ct, y[tail] // ch, x[tail] // cw
    partial = (((a + 1) * ct > T) | ((b + 1) * ch > H) | ((c + 1) * cw > W))
    assert partial.all()


@pytest.mark.parametrize("T,H,W,cub", [(3, 5, 7, (1, 1, 7)), (21, 30, 52, (1, 1, 52)), (4, 6, 4, (1, 2, 4)),
                                       (2, 8, 8, (1, 8, 8)), (3, 4, 5, (3, 4, 5)), (5, 3, 2, (1, 3, 2))])
def test_whole_row_cuboids_give_frame_major_order(T, H, W, cub):
    """Cuboids spanning whole rows (ch | H, cw = W) tile the grid in frame-major order."""
    np.testing.assert_array_equal(ol.cuboid_order(T, H, W, cub), np.arange(T * H * W))


def test_raster_is_identity():
    np.testing.assert_array_equal(ol.cuboid_order(3, 4, 5, None), np.arange(60))
    np.testing.assert_array_equal(ol.cuboid_order(3, 4, 5, (0, 0, 0)), np.arange(60))


def _box_gap(lo_a, hi_a, lo_b, hi_b):
    return max(0, lo_b - hi_a, lo_a - hi_b)


@pytest.mark.parametrize("grid,tw", [((21, 30, 52, (4, 4, 4)), 1), ((21, 30, 52, (1, 8, 8)), 2),
                                     ((41, 45, 80, (2, 8, 8)), 1), ((5, 10, 14, (2, 4, 8)), 0)], ids=str)
def test_rstar_full_blocks_closed_form(grid, tw):
    """r* of two full cuboid blocks = max(y gap, x gap) of the boxes when their frame gap is <= Tw."""
    T, H, W, (ct, ch, cw) = grid
    blk = ct * ch * cw
    o = ol.cuboid_order(T, H, W, (ct, ch, cw))
    Ft, Fy, Fx = T // ct, H // ch, W // cw
    F = Ft * Fy * Fx
    rng = np.random.default_rng(11)
    qbs = sorted(set(rng.integers(0, F, size=6).tolist()) | {0, F - 1})
    rs = om.window_rstar_bruteforce(T, H, W, blk, tw, qblocks=qbs, order=o)

    def box(j):
        a, r = divmod(j, Fy * Fx)
        b, c = divmod(r, Fx)
        return (a * ct, a * ct + ct - 1), (b * ch, b * ch + ch - 1), (c * cw, c * cw + cw - 1)

    for r, qb in enumerate(qbs):
        (qt, qy, qx) = box(qb)
        for kb in range(F):
            kt, ky, kx = box(kb)
            if _box_gap(*qt, *kt) > tw:
                want = om.RSTAR_INF
            else:
                want = max(_box_gap(*qy, *ky), _box_gap(*qx, *kx))
            assert rs[r, kb] == want, (qb, kb)


@pytest.mark.parametrize("grid", [(5, 10, 14, (2, 4, 8)), (3, 7, 5, (2, 2, 2)), (4, 6, 9, (3, 2, 2))], ids=str)
def test_rstar_symmetric_with_zero_diagonal(grid):
    T, H, W, cub = grid
    blk = cub[0] * cub[1] * cub[2]
    o = ol.cuboid_order(T, H, W, cub)
    for tw in (0, 1, 2):
        rs = om.window_rstar_bruteforce(T, H, W, blk, tw, order=o)
        np.testing.assert_array_equal(rs, rs.T)
        assert (np.diag(rs) == 0).all()


def test_permute_roundtrip():
    T, H, W, cub = 5, 10, 14, (2, 4, 8)
    o = ol.cuboid_order(T, H, W, cub)
    n_pad = -(-o.size // 64) * 64
    x = np.random.default_rng(3).standard_normal((2, 3, n_pad, 4))
    y = ol.permute_tokens(x, o)
    np.testing.assert_array_equal(y[:, :, :o.size], x[:, :, o])
    np.testing.assert_array_equal(y[:, :, o.size:], x[:, :, o.size:])
    np.testing.assert_array_equal(ol.permute_tokens(y, o, inverse=True), x)
