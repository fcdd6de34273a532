"""Pins for the canonical scale sums (not gpu).

The canonical order is a reading (the pages fix none). Pins: exact results on
dyadic data where every order is exact, an fsum error bound on random data,
and hand-derived values that differ between association orders, so that a
different tree or segment shape fails.
"""
from fractions import Fraction
import math

import numpy as np

from oracle import canonical_row_sums, canonical_col_sums, TILE_COLS, TILE_ROWS

TINY = 2.0 ** -53


def test_dyadic_sums_are_exact():
    rng = np.random.default_rng(3)
    # values k * 2^-10 with k < 2^12: every partial sum is exact in float64
    a = rng.integers(0, 4096, size=(70, 300)).astype(np.float64) * 2.0 ** -10
    rs = canonical_row_sums(a)
    cs = canonical_col_sums(a)
    for i in range(a.shape[0]):
        assert Fraction(rs[i]) == sum(Fraction(v) for v in a[i])
    for j in range(a.shape[1]):
        assert Fraction(cs[j]) == sum(Fraction(v) for v in a[:, j])


def test_fsum_bound():
    rng = np.random.default_rng(4)
    a = np.abs(rng.standard_normal((129, 1000)) * 0.02)
    rs = canonical_row_sums(a)
    cs = canonical_col_sums(a)
    for i in range(a.shape[0]):
        ex = math.fsum(a[i])
        assert abs(rs[i] - ex) <= a.shape[1] * 2.0 ** -52 * ex
    for j in range(a.shape[1]):
        ex = math.fsum(a[:, j])
        assert abs(cs[j] - ex) <= a.shape[0] * 2.0 ** -52 * ex


def _row(cols, entries):
    r = np.zeros((1, cols))
    for c, v in entries.items():
        r[0, c] = v
    return r


def test_row_sum_lane_order_is_sequential():
    # within a lane (columns l, l+64, l+128, l+192) the sum is left to right:
    # ((1 + t) + t) = 1 under ties-to-even, whereas 1 + (t + t) = 1 + 2^-52
    a = _row(256, {0: 1.0, 64: TINY, 128: TINY})
    assert canonical_row_sums(a)[0] == 1.0


def test_row_sum_tree_shape():
    # lanes 1 and 33 meet at the first tree level (s = 32): t + t = 2^-52,
    # then 1 + 2^-52 is exact
    a = _row(256, {0: 1.0, 1: TINY, 33: TINY})
    assert canonical_row_sums(a)[0] == 1.0 + 2.0 ** -52
    # lanes 1 and 2 never meet before lane 0 absorbs them one at a time
    # (s = 2: v0 = 1 + t -> 1; s = 1: v0 = 1 + (t) -> 1)
    a = _row(256, {0: 1.0, 1: TINY, 2: TINY})
    assert canonical_row_sums(a)[0] == 1.0


def test_row_sum_tiles_sequential():
    # tile totals are added left to right: (1 + t) + t = 1
    a = _row(3 * TILE_COLS, {0: 1.0, TILE_COLS: TINY, 2 * TILE_COLS: TINY})
    assert canonical_row_sums(a)[0] == 1.0


def test_col_sum_segment_and_tile_shape():
    col = np.zeros((3 * TILE_ROWS, 1))
    # segment (16 rows) sums are sequential: rows 0,1,2 -> (1 + t) + t = 1
    col[0, 0], col[1, 0], col[2, 0] = 1.0, TINY, TINY
    assert canonical_col_sums(col)[0] == 1.0
    # rows 16 and 32 start segments 1 and 2 of tile 0; segment sums are added
    # left to right: ((1 + t) + t) = 1
    col[:] = 0
    col[0, 0], col[16, 0], col[32, 0] = 1.0, TINY, TINY
    assert canonical_col_sums(col)[0] == 1.0
    # row 70 and 71 are in the same segment of tile 1: t + t = 2^-52 and the
    # tile total is then added to tile 0: 1 + 2^-52
    col[:] = 0
    col[0, 0], col[70, 0], col[71, 0] = 1.0, TINY, TINY
    assert canonical_col_sums(col)[0] == 1.0 + 2.0 ** -52


def test_padding_does_not_change_sums():
    rng = np.random.default_rng(5)
    a = np.abs(rng.standard_normal((37, 301)))
    b = np.zeros((64, 512))
    b[:37, :301] = a
    assert np.array_equal(canonical_row_sums(a), canonical_row_sums(b)[:37])
    assert np.array_equal(canonical_col_sums(a), canonical_col_sums(b)[:301])
