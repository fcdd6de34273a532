"""Pins for the normalized mean-|.| scale mode (not gpu).

Reading: with the literal mean-|.| rule g_i h_j is about mean|M|^2, far below
|M|, so B_2 differs from B_1 in about 1% of the weights; dividing h by the
matrix's global mean |M| makes g_i h_j track |M_ij| (the pages' App. B,
Corollary 1: the second path approximates the first path's residual).
Pins: a rank-1 |M| for which the scales are exact, exact rational rounding
on small random inputs, hand-derived values of the canonical total's order,
the flip fraction's closed form erf(1/sqrt(pi)) for Gaussian weights, and
the residual-norm decrease.
"""
from fractions import Fraction
import math

import numpy as np

import oracle
from oracle import canonical_row_sums, canonical_col_sums, canonical_total, meanabs_scales
from synth.inputs import weight_f32

TINY = 2.0 ** -53


def test_rank_one_scales_are_exact():
    # |M| = a b^T with b of mean 1: g = a, h = b exactly (all sums and
    # divisions exact on these dyadic values)
    rng = np.random.default_rng(7)
    rows, cols = 96, 320
    a = rng.integers(1, 64, rows).astype(np.float64) / 64.0
    b = np.ones(cols)
    b[:cols // 2] = 0.5
    b[cols // 2:] = 1.5
    m = a[:, None] * b[None, :]
    g, h = meanabs_scales(m, normalized=True)
    assert np.array_equal(g.astype(np.float64), a)
    assert np.array_equal(h.astype(np.float64), b)
    # the literal rule gives h = mean_i a_i * b_j instead
    g0, h0 = meanabs_scales(m)
    assert np.array_equal(g0, g)
    assert not np.array_equal(h0, h)


def test_normalized_h_matches_exact_rational():
    rng = np.random.default_rng(8)
    for shape in ((5, 7), (33, 70), (64, 300)):
        m = np.abs(rng.standard_normal(shape)) * 0.02
        rows, cols = shape
        g, h = meanabs_scales(m, normalized=True)
        fm = [[Fraction(float(v)) for v in r] for r in m]
        tot = sum(sum(r) for r in fm)
        mu = tot / (rows * cols)
        for j in range(cols):
            ex = sum(fm[i][j] for i in range(rows)) / rows / mu
            want = oracle.frac_round_to_format(ex, 11, -14, 15)
            assert Fraction(float(h[j])) == want, j
        for i in range(rows):
            want = oracle.frac_round_to_format(sum(fm[i]) / cols, 11, -14, 15)
            assert Fraction(float(g[i])) == want, i


def test_canonical_total_order():
    # lane l sums rows l, l+64, ... left to right: (1 + t) + t = 1
    s = np.zeros(192)
    s[0], s[64], s[128] = 1.0, TINY, TINY
    assert canonical_total(s) == 1.0
    # lanes 1 and 33 meet at the first tree level: t + t = 2^-52, then 1 + 2^-52
    s = np.zeros(64)
    s[0], s[1], s[33] = 1.0, TINY, TINY
    assert canonical_total(s) == 1.0 + 2.0 ** -52
    # lanes 1 and 2 reach lane 0 one at a time: 1 + t = 1 twice
    s[:] = 0
    s[0], s[1], s[2] = 1.0, TINY, TINY
    assert canonical_total(s) == 1.0
    # dyadic values: exact
    v = np.random.default_rng(9).integers(0, 1 << 20, 1000).astype(np.float64) * 2.0 ** -20
    assert Fraction(canonical_total(v)) == sum(Fraction(float(x)) for x in v)


def test_flip_fraction_closed_form():
    # g_i -> E|W|, h_j -> 1: B_2 flips where |W| < E|W| = sigma sqrt(2/pi),
    # probability erf(1/sqrt(pi)) = 0.5751 for Gaussian W
    w = weight_f32(1024, 1024, 21).numpy()
    d = oracle.derive(w, mode="meanabs_normalized")
    flip = float(np.mean(d.s1 != d.s2))
    assert abs(flip - math.erf(1.0 / math.sqrt(math.pi))) < 0.01, flip
    # and the literal rule flips about 1%
    d0 = oracle.derive(w)
    assert float(np.mean(d0.s1 != d0.s2)) < 0.02


def test_normalized_residual_norms_decrease():
    w = weight_f32(512, 768, 22).numpy()
    d = oracle.derive(w, mode="meanabs_normalized")
    W = w.astype(np.float64)
    paths = [g.astype(np.float64)[:, None] * np.where(s, -1.0, 1.0) * h.astype(np.float64)[None, :]
             for s, g, h in d.paths]
    n0 = np.linalg.norm(W)
    n1 = np.linalg.norm(W - paths[0])
    n2 = np.linalg.norm(W - paths[0] - paths[1])
    assert n0 > n1 > n2
    assert n1 < 0.7 * n0 and n2 < 0.7 * n1
    # three paths: one more step of the same recursion
    d3 = oracle.derive(w, mode="meanabs_normalized", n_paths=3)
    assert np.array_equal(d3.s2, d.s2) and np.array_equal(d3.g2, d.g2)
    p3 = d3.g3.astype(np.float64)[:, None] * np.where(d3.s3, -1.0, 1.0) * d3.h3.astype(np.float64)[None, :]
    assert np.linalg.norm(W - paths[0] - paths[1] - p3) < n2


def test_zero_matrix_gives_zero_scales():
    g, h = meanabs_scales(np.zeros((8, 40)), normalized=True)
    assert not g.any() and not h.any()
