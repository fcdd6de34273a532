"""Pins for the initialisation oracle (not gpu): iterative residual SVID
(paper §4.3 eq., App. F.3) with I/O channel importance preconditioning
(paper §4.3 eqs.). Each pin is independent of the oracle's own formulas."""
import math

import numpy as np
import pytest

from oracle import svid, svid_leading, residual_svid, svid_objective
from synth.inputs import weight_f32


def _what(s, g, h):
    return g[:, None] * np.where(s, -1.0, 1.0) * h[None, :]


def test_exact_recovery_of_sign_times_rank1():
    rng = np.random.default_rng(1)
    a, b = rng.uniform(0.5, 2.0, 7), rng.uniform(0.1, 1.0, 11)
    sgn = rng.integers(0, 2, (7, 11)).astype(bool)
    r = np.where(sgn, -1.0, 1.0) * np.outer(a, b)
    s, g, h = svid(r)
    assert np.array_equal(s, sgn)
    np.testing.assert_allclose(np.outer(g, h), np.outer(a, b), rtol=1e-12)
    assert np.linalg.norm(g) == pytest.approx(np.linalg.norm(h), rel=1e-12)


def test_leading_singular_value_2x2_closed_form():
    r = np.array([[3.0, -1.0], [-2.0, 4.0]])
    _, g, h = svid(r)
    a = np.abs(r)
    m = a.T @ a                                 # [[13, 11], [11, 17]]
    tr, det = np.trace(m), np.linalg.det(m)
    lam = (tr + math.sqrt(tr * tr - 4 * det)) / 2   # largest eigenvalue of AᵀA
    sigma = math.sqrt(lam)
    assert np.linalg.norm(g) * np.linalg.norm(h) == pytest.approx(sigma, rel=1e-12)
    # the right singular vector solves (AᵀA − λ I) v = 0
    v = h / np.linalg.norm(h)
    np.testing.assert_allclose(m @ v, lam * v, rtol=1e-12)


def test_svid_is_optimal_against_perturbations():
    rng = np.random.default_rng(3)
    r = rng.normal(size=(9, 13))
    s, g, h = svid(r)
    best = np.linalg.norm(r - _what(s, g, h))
    for _ in range(200):
        g2 = np.abs(g * (1 + 0.05 * rng.normal(size=g.shape)))
        h2 = np.abs(h * (1 + 0.05 * rng.normal(size=h.shape)))
        s2 = s.copy()
        flip = rng.random(s.shape) < 0.05
        s2[flip] = ~s2[flip]
        for cand in ((s, g2, h2), (s2, g, h), (s2, g2, h2)):
            assert np.linalg.norm(r - _what(*cand)) >= best - 1e-12


@pytest.mark.parametrize("n_paths", [2, 3])
def test_residual_never_rises(n_paths):
    w = weight_f32(48, 80, 77).numpy().astype(np.float64)
    hist = []
    residual_svid(w, n_paths=n_paths, sweeps=6, history=hist)
    assert len(hist) == 6 * n_paths
    for a, b in zip(hist, hist[1:]):
        assert b <= a * (1 + 1e-12)
    # the iterations improve on the greedy sweep
    assert hist[-1] < hist[n_paths - 1]


def test_first_sweep_is_greedy():
    w = weight_f32(30, 50, 5).numpy().astype(np.float64)
    p = residual_svid(w, n_paths=2, sweeps=1)
    s1, g1, h1 = svid(w)
    s2, g2, h2 = svid(w - _what(s1, g1, h1))
    assert np.array_equal(p[0][0], s1) and np.array_equal(p[1][0], s2)
    np.testing.assert_allclose(np.outer(p[0][1], p[0][2]), np.outer(g1, h1), rtol=1e-10)
    np.testing.assert_allclose(np.outer(p[1][1], p[1][2]), np.outer(g2, h2), rtol=1e-10)


def test_preconditioning_maps_back():
    w = weight_f32(40, 60, 9).numpy().astype(np.float64)
    rng = np.random.default_rng(2)
    fo, fi = rng.uniform(0.5, 2.0, 40), rng.uniform(0.5, 2.0, 60)
    plain = residual_svid(w, sweeps=3)
    ones = residual_svid(w, sweeps=3, f_out=np.ones(40), f_in=np.ones(60))
    for a, b in zip(plain, ones):
        assert np.array_equal(a[0], b[0])
        np.testing.assert_allclose(a[1], b[1], rtol=1e-12)
    pre = residual_svid(w, sweeps=3, f_out=fo, f_in=fi)
    direct = residual_svid(fo[:, None] * w * fi[None, :], sweeps=3)
    for (s, g, h), (sd, gd, hd) in zip(pre, direct):
        # the cores are those of the preconditioned matrix; the scales are
        # mapped back, so f_out g h f_in reproduces the preconditioned fit
        assert np.array_equal(s, sd)
        np.testing.assert_allclose(np.outer(fo * g, fi * h), np.outer(gd, hd), rtol=1e-9)
    # the preconditioned objective weights errors by the channel factors
    wh = sum(_what(*p) for p in pre)
    assert np.linalg.norm(fo[:, None] * (w - wh) * fi[None, :]) == pytest.approx(
        svid_objective(fo[:, None] * w * fi[None, :], direct), rel=1e-9)


def test_leading_triple_matches_full_svd():
    w = weight_f32(120, 200, 41).numpy().astype(np.float64)
    s, g, h = svid(w)
    s2, g2, h2 = svid_leading(w)
    assert np.array_equal(s, s2)
    np.testing.assert_allclose(g2, g, rtol=1e-9, atol=1e-12)
    np.testing.assert_allclose(h2, h, rtol=1e-9, atol=1e-12)


def _planted(out, inp, n_paths, ratio, seed):
    """W = sum_p outer(g_p, h_p) * (+-1)_p with g, h in [1, 1.5] and path p
    scaled by ratio^-p: every sign decision of the SVID has a margin."""
    rng = np.random.default_rng(seed)
    sg = [rng.integers(0, 2, (out, inp)).astype(bool) for _ in range(n_paths)]
    a = [rng.uniform(1.0, 1.5, out) * ratio ** -p for p in range(n_paths)]
    b = [rng.uniform(1.0, 1.5, inp) for _ in range(n_paths)]
    w = sum(_what(sg[p], a[p], b[p]) for p in range(n_paths))
    return w, sg, a, b


@pytest.mark.parametrize("n_paths", [2, 3])
def test_twenty_sweeps_recover_planted_paths(n_paths):
    # a weight that is exactly a sum of well-separated sign x rank-1 paths is
    # recovered path by path: the signs exactly, each rank-1 magnitude to
    # within the power-free SVD's rounding
    w, sg, a, b = _planted(96, 160, n_paths, 4.0, 31 + n_paths)
    paths = residual_svid(w, n_paths=n_paths, sweeps=20)
    for p, (s, g, h) in enumerate(paths):
        assert np.array_equal(s, sg[p]), p
        o = np.outer(a[p], b[p])
        assert np.linalg.norm(np.outer(g, h) - o) <= 1e-6 * np.linalg.norm(o), p
    assert svid_objective(w, paths) <= 1e-9 * np.linalg.norm(w)
