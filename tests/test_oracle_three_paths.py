"""Pins for the oracle's 3-path (3-bit) variant (not gpu).

The third path continues the coupled derivation one step (each path corrects
the residual of its predecessor: paper abstract and §1; §4.2 steps 1-3 for the
first two paths; App. E.1 "Weight Packing" packs 2-bit and 3-bit models).
Pins: brute-force argmin over all sign vectors on 4x8 with exact rationals
(B_3 is the least-squares sign of R_2), the closed flip rule B_3 = B_2 xor
[|R_1| < e_2], a single-rounding check of R_2 in rationals, the residual-norm
identity for the third step, the device layout with three planes (hand
positions and round trip), and two GEMV formulations agreeing exactly.
"""
from fractions import Fraction
import itertools

import numpy as np
import pytest

from oracle import (derive, frac_round_to_format, weff, gemv, frac_gemv, frac_gemv_additions,
                    pack_words, device_planes, device_planes_to_words, planes_bytes)
from synth.inputs import weight_f32, act_bf16, bf16_values, random_f16_scales


def _brute_rows(target, g, h):
    out, inp = len(target), len(target[0])
    best_rows = []
    for i in range(out):
        best, best_b = None, None
        for bits in itertools.product((1, -1), repeat=inp):  # +1 first: ties keep +1
            err = sum((target[i][j] - g[i] * h[j] * bits[j]) ** 2 for j in range(inp))
            if best is None or err < best:
                best, best_b = err, bits
        best_rows.append([b == -1 for b in best_b])
    return np.array(best_rows)


def _frac_mat(a):
    return [[Fraction(float(v)) for v in row] for row in a]


@pytest.mark.parametrize("seed", [111, 112, 113])
def test_b3_brute_force_4x8(seed):
    w = weight_f32(4, 8, seed).numpy()
    d = derive(w, n_paths=3)
    assert d.n_paths == 3
    g3 = [Fraction(float(v)) for v in d.g3]
    h3 = [Fraction(float(v)) for v in d.h3]
    assert all(v > 0 for v in g3 + h3)
    assert np.array_equal(_brute_rows(_frac_mat(d.r2), g3, h3), d.s3)
    # the first two paths are those of the 2-path derivation
    d2 = derive(w)
    assert np.array_equal(d.s1, d2.s1) and np.array_equal(d.s2, d2.s2)
    assert np.array_equal(d.g2, d2.g2) and np.array_equal(d.h2, d2.h2)


@pytest.mark.parametrize("seed", [121, 122])
def test_b3_closed_form(seed):
    w = weight_f32(128, 512, seed).numpy()
    d = derive(w, n_paths=3)
    e2 = d.g2.astype(np.float64)[:, None] * d.h2.astype(np.float64)[None, :]
    r = d.r.astype(np.float64)
    ar = np.abs(r)
    flip = (ar < e2) | ((ar == e2) & (r < 0))
    assert np.array_equal(d.s3, d.s2 ^ flip)
    assert 0 < np.mean(flip) < 0.5


def test_b3_closed_form_ties_and_zero_residual():
    # R_1 = ±e_2 exactly gives R_2 = +0 (bit 0); R_1 = ±0 gives R_2 = -e_2 (bit 1)
    g = np.array([0.5], dtype=np.float16)
    h = np.array([0.25, 0.25, 0.25, 0.25], dtype=np.float16)
    # e_1 = 0.125; W = e_1 + r1 with r1 in {0.0625, -0.0625, 0, ...}
    w = np.array([[0.1875, 0.0625, 0.125, -0.125]], dtype=np.float32)
    g2 = np.array([0.25], dtype=np.float16)
    h2 = np.array([0.25, 0.25, 0.25, 0.25], dtype=np.float16)   # e_2 = 0.0625
    d = derive(w, mode="given", g1=g, h1=h, g2=g2, h2=h2, n_paths=3)
    assert d.r.tolist() == [[0.0625, -0.0625, 0.0, 0.0]]
    assert d.s2.tolist() == [[False, True, False, False]]
    assert d.r2.tolist() == [[0.0, 0.0, -0.0625, -0.0625]]
    assert d.s3.tolist() == [[False, False, True, True]]


def test_r2_single_rounding():
    rng = np.random.default_rng(131)
    w = (rng.standard_normal((6, 40)) * np.exp2(rng.integers(-30, 2, (6, 40)))).astype(np.float32)
    d = derive(w, n_paths=3)
    for i in range(w.shape[0]):
        for j in range(w.shape[1]):
            b = -1 if d.s2[i, j] else 1
            ex = Fraction(float(d.r[i, j])) - b * Fraction(float(d.g2[i])) * Fraction(float(d.h2[j]))
            assert Fraction(float(d.r2[i, j])) == frac_round_to_format(ex, 24, -126, 127)


def test_third_step_residual_identity_and_hierarchy():
    """‖R2‖² − ‖R2 − W3‖² = Σ e3 (2|R2| − e3) with R2 = W − W1 − W2 and
    B3 = sign(R2); at config-like inputs (σ = 0.02) each path lowers the
    residual norm: ‖W‖ ≥ ‖W−W1‖ ≥ ‖W−W1−W2‖ ≥ ‖W−W1−W2−W3‖."""
    w = weight_f32(256, 1024, 141).numpy().astype(np.float64)
    d = derive(w.astype(np.float32), n_paths=3)
    terms = [g.astype(np.float64)[:, None] * np.where(s, -1.0, 1.0) * h.astype(np.float64)[None, :]
             for s, g, h in d.paths]
    r2 = w - terms[0] - terms[1]
    e3 = d.g3.astype(np.float64)[:, None] * d.h3.astype(np.float64)[None, :]
    lhs = np.sum(r2 ** 2) - np.sum((r2 - terms[2]) ** 2)
    rhs = np.sum(e3 * (2 * np.abs(r2) - e3))
    assert abs(lhs - rhs) <= 1e-9 * abs(rhs)
    norms = [np.linalg.norm(w), np.linalg.norm(w - terms[0]), np.linalg.norm(r2),
             np.linalg.norm(r2 - terms[2])]
    assert norms[0] >= norms[1] >= norms[2] >= norms[3]
    assert np.array_equal(weff(d), terms[0] + terms[1] + terms[2])


def test_device_layout_three_planes():
    out, inp = 150, 300      # 3 row groups, 3 column groups (ragged)
    rng = np.random.default_rng(151)
    ws = [pack_words(rng.integers(0, 2, (out, inp)).astype(bool)) for _ in range(3)]
    buf = device_planes(ws[0], ws[1], out, inp, ws[2])
    assert buf.size * 4 == planes_bytes(out, inp, 3)
    unit = lambda rg, kg, p, r: ((((rg * 3 + kg) * 3 + p) * 64) + r) * 4
    assert buf[unit(0, 0, 2, 0)] == ws[2][0, 0]
    assert buf[unit(1, 2, 2, 5) + 1] == ws[2][69, 9]
    assert buf[unit(2, 1, 1, 20) + 3] == ws[1][148, 7]
    assert buf[unit(1, 0, 0, 63)] == ws[0][127, 0]
    back = device_planes_to_words(buf, out, inp, 3)
    for a, b in zip(back, ws):
        assert np.array_equal(a, b)
    # two planes: the same bytes as before for paths 0 and 1
    assert np.array_equal(device_planes_to_words(device_planes(ws[0], ws[1], out, inp), out, inp)[1], ws[1])


def test_three_path_gemv_formulations_agree_exactly():
    w = weight_f32(5, 13, 161).numpy()
    d = derive(w, n_paths=3)
    x = bf16_values(act_bf16(2, 13, 162))
    a = frac_gemv(d, x)
    b = frac_gemv_additions(d, x)
    assert a == b
    y = gemv(d, x)
    for bi in range(2):
        for i in range(5):
            assert abs(float(a[bi][i]) - y[bi, i]) <= 1e-15 * max(1.0, abs(float(a[bi][i])))


def test_three_path_given_scales():
    w = weight_f32(64, 256, 171).numpy()
    g = random_f16_scales(64, 3)
    h = random_f16_scales(256, 4)
    d = derive(w, mode="given", g1=g, h1=h, g2=g, h2=h, g3=g, h3=h, n_paths=3)
    assert np.array_equal(d.g3, g) and np.array_equal(d.h3, h)
    e = g.astype(np.float64)[:, None] * h.astype(np.float64)[None, :]
    r = d.r.astype(np.float64)
    flip = (np.abs(r) < e) | ((np.abs(r) == e) & (r < 0))
    assert np.array_equal(d.s3, d.s2 ^ flip)
