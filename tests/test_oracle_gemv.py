"""Pins for the oracle's linear layer (not gpu).

y = Σ_p g_p ⊙ (B_p (h_p ⊙ x)) (paper §4.1 eqs.). Pins: the reconstruct-then-
multiply form and the add/subtract form (paper §5.4, App. E.1) agree exactly
in rational arithmetic; float64 agrees with the rationals; unit-vector probes,
all-+1 planes, path additivity and the single-path reduction.
"""
from fractions import Fraction

import numpy as np
import pytest

from oracle import (derive, Derived, gemv, gemv_additions, gemm, frac_gemv,
                    frac_gemv_additions, weff, normwise_rel_err)
from synth.inputs import weight_f32, act_bf16, bf16_values


@pytest.mark.parametrize("seed", [101, 102])
def test_two_formulations_exact_4x8(seed):
    w = weight_f32(4, 8, seed).numpy()
    d = derive(w)
    x = bf16_values(act_bf16(2, 8, seed + 1))
    a = frac_gemv(d, x)
    b = frac_gemv_additions(d, x)
    assert a == b
    y = gemv(d, x)
    for bi in range(2):
        for i in range(4):
            ref = a[bi][i]
            assert abs(Fraction(float(y[bi, i])) - ref) <= abs(ref) * Fraction(1, 10 ** 14) + Fraction(1, 10 ** 300)


def test_float64_formulations_agree():
    w = weight_f32(96, 700, 111).numpy()
    d = derive(w)
    x = bf16_values(act_bf16(3, 700, 112))
    assert normwise_rel_err(gemv_additions(d, x), gemv(d, x)) < 1e-13


def test_unit_vector_probe_returns_weff_column():
    w = weight_f32(32, 100, 121).numpy()
    d = derive(w)
    we = weff(d)
    for j in (0, 37, 99):
        x = np.zeros((1, 100))
        x[0, j] = 1.0
        assert np.array_equal(gemv(d, x)[0], we[:, j])
        # each entry is g1*(±h1) + g2*(±h2) of fp16 values
        i = 5
        ref = (float(d.g1[i]) * (-1 if d.s1[i, j] else 1) * float(d.h1[j]) +
               float(d.g2[i]) * (-1 if d.s2[i, j] else 1) * float(d.h2[j]))
        assert we[i, j] == ref


def test_all_plus_one_planes_closed_form():
    out, inp = 8, 40
    rng = np.random.default_rng(131)
    f = lambda n: rng.uniform(0.01, 0.03, n).astype(np.float16)
    d = Derived(np.zeros((out, inp), bool), np.zeros((out, inp), bool), f(out), f(inp), f(out), f(inp))
    y = gemv(d, np.ones((1, inp)))[0]
    ref = (d.g1.astype(np.float64) * d.h1.astype(np.float64).sum() +
           d.g2.astype(np.float64) * d.h2.astype(np.float64).sum())
    assert np.allclose(y, ref, rtol=1e-14, atol=0)


def test_path_additivity_and_single_path_reduction():
    w = weight_f32(48, 256, 141).numpy()
    d = derive(w)
    x = bf16_values(act_bf16(2, 256, 142))
    z16o = np.zeros_like(d.g1)
    p1 = Derived(d.s1, d.s2, d.g1, d.h1, z16o, d.h2)
    p2 = Derived(d.s1, d.s2, z16o, d.h1, d.g2, d.h2)
    assert normwise_rel_err(gemv(p1, x) + gemv(p2, x), gemv(d, x)) < 1e-14
    # g2 = 0: a single binary layer y = g1 ⊙ (B1 (h1 ⊙ x))
    b1 = np.where(d.s1, -1.0, 1.0)
    single = d.g1.astype(np.float64)[None, :] * ((x * d.h1.astype(np.float64)[None, :]) @ b1.T)
    assert normwise_rel_err(gemv(p1, x), single) < 1e-14


def test_gemm_rows_equal_gemv():
    w = weight_f32(64, 128, 151).numpy()
    d = derive(w)
    xm = bf16_values(act_bf16(20, 128, 152))
    ym = gemm(d, xm)
    assert np.array_equal(ym[7], gemv(d, xm[7:8])[0])
    assert np.array_equal(gemm(d, xm, rows=[3, 9]), ym[[3, 9]])


def test_gemv_is_linear():
    w = weight_f32(64, 512, 161).numpy()
    d = derive(w)
    x1 = bf16_values(act_bf16(1, 512, 162))
    x2 = bf16_values(act_bf16(1, 512, 163))
    assert normwise_rel_err(gemv(d, 2 * x1 - 3 * x2), 2 * gemv(d, x1) - 3 * gemv(d, x2)) < 1e-13


def test_normwise_err_definition():
    assert normwise_rel_err(np.array([[1.0, 2.0]]), np.array([[1.0, 4.0]])) == 0.5
    assert normwise_rel_err(np.array([[1.0, 2.0], [0.0, 0.0]]), np.array([[1.0, 2.0], [0.0, 0.0]])) == 0.0
