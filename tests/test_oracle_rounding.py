"""Pins for the oracle's fp16 / bf16 rounding (not gpu).

f16_rne is numpy's direct float64->float16 cast; bf16_rne is the oracle's own
frexp/rint routine. Both are checked against frac_round_to_format, an exact
rational implementation of IEEE round-to-nearest-even, and bf16_rne also
against torch's float32->bfloat16 conversion.
"""
from fractions import Fraction
import math

import numpy as np
import pytest
import torch

from oracle import f16_rne, bf16_rne, frac_round_to_format


def _f16_ref(v: float):
    r = frac_round_to_format(Fraction(v), 11, -14, 15)
    return float(r)


def test_frac_rounding_known_values():
    # fp16: 1 + 2^-11 is the midpoint between 1 and 1 + 2^-10 -> even (1.0)
    assert frac_round_to_format(Fraction(1) + Fraction(1, 2 ** 11), 11, -14, 15) == 1
    # 1 + 3*2^-11 is between 1+2^-10 (odd) and 1+2^-9 (even) -> 1+2^-9
    assert frac_round_to_format(Fraction(1) + Fraction(3, 2 ** 11), 11, -14, 15) == 1 + Fraction(1, 2 ** 9)
    # largest fp16 is 65504; 65520 is the midpoint to 2^16 -> overflow (ties to even -> inf)
    assert frac_round_to_format(Fraction(65519), 11, -14, 15) == 65504
    assert frac_round_to_format(Fraction(65520), 11, -14, 15) == math.inf
    # smallest subnormal 2^-24; half of it ties to 0 (even)
    assert frac_round_to_format(Fraction(1, 2 ** 25), 11, -14, 15) == 0
    assert frac_round_to_format(Fraction(3, 2 ** 26), 11, -14, 15) == Fraction(1, 2 ** 24)


def test_f16_rne_all_midpoints():
    """numpy's float64->float16 cast is a direct RNE: check every positive fp16
    midpoint, and one float64 ulp either side of it, against exact rounding."""
    allh = np.arange(0, 0x7C00, dtype=np.uint16).view(np.float16).astype(np.float64)
    mids = (allh[:-1] + allh[1:]) / 2.0           # exact in float64
    cases = np.concatenate([mids, np.nextafter(mids, np.inf), np.nextafter(mids, -np.inf)])
    got = f16_rne(cases).astype(np.float64)
    ref = np.array([_f16_ref(float(c)) for c in cases])
    assert np.array_equal(got, ref)
    got_neg = f16_rne(-cases).astype(np.float64)
    assert np.array_equal(got_neg, -ref)


def test_f16_rne_overflow_and_tiny():
    assert f16_rne(np.array([65519.0]))[0] == np.float16(65504)
    assert np.isinf(f16_rne(np.array([65520.0]))[0])
    assert f16_rne(np.array([2.0 ** -25]))[0] == 0
    assert f16_rne(np.array([2.0 ** -25 + 2.0 ** -60]))[0] == np.float16(2.0 ** -24)


def test_bf16_rne_matches_torch_on_float32_values():
    rng = np.random.default_rng(1)
    v = np.concatenate([
        rng.standard_normal(200000),
        rng.standard_normal(20000) * 1e-38,       # float32 subnormal range
        rng.standard_normal(20000) * 1e30,
    ]).astype(np.float32)
    # include exact bf16 midpoints (float32 values whose low 16 bits are 0x8000)
    u = rng.integers(0, 0x7F00, size=20000, dtype=np.uint32) << 16 | 0x8000
    v = np.concatenate([v, u.view(np.float32), -u.view(np.float32)])
    ref = torch.from_numpy(v).to(torch.bfloat16).to(torch.float32).numpy().astype(np.float64)
    got = bf16_rne(v.astype(np.float64))
    assert np.array_equal(got, ref)


def test_bf16_rne_against_fraction_double_inputs():
    # float64 inputs that are NOT float32 values (a float32 detour would double-round)
    rng = np.random.default_rng(2)
    v = rng.standard_normal(3000) * np.exp2(rng.integers(-140, 120, 3000))
    for x in v:
        r = frac_round_to_format(Fraction(float(x)), 8, -126, 127)
        assert bf16_rne(np.array([x]))[0] == float(r)
    # a double-rounding trap: 1 + 2^-8 + 2^-30 rounds up in one step
    x = 1.0 + 2.0 ** -8 + 2.0 ** -30
    assert bf16_rne(np.array([x]))[0] == 1.0 + 2.0 ** -7
    # bf16 max is (2 - 2^-7) 2^127; the midpoint to 2^128 is max + 2^119
    top = (2.0 - 2.0 ** -7) * 2.0 ** 127
    assert bf16_rne(np.array([top + 2.0 ** 119 - 2.0 ** 80]))[0] == top
    assert np.isinf(bf16_rne(np.array([top + 2.0 ** 119]))[0])
