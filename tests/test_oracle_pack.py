"""Pins for packing and the device plane layout (not gpu).

Paper App. E.1 ("Weight Packing"): 32 columns per uint32, +1 -> 0 and
-1 -> 1. LSB-first column order is a reading. The device layout pins are
hand-derived positions from the layout's description plus a round trip.
"""
import numpy as np
import pytest

from oracle import (pack_words, unpack_words, device_planes, device_planes_to_words,
                    planes_bytes)
from synth.inputs import random_signs


def test_word_patterns():
    assert pack_words(np.zeros((1, 32), bool))[0, 0] == 0x00000000
    assert pack_words(np.ones((1, 32), bool))[0, 0] == 0xFFFFFFFF
    alt = np.array([[c % 2 == 1 for c in range(32)]])   # +1, -1, +1, -1, ...
    assert pack_words(alt)[0, 0] == 0xAAAAAAAA
    first = np.zeros((1, 32), bool)
    first[0, 0] = True
    assert pack_words(first)[0, 0] == 0x00000001
    last = np.zeros((1, 32), bool)
    last[0, 31] = True
    assert pack_words(last)[0, 0] == 0x80000000


def test_padding_bits_zero_and_round_trip():
    s = random_signs(5, 37, 1)
    s[:, 32:] = True
    w = pack_words(s)
    assert w.shape == (5, 2)
    assert np.all(w[:, 1] == 0x1F)             # 5 valid bits, 27 padding bits 0
    assert np.array_equal(unpack_words(w, 37), s)
    s2 = random_signs(7, 300, 2)
    assert np.array_equal(unpack_words(pack_words(s2), 300), s2)


def test_footprint_closed_forms():
    # 32x smaller than fp32 per path, 8x smaller than fp16 for 2 paths
    for out, inp in [(4096, 4096), (11008, 4096), (4096, 11008), (14336, 4096), (1024, 4096)]:
        pb = planes_bytes(out, inp, 2)
        assert pb == 2 * out * inp // 8
        assert out * inp * 4 == 32 * pb // 2
        assert out * inp * 2 == 8 * pb
    assert planes_bytes(1, 1, 2) == 2048           # one row group x one column group
    assert planes_bytes(65, 129, 2) == 2 * 2 * 2048


def test_device_layout_hand_positions():
    out, inp = 130, 300            # 3 row groups, 3 column groups (nw = 10)
    rng = np.random.default_rng(7)
    w1 = rng.integers(0, 2 ** 32, size=(out, 10), dtype=np.uint64).astype(np.uint32)
    w2 = rng.integers(0, 2 ** 32, size=(out, 10), dtype=np.uint64).astype(np.uint32)
    w1[:, 9] &= 0xFFF                      # 300 = 9*32 + 12 valid bits
    w2[:, 9] &= 0xFFF
    buf = device_planes(w1, w2, out, inp)
    assert buf.size * 4 == planes_bytes(out, inp)
    unit = lambda rg, kg, p, r: ((((rg * 3 + kg) * 2 + p) * 64) + r) * 4
    # row 65 word 5 of path 1 -> (rg 1, kg 1, p 0, r 1), dword 1
    assert buf[unit(1, 1, 0, 1) + 1] == w1[65, 5]
    # row 129 word 9 of path 2 -> (rg 2, kg 2, p 1, r 1), dword 1
    assert buf[unit(2, 2, 1, 1) + 1] == w2[129, 9]
    # row 0 word 0 of path 2 -> (0, 0, 1, 0) dword 0
    assert buf[unit(0, 0, 1, 0)] == w2[0, 0]
    # words 10, 11 of every row (beyond nw) and rows >= 130 are zero
    assert np.all(buf.reshape(3, 3, 2, 64, 4)[:, 2, :, :, 2:] == 0)
    assert np.all(buf.reshape(3, 3, 2, 64, 4)[2, :, :, 2:, :] == 0)
    r1, r2 = device_planes_to_words(buf, out, inp)
    assert np.array_equal(r1, w1) and np.array_equal(r2, w2)


def test_device_layout_is_a_bijection_on_bits():
    out, inp = 64, 128
    # each canonical bit lands in a distinct device bit
    seen = set()
    for p in range(2):
        for i in range(out):
            for k in range(4):
                w1 = np.zeros((out, 4), np.uint32)
                w2 = np.zeros((out, 4), np.uint32)
                (w1 if p == 0 else w2)[i, k] = 1
                idx = int(np.flatnonzero(device_planes(w1, w2, out, inp))[0])
                assert idx not in seen
                seen.add(idx)
    assert len(seen) == 2 * out * 4


def test_golden_pack_patterns():
    import os
    path = os.path.join(os.path.dirname(__file__), "golden", "e1_pack_patterns.txt")
    n = 0
    for line in open(path):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        signs, hexw = line.split()
        s = np.array([[c == "-" for c in signs]])
        assert pack_words(s)[0, 0] == int(hexw, 16), line
        n += 1
    assert n == 8
