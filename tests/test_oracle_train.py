"""Pins for the training-side oracle (not gpu).

The coupled forward and the straight-through backward of one layer (paper
§4.2 "The Coupled Forward Pass" and "Backward Pass and Parameter Updates").
Pins, each independent of the oracle's own formulas:
  * torch.autograd in float64 on the graph W_hat = Σ_i g_i ⊙ B_i ⊙ h_i (B_i
    constant), Y = X W_hatᵀ, L = <Y, dY>: gradients of W_hat, g_i, h_i and X;
  * exact finite differences in Fraction on a tiny layer (L is linear in
    each scale, so one difference is the derivative exactly);
  * one-hot closed forms; the Euler identities of a bilinear term;
  * the straight-through property (dW does not depend on W, g, h);
  * the transposed layer's bits by hand positions in the device layout.
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import (derive, weff, gemm, device_planes, pack_words, planes_bytes,
                    train_forward, transposed, grad_weight, grad_scales, grad_input,
                    grad_weight_entries, grad_g_rows, grad_h_cols, grad_input_cols)
from synth.inputs import weight_f32, act_bf16, grad_bf16, bf16_values, random_f16_scales


def _case(out, inp, n, seed, n_paths=2):
    w = weight_f32(out, inp, seed).numpy()
    g1, h1 = random_f16_scales(out, seed + 1), random_f16_scales(inp, seed + 2)
    g2, h2 = random_f16_scales(out, seed + 3, 0.002, 0.01), random_f16_scales(inp, seed + 4, 0.002, 0.01)
    kw = {}
    if n_paths == 3:
        kw = dict(g3=random_f16_scales(out, seed + 5, 0.001, 0.004),
                  h3=random_f16_scales(inp, seed + 6, 0.001, 0.004))
    d = derive(w, "given", g1=g1, h1=h1, g2=g2, h2=h2, n_paths=n_paths, **kw)
    x = bf16_values(act_bf16(n, inp, seed + 7))
    dy = bf16_values(grad_bf16(n, out, seed + 8))
    return d, x, dy


@pytest.mark.parametrize("n_paths", [2, 3])
@pytest.mark.parametrize("shape", [(7, 11, 5), (64, 96, 33)])
def test_backward_matches_autograd(shape, n_paths):
    out, inp, n = shape
    d, x, dy = _case(out, inp, n, 900 + out, n_paths)
    gs = [torch.tensor(p[1].astype(np.float64), requires_grad=True) for p in d.paths]
    hs = [torch.tensor(p[2].astype(np.float64), requires_grad=True) for p in d.paths]
    bs = [torch.tensor(np.where(p[0], -1.0, 1.0)) for p in d.paths]
    xt = torch.tensor(x, requires_grad=True)
    what = sum(g[:, None] * b * h[None, :] for g, b, h in zip(gs, bs, hs))
    what.retain_grad()
    y = xt @ what.T
    (y * torch.tensor(dy)).sum().backward()
    np.testing.assert_allclose(grad_weight(x, dy), what.grad.numpy(), rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(grad_input(d, dy), xt.grad.numpy(), rtol=1e-12, atol=1e-15)
    for (dg, dh), g, h in zip(grad_scales(d, x, dy), gs, hs):
        np.testing.assert_allclose(dg, g.grad.numpy(), rtol=1e-10, atol=1e-14)
        np.testing.assert_allclose(dh, h.grad.numpy(), rtol=1e-10, atol=1e-14)


def test_finite_differences_exact():
    """L = <X W_hatᵀ, dY> is linear in every g_i[o] and h_i[j]: with exact
    rationals, L(s + 1) − L(s) is the partial derivative itself."""
    out, inp, n = 3, 5, 2
    d, x, dy = _case(out, inp, n, 71)
    fx = [[Fraction(float(v)) for v in r] for r in x]
    fdy = [[Fraction(float(v)) for v in r] for r in dy]
    paths = [(p[0], [Fraction(float(v)) for v in p[1]], [Fraction(float(v)) for v in p[2]])
             for p in d.paths]

    def loss(ps):
        tot = Fraction(0)
        for k in range(n):
            for o in range(out):
                yo = Fraction(0)
                for s, g, h in ps:
                    for j in range(inp):
                        yo += g[o] * (-1 if s[o, j] else 1) * h[j] * fx[k][j]
                tot += yo * fdy[k][o]
        return tot

    base = loss(paths)
    res = grad_scales(d, x, dy)
    for pi, (s, g, h) in enumerate(paths):
        for o in range(out):
            g2 = list(g)
            g2[o] += 1
            ps = list(paths)
            ps[pi] = (s, g2, h)
            assert float(loss(ps) - base) == pytest.approx(res[pi][0][o], rel=1e-14, abs=1e-18)
        for j in range(inp):
            h2 = list(h)
            h2[j] += 1
            ps = list(paths)
            ps[pi] = (s, g, h2)
            assert float(loss(ps) - base) == pytest.approx(res[pi][1][j], rel=1e-14, abs=1e-18)


def test_one_hot_closed_forms():
    out, inp = 6, 9
    d, _, _ = _case(out, inp, 1, 33)
    o, i = 4, 7
    x = np.zeros((2, inp))
    dy = np.zeros((2, out))
    x[1, i] = 1.0
    dy[1, o] = 1.0
    dw = grad_weight(x, dy)
    ref = np.zeros((out, inp))
    ref[o, i] = 1.0
    assert np.array_equal(dw, ref)
    for (s, g, h), (dg, dh) in zip(d.paths, grad_scales(d, x, dy)):
        sg = -1.0 if s[o, i] else 1.0
        eg = np.zeros(out)
        eg[o] = sg * float(h[i])
        eh = np.zeros(inp)
        eh[i] = sg * float(g[o])
        assert np.array_equal(dg, eg) and np.array_equal(dh, eh)
    dx = grad_input(d, dy)
    assert np.array_equal(dx[0], np.zeros(inp))
    assert np.array_equal(dx[1], weff(d)[o])


@pytest.mark.parametrize("n_paths", [2, 3])
def test_euler_identities(n_paths):
    """W_hat_i is bilinear in (g_i, h_i): <g_i, dg_i> = <h_i, dh_i> =
    <dW, W_hat_i>, and the sum over paths is <dY, Y>."""
    d, x, dy = _case(40, 70, 13, 5, n_paths)
    dw = grad_weight(x, dy)
    _, y = train_forward(weight_f32(40, 70, 5).numpy(), x, d.g1, d.h1, d.g2, d.h2, n_paths,
                         d.g3, d.h3)
    tot = 0.0
    for (s, g, h), (dg, dh) in zip(d.paths, grad_scales(d, x, dy)):
        wp = g.astype(np.float64)[:, None] * np.where(s, -1.0, 1.0) * h.astype(np.float64)[None, :]
        a = float(np.dot(g.astype(np.float64), dg))
        b = float(np.dot(h.astype(np.float64), dh))
        c = float((dw * wp).sum())
        assert a == pytest.approx(c, rel=1e-10) and b == pytest.approx(c, rel=1e-10)
        tot += c
    assert tot == pytest.approx(float((dy * y).sum()), rel=1e-10)


def test_straight_through():
    """The update handed to W_FP is the gradient of W_hat: it depends on the
    batch only, not on W_FP, the scales or the cores."""
    x = bf16_values(act_bf16(9, 20, 3))
    dy = bf16_values(grad_bf16(9, 12, 4))
    ref = dy.T @ x
    assert np.array_equal(grad_weight(x, dy), ref)
    for seed in (1, 2):
        d, _, _ = _case(12, 20, 1, seed)
        dx = grad_input(d, dy)
        assert dx.shape == (9, 20)
    np.testing.assert_allclose(grad_weight_entries(x, dy, [0, 5, 11], [19, 0, 7]),
                               ref[[0, 5, 11], [19, 0, 7]], rtol=1e-15)


def test_forward_is_frozen_layer_forward():
    """The training forward equals the inference forward of the layer derived
    with the same scales (paper §4.2: inference uses the cores derived from the
    trained W_FP)."""
    w = weight_f32(30, 50, 8).numpy()
    x = bf16_values(act_bf16(4, 50, 9))
    g1, h1 = random_f16_scales(30, 1), random_f16_scales(50, 2)
    g2, h2 = random_f16_scales(30, 3, 0.002, 0.01), random_f16_scales(50, 4, 0.002, 0.01)
    d, y = train_forward(w, x, g1, h1, g2, h2)
    assert np.array_equal(d.s1, w < 0)
    assert np.array_equal(y, gemm(derive(w, "given", g1=g1, h1=h1, g2=g2, h2=h2), x))


@pytest.mark.parametrize("n_paths", [2, 3])
def test_transposed_layer(n_paths):
    out, inp = 150, 200
    d, x, dy = _case(out, inp, 6, 21, n_paths)
    t = transposed(d)
    assert t.shape == (inp, out)
    np.testing.assert_allclose(gemm(t, dy), grad_input(d, dy), rtol=1e-12, atol=1e-15)
    np.testing.assert_array_equal(weff(t), weff(d).T)
    # hand positions: bit (o, i) of B_p sits, in the device planes of the
    # transposed layer, in unit (i // 64, o // 128, p, i % 64), word (o // 32) % 4,
    # bit o % 32
    words = [pack_words(p[0]) for p in t.paths]
    buf = device_planes(*words[:2], inp, out, words[2] if n_paths == 3 else None)
    assert buf.size * 4 == planes_bytes(inp, out, n_paths)
    kg = (out + 127) // 128
    u = buf.reshape((inp + 63) // 64, kg, n_paths, 64, 4)
    rng = np.random.default_rng(0)
    for _ in range(200):
        o, i, p = int(rng.integers(out)), int(rng.integers(inp)), int(rng.integers(n_paths))
        bit = (int(u[i // 64, o // 128, p, i % 64, (o // 32) % 4]) >> (o % 32)) & 1
        assert bit == int(d.paths[p][0][o, i])


def test_sampled_forms_agree():
    d, x, dy = _case(48, 80, 10, 77)
    rows, cols = np.array([0, 13, 47]), np.array([1, 40, 79])
    for p, (dg, dh) in enumerate(grad_scales(d, x, dy)):
        s, g, h = d.paths[p]
        np.testing.assert_allclose(grad_g_rows(s[rows], h, x, dy[:, rows]), dg[rows], rtol=1e-12)
        np.testing.assert_allclose(grad_h_cols(s[:, cols], g, dy, x[:, cols]), dh[cols], rtol=1e-12)
    np.testing.assert_allclose(grad_input_cols(weff(d)[:, cols], dy), grad_input(d, dy)[:, cols],
                               rtol=1e-12)
