"""GPU parity of the effective-weight GEMM variant (rabit_gemm_ex and
rabit_grad_input_ex with RABIT_GEMM_WEFF) against the CPU oracle.

Each weight of the tile is e = Σ_p r_p (±h_p) in fp16 (r_p = fp16(g_p / f),
f = max_p g_p), so it carries about one fp16 rounding (2^-11 relative, the
ratio's rounding included): an emulation of this arithmetic in numpy gives
3.5e-4 normwise on the synthetic layers, for two and three paths. Bound:
1e-3 normwise. The exact path's error is about 1e-7, so an error above 1e-5
also shows that the fp16 variant, not the exact one, ran.
"""
import numpy as np
import pytest
import torch

import oracle
from synth.inputs import weight_f32, act_bf16, grad_bf16, bf16_values

pytestmark = pytest.mark.gpu
TOL = 1e-3


def say(*a):
    print("[case]", *a, flush=True)


def packed(rabit, out, inp, seed, P):
    w = weight_f32(out, inp, seed)
    layer = rabit.PackedLayer.empty(out, inp, n_paths=P)
    rabit.pack(w.cuda(), layer)
    return layer, oracle.derive(w.numpy(), n_paths=P)


@pytest.mark.parametrize("P", [2, 3])
@pytest.mark.parametrize("shape", [(256, 512, 64), (1000, 1100, 300), (130, 260, 1), (4096, 4096, 512),
                                   (256, 4100, 64)])
def test_gemm_weff(gpu_lib, shape, P):
    out, inp, m = shape
    say("gemm weff", shape, P)
    layer, d = packed(gpu_lib, out, inp, 6000 + out + m, P)
    x = act_bf16(m, inp, 6100 + m)
    y = gpu_lib.gemm(layer, x.cuda(), weff=True).cpu().numpy().astype(np.float64)
    err = oracle.normwise_rel_err(y, oracle.gemm(d, bf16_values(x)))
    assert 1e-5 < err <= TOL, err


@pytest.mark.parametrize("P", [2, 3])
@pytest.mark.parametrize("shape", [(256, 384, 100), (200, 333, 37), (1000, 1100, 300)])
def test_grad_input_weff(gpu_lib, shape, P):
    out, inp, m = shape
    say("grad_input weff", shape, P)
    layer, d = packed(gpu_lib, out, inp, 6200 + out + m, P)
    dy = grad_bf16(m, out, 6300 + m)
    dx = gpu_lib.grad_input(layer, dy.cuda(), weff=True).cpu().numpy().astype(np.float64)
    err = oracle.normwise_rel_err(dx, oracle.grad_input(d, bf16_values(dy)))
    assert 1e-5 < err <= TOL, err


def test_gemm_weff_full_size_rows(gpu_lib):
    """Llama-3-8B gate shape (14336 x 4096) at M = 2048, as the bench times it:
    sampled token rows against the oracle."""
    out, inp, m = 14336, 4096, 2048
    say("gemm weff full size", out, inp, m)
    layer, d = packed(gpu_lib, out, inp, 6400, 2)
    x = act_bf16(m, inp, 6401)
    y = gpu_lib.gemm(layer, x.cuda(), weff=True)
    rows = [0, 1, 777, 1500, m - 1]
    ref = oracle.gemm(d, bf16_values(x), rows=rows)
    err = oracle.normwise_rel_err(y[rows].cpu().numpy().astype(np.float64), ref)
    assert 1e-5 < err <= TOL, err


@pytest.mark.parametrize("P", [2, 3])
def test_weff_signed_and_zero_scales(gpu_lib, P):
    """Learnable scales may be negative or zero: a row with g_1 = 0 and a
    negative g_2, rows of mixed signs, and negative h entries."""
    out, inp, m = 192, 320, 40
    say("weff signed scales", P)
    w = weight_f32(out, inp, 6500).numpy()
    rng = np.random.default_rng(3)
    g = [(rng.uniform(0.005, 0.03, out) * rng.choice([-1.0, 1.0], out)).astype(np.float16) for _ in range(P)]
    h = [(rng.uniform(0.005, 0.03, inp) * rng.choice([-1.0, 1.0], inp)).astype(np.float16) for _ in range(P)]
    g[0][:8] = 0
    g[1][:8] = -np.abs(g[1][:8])
    layer = gpu_lib.PackedLayer.empty(out, inp, n_paths=P)
    layer.g.copy_(torch.from_numpy(np.stack(g)).view(torch.int16))
    layer.h.copy_(torch.from_numpy(np.stack(h)).view(torch.int16))
    gpu_lib.pack(torch.from_numpy(w).cuda(), layer, gpu_lib.RABIT_SCALES_GIVEN)
    kw = dict(g3=g[2], h3=h[2]) if P == 3 else {}
    d = oracle.derive(w, "given", g1=g[0], h1=h[0], g2=g[1], h2=h[1], n_paths=P, **kw)
    x = act_bf16(m, inp, 6501)
    for weff in (False, True):
        y = gpu_lib.gemm(layer, x.cuda(), weff=weff).cpu().numpy().astype(np.float64)
        err = oracle.normwise_rel_err(y, oracle.gemm(d, bf16_values(x)))
        assert err <= (TOL if weff else 2e-3), (weff, err)
    dy = grad_bf16(m, out, 6502)
    dx = gpu_lib.grad_input(layer, dy.cuda(), weff=True).cpu().numpy().astype(np.float64)
    assert oracle.normwise_rel_err(dx, oracle.grad_input(d, bf16_values(dy))) <= TOL


@pytest.mark.parametrize("batch", [1, 3])
def test_gemv_and_grad_weight_signed_scales(gpu_lib, batch):
    """The decode GEMV and the dW kernel with scales of both signs (and zeros)."""
    out, inp = 256, 700
    say("gemv / grad_weight signed scales", batch)
    w = weight_f32(out, inp, 6600).numpy()
    rng = np.random.default_rng(5)
    g = [(rng.uniform(0.005, 0.03, out) * rng.choice([-1.0, 1.0], out)).astype(np.float16) for _ in range(2)]
    h = [(rng.uniform(0.005, 0.03, inp) * rng.choice([-1.0, 1.0], inp)).astype(np.float16) for _ in range(2)]
    g[0][:5] = 0
    h[1][:7] = 0
    layer = gpu_lib.PackedLayer.empty(out, inp)
    layer.g.copy_(torch.from_numpy(np.stack(g)).view(torch.int16))
    layer.h.copy_(torch.from_numpy(np.stack(h)).view(torch.int16))
    gpu_lib.pack(torch.from_numpy(w).cuda(), layer, gpu_lib.RABIT_SCALES_GIVEN)
    d = oracle.derive(w, "given", g1=g[0], h1=h[0], g2=g[1], h2=h[1])
    x = act_bf16(batch, inp, 6601)
    y = gpu_lib.gemv(layer, x.cuda()).cpu().numpy().astype(np.float64)
    assert oracle.normwise_rel_err(y, oracle.gemv(d, bf16_values(x))) <= 2e-3
    xm = act_bf16(50, inp, 6602)
    dy = grad_bf16(50, out, 6603)
    dw, dg, dh = gpu_lib.grad_weight(layer, xm.cuda(), dy.cuda())
    xv, dyv = bf16_values(xm), bf16_values(dy)
    assert oracle.normwise_rel_err(dw.cpu().numpy().astype(np.float64), oracle.grad_weight(xv, dyv)) <= 1e-5
    for p, (rg, rh) in enumerate(oracle.grad_scales(d, xv, dyv)):
        assert oracle.normwise_rel_err(dg[p].cpu().numpy().astype(np.float64), rg) <= 1e-4
        assert oracle.normwise_rel_err(dh[p].cpu().numpy().astype(np.float64), rh) <= 1e-4
