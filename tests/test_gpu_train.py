"""GPU parity of the training side (paper §4.2, "Backward Pass and Parameter
Updates") through the C ABI against the CPU oracle (oracle/rabit_train.py):

  * rabit_transpose_planes: bit-exact against the oracle's device layout of
    the transposed layer; at full size, transposing twice is the identity;
  * rabit_grad_weight: dW normwise <= 1e-5 (each entry is a float32 sum of M
    exact bf16 products: worst case M * 2^-24 of the sum of |products|, about
    1e-7 typical), dg and dh normwise <= 1e-4 (float32 sums of float32 dW
    values over up to 11008 terms per tile row/column);
  * rabit_grad_input: normwise <= 2e-3 (the prefill GEMM's arithmetic);
  * full Llama-2-7B MLP shapes at M = 2048: sampled entries, rows and columns
    computed one by one by the oracle.
"""
import numpy as np
import pytest
import torch

import oracle
from synth.inputs import weight_f32, act_bf16, grad_bf16, bf16_values, random_f16_scales

pytestmark = pytest.mark.gpu

TOL_DW, TOL_SCALE, TOL_DX = 1e-5, 1e-4, 2e-3


def say(*a):
    print("[case]", *a, flush=True)


def make(rabit, out, inp, seed, n_paths=2):
    """Layer derived on the GPU with given scales (the training forward's
    derivation) and the oracle's Derived for the same W and scales."""
    w = weight_f32(out, inp, seed).numpy()
    g = [random_f16_scales(out, seed + 1), random_f16_scales(out, seed + 2, 0.002, 0.01),
         random_f16_scales(out, seed + 3, 0.001, 0.004)][:n_paths]
    h = [random_f16_scales(inp, seed + 4), random_f16_scales(inp, seed + 5, 0.002, 0.01),
         random_f16_scales(inp, seed + 6, 0.001, 0.004)][:n_paths]
    layer = rabit.PackedLayer.empty(out, inp, n_paths=n_paths)
    layer.g.copy_(torch.from_numpy(np.stack(g)).view(torch.int16))
    layer.h.copy_(torch.from_numpy(np.stack(h)).view(torch.int16))
    rabit.pack(torch.from_numpy(w).cuda(), layer, rabit.RABIT_SCALES_GIVEN)
    kw = dict(g3=g[2], h3=h[2]) if n_paths == 3 else {}
    d = oracle.derive(w, "given", g1=g[0], h1=h[0], g2=g[1], h2=h[1], n_paths=n_paths, **kw)
    words = rabit.unpack(layer).cpu().numpy().view(np.uint32)
    for p, (s, _, _) in enumerate(d.paths):
        assert np.array_equal(words[p], oracle.pack_words(s)), f"planes of path {p + 1} differ"
    return layer, d


def batch(out, inp, m, seed):
    x = act_bf16(m, inp, seed + 7)
    dy = grad_bf16(m, out, seed + 8)
    return x, dy, bf16_values(x), bf16_values(dy)


# Shapes whose out and in are multiples of 8 take the dW kernel's ring loader
# (ragged tiles: 384 = 1.5 x 256 columns, 200 / 264 / 1104 off the tile
# grid; token counts off the 32-token step), the others its staged loader.
SHAPES = [(256, 384, 100), (200, 333, 37), (130, 520, 1), (384, 256, 513), (64, 128, 32),
          (1, 1, 3), (1000, 1100, 300), (200, 264, 45), (1000, 1104, 300)]


@pytest.mark.parametrize("n_paths", [2, 3])
@pytest.mark.parametrize("shape", [(256, 512), (100, 300), (1, 1), (65, 129), (300, 64)])
def test_transpose_planes_bit_exact(gpu_lib, shape, n_paths):
    out, inp = shape
    say("transpose", shape, n_paths)
    layer, d = make(gpu_lib, out, inp, 4000 + out, n_paths)
    pt = gpu_lib.transpose_planes(layer).cpu().numpy().view(np.uint32)
    t = oracle.transposed(d)
    words = [oracle.pack_words(s) for s, _, _ in t.paths]
    ref = oracle.device_planes(words[0], words[1], inp, out, words[2] if n_paths == 3 else None)
    assert np.array_equal(pt, ref)


@pytest.mark.parametrize("n_paths", [2, 3])
def test_transpose_twice_is_identity_full_size(gpu_lib, n_paths):
    out, inp = 11008, 4096
    say("transpose twice", out, inp, n_paths)
    layer, _ = make(gpu_lib, out, inp, 4100, n_paths)
    pt = gpu_lib.transpose_planes(layer)
    lt = gpu_lib.PackedLayer(planes=pt, g=layer.h, h=layer.g, out_features=inp, in_features=out,
                             n_paths=n_paths)
    back = gpu_lib.transpose_planes(lt)
    assert torch.equal(back, layer.planes)


@pytest.mark.parametrize("n_paths", [2, 3])
@pytest.mark.parametrize("shape", SHAPES)
def test_grad_weight(gpu_lib, shape, n_paths):
    out, inp, m = shape
    say("grad_weight", shape, n_paths)
    layer, d = make(gpu_lib, out, inp, 4200 + out + m, n_paths)
    x, dy, xv, dyv = batch(out, inp, m, 4200 + inp)
    dw, dg, dh = gpu_lib.grad_weight(layer, x.cuda(), dy.cuda())
    ref_w = oracle.grad_weight(xv, dyv)
    err = oracle.normwise_rel_err(dw.cpu().numpy().astype(np.float64), ref_w)
    assert err <= TOL_DW, err
    dg, dh = dg.cpu().numpy().astype(np.float64), dh.cpu().numpy().astype(np.float64)
    for p, (rg, rh) in enumerate(oracle.grad_scales(d, xv, dyv)):
        eg = oracle.normwise_rel_err(dg[p], rg)
        eh = oracle.normwise_rel_err(dh[p], rh)
        assert eg <= TOL_SCALE and eh <= TOL_SCALE, (p, eg, eh)


@pytest.mark.parametrize("n_paths", [2, 3])
def test_grad_weight_loaders_agree(gpu_lib, n_paths):
    """The ring loader (in a multiple of 8) and the staged loader give the
    same bits: a 200 x 264 layer against the same layer with a 265th input
    column whose X column is zero (so its dW column is zero and adds nothing
    to dg); dW, dg and dh of the first 264 columns compared bit for bit."""
    out, inp, m = 200, 264, 77
    say("grad_weight loaders", n_paths)
    w = weight_f32(out, inp + 1, 4250).numpy()
    g = [random_f16_scales(out, 4251), random_f16_scales(out, 4252, 0.002, 0.01),
         random_f16_scales(out, 4253, 0.001, 0.004)][:n_paths]
    h = [random_f16_scales(inp + 1, 4254), random_f16_scales(inp + 1, 4255, 0.002, 0.01),
         random_f16_scales(inp + 1, 4256, 0.001, 0.004)][:n_paths]
    layers = []
    for n in (inp, inp + 1):
        layer = gpu_lib.PackedLayer.empty(out, n, n_paths=n_paths)
        layer.g.copy_(torch.from_numpy(np.stack(g)).view(torch.int16))
        layer.h.copy_(torch.from_numpy(np.ascontiguousarray(np.stack(h)[:, :n])).view(torch.int16))
        gpu_lib.pack(torch.from_numpy(np.ascontiguousarray(w[:, :n])).cuda(), layer, gpu_lib.RABIT_SCALES_GIVEN)
        layers.append(layer)
    x = act_bf16(m, inp, 4257)
    dy = grad_bf16(m, out, 4258).cuda()
    x1 = torch.zeros(m, inp + 1, dtype=torch.bfloat16)
    x1[:, :inp] = x
    ra = gpu_lib.grad_weight(layers[0], x.cuda(), dy)
    rb = gpu_lib.grad_weight(layers[1], x1.cuda(), dy)
    torch.cuda.synchronize()
    assert torch.equal(ra[0], rb[0][:, :inp])
    assert torch.equal(ra[1], rb[1])
    assert torch.equal(ra[2], rb[2][:, :inp])


def test_grad_weight_accumulate(gpu_lib):
    out, inp, m = 300, 260, 70
    say("grad_weight accumulate")
    layer, d = make(gpu_lib, out, inp, 4300)
    x1, dy1, xv1, dyv1 = batch(out, inp, m, 4301)
    x2, dy2, xv2, dyv2 = batch(out, inp, m + 9, 4302)
    dw, dg, dh = gpu_lib.grad_weight(layer, x1.cuda(), dy1.cuda())
    gpu_lib.grad_weight(layer, x2.cuda(), dy2.cuda(), dw=dw, dg=dg, dh=dh, accumulate=True)
    ref_w = oracle.grad_weight(xv1, dyv1) + oracle.grad_weight(xv2, dyv2)
    assert oracle.normwise_rel_err(dw.cpu().numpy().astype(np.float64), ref_w) <= TOL_DW
    r1, r2 = oracle.grad_scales(d, xv1, dyv1), oracle.grad_scales(d, xv2, dyv2)
    for p in range(2):
        assert oracle.normwise_rel_err(dg[p].cpu().numpy().astype(np.float64), r1[p][0] + r2[p][0]) <= TOL_SCALE
        assert oracle.normwise_rel_err(dh[p].cpu().numpy().astype(np.float64), r1[p][1] + r2[p][1]) <= TOL_SCALE


@pytest.mark.parametrize("n_paths", [2, 3])
@pytest.mark.parametrize("shape", SHAPES)
def test_grad_input(gpu_lib, shape, n_paths):
    out, inp, m = shape
    say("grad_input", shape, n_paths)
    layer, d = make(gpu_lib, out, inp, 4400 + out + m, n_paths)
    _, dy, _, dyv = batch(out, inp, m, 4400 + inp)
    dx = gpu_lib.grad_input(layer, dy.cuda()).cpu().numpy().astype(np.float64)
    err = oracle.normwise_rel_err(dx, oracle.grad_input(d, dyv))
    assert err <= TOL_DX, err
    dxb = gpu_lib.grad_input(layer, dy.cuda(), gpu_lib.RABIT_OUT_BF16)
    assert dxb.dtype == torch.bfloat16


def test_grad_weight_full_size_sampled(gpu_lib):
    """Llama-2-7B gate projection shape (11008 x 4096) at M = 2048, in the
    launch configuration the bench times: sampled dW entries, dg rows, dh
    columns and dX columns, each from the oracle's sums."""
    out, inp, m = 11008, 4096, 2048
    say("grad full size", out, inp, m)
    layer, d = make(gpu_lib, out, inp, 4500)
    x, dy, xv, dyv = batch(out, inp, m, 4501)
    dw, dg, dh = gpu_lib.grad_weight(layer, x.cuda(), dy.cuda())
    dx = gpu_lib.grad_input(layer, dy.cuda())
    torch.cuda.synchronize()
    rng = np.random.default_rng(5)
    rows = np.concatenate([rng.choice(out, 20, replace=False), [0, out - 1]])
    cols = np.concatenate([rng.choice(inp, 20, replace=False), [0, inp - 1]])
    ri, ci = np.repeat(rows, len(cols)), np.tile(cols, len(rows))
    got = dw.cpu().numpy().astype(np.float64)[ri, ci]
    ref = oracle.grad_weight_entries(xv, dyv, ri, ci)
    assert oracle.normwise_rel_err(got, ref) <= TOL_DW
    dg, dh = dg.cpu().numpy().astype(np.float64), dh.cpu().numpy().astype(np.float64)
    for p, (s, gp, hp) in enumerate(d.paths):
        rg = oracle.grad_g_rows(s[rows], hp, xv, dyv[:, rows])
        rh = oracle.grad_h_cols(s[:, cols], gp, dyv, xv[:, cols])
        assert oracle.normwise_rel_err(dg[p][rows], rg) <= TOL_SCALE
        assert oracle.normwise_rel_err(dh[p][cols], rh) <= TOL_SCALE
    wcols = oracle.weff(d)[:, cols]
    ref_x = oracle.grad_input_cols(wcols, dyv)
    assert oracle.normwise_rel_err(dx.cpu().numpy().astype(np.float64)[:, cols], ref_x) <= TOL_DX
