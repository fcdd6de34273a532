"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Bars: packed words and fp16 scales bit-exact;
GEMV/GEMM/decode outputs within a normwise relative error of 2e-3 per batch
row (max_i |y - ŷ| / max_i |ŷ|); unit-vector probes bit-exact.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
from synth.inputs import (weight_f32, act_bf16, bf16_values, random_f16_scales, seed_w, seed_x)

pytestmark = pytest.mark.gpu
TOL = 2e-3


def say(*a):
    print("[case]", *a, flush=True)
    sys.stdout.flush()


def pack_gpu(rabit, w_cpu, mode=None, g=None, h=None):
    mode = rabit.RABIT_SCALES_MEANABS if mode is None else mode
    out, inp = w_cpu.shape
    layer = rabit.PackedLayer.empty(out, inp)
    if g is not None:
        gg = torch.zeros(2, out, dtype=torch.float16)
        hh = torch.zeros(2, inp, dtype=torch.float16)
        gg[0] = torch.from_numpy(g)
        hh[0] = torch.from_numpy(h)
        layer.g.copy_(gg.view(torch.int16))
        layer.h.copy_(hh.view(torch.int16))
    rabit.pack(w_cpu.cuda(), layer, mode)
    torch.cuda.synchronize()
    return layer


def check_pack(rabit, layer, d, out, inp, check_scales=True):
    words = rabit.unpack(layer).cpu().numpy().view(np.uint32)
    w1, w2 = oracle.pack_words(d.s1), oracle.pack_words(d.s2)
    assert np.array_equal(words[0], w1), "path-1 words differ"
    assert np.array_equal(words[1], w2), "path-2 words differ"
    raw = layer.planes.cpu().numpy().view(np.uint32)
    assert np.array_equal(raw, oracle.device_planes(w1, w2, out, inp)), "device layout differs"
    if check_scales:
        g = layer.g.cpu().numpy().view(np.float16)
        h = layer.h.cpu().numpy().view(np.float16)
        for name, got, ref in (("g1", g[0], d.g1), ("h1", h[0], d.h1), ("g2", g[1], d.g2), ("h2", h[1], d.h2)):
            bad = np.flatnonzero(got.view(np.uint16) != ref.view(np.uint16))
            assert bad.size == 0, f"{name}: {bad.size} fp16 scales differ, first at {bad[:5]}"


def fx_bound(d, xv):
    """Elementwise error bound of the GEMV arithmetic stated in rabit.h.

    Per (batch row, path, range of 512 columns) h_p*x is rounded to a grid of
    step 2^(ilogb(max |h_p*x|) - 18), so each element is off by at most half a
    step; the signed sums are exact and g_p is applied in float64; each
    range's partial is rounded to float32 (within 2^-24 of Σ_p |g_p| Σ_range
    |rounded h_p*x|). The fp32 output rounding is covered separately
    (2^-23 |y|)."""
    xb = np.atleast_2d(xv)
    B, K = xb.shape
    bound = np.zeros((B, d.g1.shape[0]))
    for g, h in ((d.g1, d.h1), (d.g2, d.h2)):
        u = np.abs(h.astype(np.float64)[None, :] * xb)
        tot = np.zeros(B)
        for c0 in range(0, K, 512):
            mr = u[:, c0:c0 + 512].max(axis=1)
            _, e = np.frexp(mr)  # mr = f 2^e, f in [0.5, 1): ilogb = e - 1
            tot += np.where(mr > 0, min(512, K - c0) * np.exp2(e - 1.0 - 19.0), 0.0)
        # the float32 rounding of every range's partial
        part = 2.0 ** -24 * (u.sum(axis=1) + tot)
        bound += np.abs(g.astype(np.float64))[None, :] * (tot + part)[:, None]
    return bound


def f16_bound(d, xv):
    """Elementwise error bound of the fp16 matrix-core path (batches from
    RABIT_GEMV_FP16_MIN_BATCH on), as rabit.h states it.

    Per (token, chunk of ranges) x is scaled by a power of two, 2^-e at most
    max|x| / 2^14, and rounded to fp16 (exact above 2^-32 of the chunk's
    largest |x|; below that off by at most 2^-25 2^-e); the products with
    ±h_p are exact and summed in fp32 over the chunk (at most in + 16 S
    roundings, each within 2^-24 of a running sum bounded by Σ|h_p x|); g_p is
    applied in float64 and each chunk's partial rounded to float32 (one more
    rounding per chunk, at most S of them)."""
    xb = np.atleast_2d(xv)
    B, K = xb.shape
    S = -(-K // 512)
    bound = np.zeros((B, d.g1.shape[0]))
    xmax = np.abs(xb).max(axis=1)
    for s_, g, h in d.paths:
        ha = np.abs(h.astype(np.float64))
        acc = (K + 17 * S) * 2.0 ** -24 * (np.abs(xb) @ ha) + ha.sum() * 2.0 ** -25 * xmax * 2.0 ** -14
        bound += np.abs(g.astype(np.float64))[None, :] * acc[:, None]
    return bound


def check_fx(y, ref, d, xv):
    """The elementwise bound of the arithmetic the batch size selects."""
    from bit_residual_binarized_amd import rabit
    xb = np.atleast_2d(xv)
    fx = f16_bound(d, xb) if xb.shape[0] >= rabit.GEMV_FP16_MIN_BATCH else fx_bound(d, xb)
    bound = fx + 2.0 ** -23 * np.abs(ref) + 1e-300
    bad = np.argwhere(np.abs(y - ref) > bound)
    assert bad.size == 0, f"{len(bad)} outputs outside the bound, first {bad[:3].tolist()}"


PACK_SHAPES = [(4, 8), (64, 256), (100, 300), (130, 1000), (1, 1), (65, 129), (256, 4096),
               (1024, 4096), (4096, 4096)]


@pytest.mark.parametrize("shape", PACK_SHAPES)
def test_pack_meanabs_bit_exact(gpu_lib, shape):
    out, inp = shape
    say("pack meanabs", shape)
    w = weight_f32(out, inp, 1000 + out + inp)
    layer = pack_gpu(gpu_lib, w)
    d = oracle.derive(w.numpy())
    check_pack(gpu_lib, layer, d, out, inp)


def test_pack_given_scales_bit_exact(gpu_lib):
    out, inp = 300, 700
    say("pack given", out, inp)
    w = weight_f32(out, inp, 77)
    g, h = random_f16_scales(out, 1), random_f16_scales(inp, 2)
    layer = pack_gpu(gpu_lib, w, gpu_lib.RABIT_SCALES_GIVEN, g, h)
    d = oracle.derive(w.numpy(), mode="given", g1=g, h1=h)
    check_pack(gpu_lib, layer, d, out, inp, check_scales=False)


def test_pack_edge_values(gpu_lib):
    # zeros, negative zeros, engineered |W| == g1 h1 ties, a zero row/column,
    # float32 subnormals
    out, inp = 64, 256
    say("pack edge values")
    w = weight_f32(out, inp, 88).numpy().copy()
    w[3] = 0.0
    w[:, 5] = -0.0
    w[7, :20] = np.float32(1e-40)
    w[8, :20] = -np.float32(3e-42)
    wt = torch.from_numpy(w)
    layer = pack_gpu(gpu_lib, wt)
    d = oracle.derive(w)
    check_pack(gpu_lib, layer, d, out, inp)
    # ties: W = ±g1 h1 exactly, with given scales
    g = np.full(out, 0.5, np.float16)
    h = np.full(inp, 0.25, np.float16)
    w2 = np.where(np.arange(inp)[None, :] % 2 == 0, 0.125, -0.125).astype(np.float32) * np.ones((out, 1), np.float32)
    layer = pack_gpu(gpu_lib, torch.from_numpy(w2), gpu_lib.RABIT_SCALES_GIVEN, g, h)
    d = oracle.derive(w2, mode="given", g1=g, h1=h)
    check_pack(gpu_lib, layer, d, out, inp, check_scales=False)


def test_pack_repeatable(gpu_lib):
    say("pack repeatable")
    w = weight_f32(512, 1024, 99)
    a = pack_gpu(gpu_lib, w)
    b = pack_gpu(gpu_lib, w)
    assert torch.equal(a.planes, b.planes) and torch.equal(a.g, b.g) and torch.equal(a.h, b.h)


def test_f64_to_f16_and_bf16_rounding(gpu_lib):
    say("f64 -> fp16/bf16 rounding")
    allh = np.arange(0, 0x7C00, dtype=np.uint16).view(np.float16).astype(np.float64)
    mids = (allh[:-1] + allh[1:]) / 2.0
    rng = np.random.default_rng(5)
    extra = np.concatenate([rng.standard_normal(100000) * np.exp2(rng.integers(-30, 18, 100000)),
                            [0.0, -0.0, 65504.0, 65519.99, 65520.0, 1e6, 2.0 ** -25, 2.0 ** -24]])
    v = np.concatenate([mids, np.nextafter(mids, np.inf), np.nextafter(mids, -np.inf), extra])
    v = np.concatenate([v, -v])
    got = gpu_lib.test_f64_to_16(torch.from_numpy(v).cuda(), bf16=False).cpu().numpy().view(np.uint16)
    ref = oracle.f16_rne(v).view(np.uint16)
    assert np.array_equal(got, ref)
    vb = np.concatenate([rng.standard_normal(200000) * np.exp2(rng.integers(-140, 120, 200000)),
                         [0.0, 1.0 + 2.0 ** -8, 1.0 + 2.0 ** -8 + 2.0 ** -30, 3.4e38, 3.4e39]])
    gotb = gpu_lib.test_f64_to_16(torch.from_numpy(vb).cuda(), bf16=True).cpu().numpy().view(np.uint16)
    refb = oracle.bf16_rne(vb).astype(np.float32).view(np.uint32) >> 16
    assert np.array_equal(gotb, refb.astype(np.uint16))
    # the short path of the RMSNorm prologues: halfway cases of every binade's
    # mantissa pattern both ways, random values, the carry into the exponent
    # and the edges of its range (outside it: the general conversion)
    mant = rng.integers(0, 128, 50000)
    ex = rng.integers(-130, 128, 50000)
    half = (1.0 + mant / 128.0 + 2.0 ** -8) * np.exp2(ex.astype(np.float64))  # exactly halfway
    vf = np.concatenate([vb, half, -half, np.nextafter(half, 0), np.nextafter(half, np.inf),
                         [2.0 ** -126, 2.0 ** -127, 2.0 ** 127 * (2 - 2.0 ** -9), 2.0 ** 128, 1.0 - 2.0 ** -10]])
    gotf = gpu_lib.test_f64_to_16(torch.from_numpy(vf).cuda(), bf16=2).cpu().numpy().view(np.uint16)
    reff = oracle.bf16_rne(vf).astype(np.float32).view(np.uint32) >> 16
    assert np.array_equal(gotf, reff.astype(np.uint16))


GEMV_SHAPES = [(4, 8), (64, 256), (100, 300), (130, 1000), (65, 129), (1, 4096), (4096, 4096),
               (11008, 4096), (4096, 11008), (1024, 4096), (512, 14336)]


@pytest.mark.parametrize("shape", GEMV_SHAPES)
def test_gemv_batch1(gpu_lib, shape):
    out, inp = shape
    say("gemv b=1", shape)
    w = weight_f32(out, inp, 2000 + out + inp)
    layer = pack_gpu(gpu_lib, w)
    d = oracle.derive(w.numpy())
    x = act_bf16(1, inp, 3000 + inp)
    y = gpu_lib.gemv(layer, x.cuda()).cpu().numpy().astype(np.float64)
    ref = oracle.gemv(d, bf16_values(x))
    err = oracle.normwise_rel_err(y, ref)
    say("  normwise err", err)
    assert err < TOL
    check_fx(y, ref, d, bf16_values(x))
    y2 = gpu_lib.gemv(layer, x.cuda()).cpu().numpy()
    assert np.array_equal(y.astype(np.float32), y2), "not repeatable"


@pytest.mark.parametrize("batch", [2, 3, 4, 8, 16, 25, 32])
def test_gemv_batches(gpu_lib, batch):
    out, inp = 1024, 4096
    say("gemv batch", batch)
    w = weight_f32(out, inp, 4000 + batch)
    layer = pack_gpu(gpu_lib, w)
    d = oracle.derive(w.numpy())
    x = act_bf16(batch, inp, seed_x(3, batch))
    y = gpu_lib.gemv(layer, x.cuda()).cpu().numpy().astype(np.float64)
    ref = oracle.gemv(d, bf16_values(x))
    err = oracle.normwise_rel_err(y, ref)
    say("  normwise err", err)
    assert err < TOL
    check_fx(y, ref, d, bf16_values(x))


def test_gemv_unit_vector_probe_bit_exact(gpu_lib):
    out, inp = 256, 640
    say("gemv unit probes")
    w = weight_f32(out, inp, 5)
    layer = pack_gpu(gpu_lib, w)
    d = oracle.derive(w.numpy())
    we = oracle.weff(d)
    for j in (0, 1, 127, 128, 333, 639):
        x = torch.zeros(1, inp, dtype=torch.bfloat16)
        x[0, j] = 1.0
        y = gpu_lib.gemv(layer, x.cuda()).cpu().numpy()
        assert np.array_equal(y[0], we[:, j].astype(np.float32)), j


def test_gemv_bf16_output_and_outlier_input(gpu_lib):
    out, inp = 512, 2048
    say("gemv bf16 out + outliers")
    w = weight_f32(out, inp, 6)
    layer = pack_gpu(gpu_lib, w)
    d = oracle.derive(w.numpy())
    x = act_bf16(2, inp, 7)
    x[0, 17] = 3000.0   # a massive activation
    x[1, 100:110] = 1e-30
    ref = oracle.gemv(d, bf16_values(x))
    yf = gpu_lib.gemv(layer, x.cuda()).cpu().numpy().astype(np.float64)
    assert oracle.normwise_rel_err(yf, ref) < TOL
    check_fx(yf, ref, d, bf16_values(x))
    yb = gpu_lib.gemv(layer, x.cuda(), y_dtype=gpu_lib.RABIT_OUT_BF16).cpu().to(torch.float32).numpy()
    assert oracle.normwise_rel_err(yb.astype(np.float64), ref) < 2 ** -8


@pytest.mark.parametrize("shape", [(1000, 3000), (300, 512), (4096, 11008)])
def test_gemv_partial_reduce_equals_gemv(gpu_lib, shape):
    out, inp = shape
    say("gemv partial/reduce", shape)
    layer = pack_gpu(gpu_lib, weight_f32(out, inp, 8))
    for batch in (1, 3, 12):
        x = act_bf16(batch, inp, 9 + batch).cuda()
        ws = gpu_lib.gemv_workspace(layer, batch)
        y = torch.empty(batch, out, device="cuda")
        gpu_lib.gemv_partial(layer, x, ws)
        gpu_lib.gemv_reduce(layer, batch, y, ws)
        assert torch.equal(y, gpu_lib.gemv(layer, x))


def test_gemv_partial_multi_equals_gemv(gpu_lib):
    say("gemv partial multi")
    inp = 1100
    layers = [pack_gpu(gpu_lib, weight_f32(o, inp, 20 + o)) for o in (300, 64, 130)]
    for batch in (1, 2, 5, 9, 32):
        x = act_bf16(batch, inp, 30 + batch).cuda()
        ws = gpu_lib.gemv_multi_workspace(layers, batch)
        views = gpu_lib.gemv_partial_multi(layers, x, ws)
        for L, v in zip(layers, views):
            y = torch.empty(batch, L.out_features, device="cuda")
            gpu_lib.gemv_reduce(L, batch, y, v)
            assert torch.equal(y, gpu_lib.gemv(L, x))


# (256, 4100, 64): 66 K steps over 14 split-K slices of 5, the last one of a single step
# M <= 32 takes the small-token tiles: (256, 14336, 16) splits K 32 ways,
# (300, 1100, 31) is ragged in every dimension
GEMM_CASES = [(64, 256, 1), (130, 1000, 37), (256, 4096, 512), (1024, 4096, 130), (300, 1100, 257),
              (256, 4100, 64), (1024, 4096, 8), (256, 14336, 16), (300, 1100, 31), (4096, 1024, 32)]


@pytest.mark.parametrize("case", GEMM_CASES)
def test_gemm(gpu_lib, case):
    out, inp, m = case
    say("gemm", case)
    w = weight_f32(out, inp, 6000 + m)
    layer = pack_gpu(gpu_lib, w)
    d = oracle.derive(w.numpy())
    xm = act_bf16(m, inp, 7000 + m)
    y = gpu_lib.gemm(layer, xm.cuda()).cpu().numpy().astype(np.float64)
    ref = oracle.gemm(d, bf16_values(xm))
    err = oracle.normwise_rel_err(y, ref)
    say("  normwise err", err)
    assert err < TOL


def test_gemm_rows_match_gemv(gpu_lib):
    out, inp, m = 512, 2048, 40
    say("gemm vs gemv rows")
    layer = pack_gpu(gpu_lib, weight_f32(out, inp, 10))
    xm = act_bf16(m, inp, 11).cuda()
    ym = gpu_lib.gemm(layer, xm).cpu().numpy().astype(np.float64)
    for r in (0, 17, 39):
        yv = gpu_lib.gemv(layer, xm[r:r + 1].contiguous()).cpu().numpy().astype(np.float64)
        assert oracle.normwise_rel_err(ym[r:r + 1], yv) < 1e-5


def _decode_case(gpu_lib, cfg, mlp_only, batch, seed, repeats=1):
    H, F = cfg.hidden, cfg.ffn
    kv = cfg.n_kv_heads * cfg.head_dim
    shapes = {"q": (H, H), "k": (kv, H), "v": (kv, H), "o": (H, H), "gate": (F, H), "up": (F, H), "down": (H, F)}
    names = ["gate", "up", "down"] if mlp_only else list(shapes)
    layers, dmats = [], []
    for li in range(cfg.n_layers):
        ld, dd = {}, {}
        for n in names:
            w = weight_f32(*shapes[n], seed + 10 * li + len(n))
            ld[n] = pack_gpu(gpu_lib, w)
            dd[n] = oracle.derive(w.numpy())
        layers.append(ld)
        dmats.append(dd)
    x = act_bf16(batch, H, seed + 99)
    ys = [gpu_lib.decode_step(cfg, layers, x.cuda()).cpu().to(torch.float32).numpy().astype(np.float64)
          for _ in range(repeats)]
    y = ys[0] if repeats == 1 else ys
    ref = bf16_values(x)
    ocfg = {"n_heads": cfg.n_heads, "n_kv_heads": cfg.n_kv_heads, "head_dim": cfg.head_dim, "rms_eps": cfg.rms_eps}
    for dd in dmats:
        ref = oracle.decode_layer(ref, dd, ocfg)
    return y, ref


def bf16_close(y, ref, tol=TOL):
    """|y - ŷ| <= tol * max|ŷ| (per batch row) + one bf16 ulp of ŷ, elementwise:
    both sides round nearly equal values to bf16, so a rounding boundary can
    fall between them (one ulp, up to 2^-8 relative)."""
    y = np.atleast_2d(y)
    ref = np.atleast_2d(ref)
    a = np.abs(ref)
    ulp = np.exp2(np.floor(np.log2(np.where(a > 0, a, 1.0))) - 7)
    allow = tol * a.max(axis=1, keepdims=True) + ulp
    bad = np.abs(y - ref) > allow
    return not bad.any(), int(bad.sum())


def test_decode_mlp_block(gpu_lib):
    say("decode mlp block")
    cfg = gpu_lib.DecoderCfg(hidden=1024, ffn=2752, n_layers=2, mlp_only=True)
    y, ref = _decode_case(gpu_lib, cfg, True, 1, 500)
    err = oracle.normwise_rel_err(y, ref)
    ok, nbad = bf16_close(y, ref)
    say("  normwise err", err, "elements outside bound", nbad)
    assert ok


def test_decode_llama7b_mlp_block(gpu_lib):
    # the benchmarked workload: one Llama-2-7B-shaped MLP block at batch 1
    say("decode llama-2-7b mlp block")
    cfg = gpu_lib.DecoderCfg(hidden=4096, ffn=11008, n_layers=1, mlp_only=True)
    y, ref = _decode_case(gpu_lib, cfg, True, 1, 700)
    ok, nbad = bf16_close(y, ref)
    say("  normwise err", oracle.normwise_rel_err(y, ref), "elements outside bound", nbad)
    assert ok


@pytest.mark.parametrize("mlp_only", [True, False])
def test_decode_batch1_inputs_from_partials_match_batch2(gpu_lib, mlp_only):
    # every step of a decode step is per batch row (fixed-point scales per
    # row and range, RMS statistics per row), and batch 1 and batch 2 run the
    # same kernels with one or two live rows: row 0 must match bit for bit
    say("decode batch 1 vs row 0 of batch 2, mlp_only", mlp_only)
    cfg = gpu_lib.DecoderCfg(hidden=1024, ffn=2752, n_heads=8, n_kv_heads=2, head_dim=128, n_layers=2,
                             mlp_only=mlp_only)
    H, F, kv = cfg.hidden, cfg.ffn, cfg.n_kv_heads * cfg.head_dim
    shapes = {"q": (H, H), "k": (kv, H), "v": (kv, H), "o": (H, H), "gate": (F, H), "up": (F, H), "down": (H, F)}
    names = ["gate", "up", "down"] if mlp_only else list(shapes)
    layers = [{n: pack_gpu(gpu_lib, weight_f32(*shapes[n], 900 + 10 * li + len(n))) for n in names}
              for li in range(cfg.n_layers)]
    x2 = act_bf16(2, H, 991).cuda()
    y1 = gpu_lib.decode_step(cfg, layers, x2[:1].contiguous()).cpu()
    y2 = gpu_lib.decode_step(cfg, layers, x2).cpu()
    assert torch.equal(y1[0].view(torch.int16), y2[0].view(torch.int16))


def test_decode_batch1_wide_hidden(gpu_lib):
    # 9 input ranges per hidden row, 36 query heads over 4 key/value groups
    say("decode batch 1, hidden 4608")
    cfg = gpu_lib.DecoderCfg(hidden=4608, ffn=1024, n_heads=36, n_kv_heads=4, head_dim=128, n_layers=1)
    y, ref = _decode_case(gpu_lib, cfg, False, 1, 800)
    ok, nbad = bf16_close(y, ref)
    say("  normwise err", oracle.normwise_rel_err(y, ref), "elements outside bound", nbad)
    assert ok


@pytest.mark.parametrize("batch", [1, 2, 4, 20, 40])
def test_decode_attention_block(gpu_lib, batch):
    say("decode attention block batch", batch)
    cfg = gpu_lib.DecoderCfg(hidden=512, ffn=1376, n_heads=8, n_kv_heads=2, head_dim=64, n_layers=2)
    y, ref = _decode_case(gpu_lib, cfg, False, batch, 600 + batch)
    err = oracle.normwise_rel_err(y, ref)
    ok, nbad = bf16_close(y, ref)
    say("  normwise err", err, "elements outside bound", nbad)
    assert ok


@pytest.mark.parametrize("batch", [1, 3, 7, 9])
def test_decode_steps_repeatable(gpu_lib, batch):
    # ragged shapes (hidden 768, 128 rows of k and v, ffn 1100), batch groups
    # of 1, 2 and 4 workgroups per range and the fp16 path: three steps on
    # the same input give the same bits, close to the oracle
    say("decode repeatable batch", batch)
    cfg = gpu_lib.DecoderCfg(hidden=768, ffn=1100, n_heads=6, n_kv_heads=1, head_dim=128, n_layers=3)
    ys, ref = _decode_case(gpu_lib, cfg, False, batch, 1300 + batch, repeats=3)
    assert np.array_equal(ys[0], ys[1]) and np.array_equal(ys[0], ys[2])
    ok, nbad = bf16_close(ys[0], ref)
    say("  normwise err", oracle.normwise_rel_err(ys[0], ref), "elements outside bound", nbad)
    assert ok


@pytest.mark.parametrize("hidden,n_heads,n_kv", [(1024, 8, 2), (512, 8, 2), (4608, 36, 4)])
def test_decode_qk_sums_batch1(gpu_lib, hidden, n_heads, n_kv):
    # at batch 1 the o launch also sums the q and k partials of the layer
    # (rows spread over its work items, more than 256 per item at hidden 512);
    # the workspace keeps the last layer's q and k in fp32 after x, x, the
    # attention output, z and the x^2 statistics (256-byte aligned areas)
    say("decode q/k sums at batch 1, hidden", hidden)
    hd = hidden // n_heads
    cfg = gpu_lib.DecoderCfg(hidden=hidden, ffn=768, n_heads=n_heads, n_kv_heads=n_kv, head_dim=hd, n_layers=1)
    H, F, kv = hidden, cfg.ffn, n_kv * hd
    shapes = {"q": (H, H), "k": (kv, H), "v": (kv, H), "o": (H, H), "gate": (F, H), "up": (F, H), "down": (H, F)}
    ws_, d = {}, {}
    for i, (n, sh) in enumerate(shapes.items()):
        w = weight_f32(*sh, 1400 + i)
        ws_[n] = pack_gpu(gpu_lib, w)
        d[n] = oracle.derive(w.numpy())
    x = act_bf16(1, H, 1499)
    work = gpu_lib.decode_workspace(cfg, 1)
    gpu_lib.decode_step(cfg, [ws_], x.cuda(), workspace=work)
    torch.cuda.synchronize()
    a = lambda n: (n + 255) // 256 * 256
    off = 3 * a(2 * H) + a(2 * F) + a(8 * 32)
    qk = work[off:off + 4 * (H + kv)].view(torch.float32).cpu().numpy().astype(np.float64)
    n = oracle.rmsnorm_bf16(bf16_values(x))
    for name, got in (("q", qk[:H]), ("k", qk[H:])):
        ref = oracle.gemv(d[name], n)[0]
        check_fx(got[None, :], ref[None, :], d[name], n)


def test_stream_read_runs(gpu_lib):
    # the measurement hook reads a buffer (whole tiles and a ragged tail)
    say("stream read hook")
    t = torch.ones(3001 * 4 + (64 << 18), dtype=torch.int32, device="cuda")
    sink = gpu_lib.stream_read(t)
    torch.cuda.synchronize()
    assert sink.numel() == 4


@pytest.mark.parametrize("shape", [(64, 256), (130, 1000), (1024, 4096), (11008, 4096)])
def test_pack_meanabs_normalized_bit_exact(gpu_lib, shape):
    # h divided by the matrix's global mean |.| (canonical total of the row sums)
    out, inp = shape
    say("pack meanabs normalized", shape)
    w = weight_f32(out, inp, 1500 + out + inp)
    layer = pack_gpu(gpu_lib, w, gpu_lib.RABIT_SCALES_MEANABS_NORMALIZED)
    d = oracle.derive(w.numpy(), mode="meanabs_normalized")
    check_pack(gpu_lib, layer, d, out, inp)
    x = act_bf16(2, inp, 1600 + inp)
    y = gpu_lib.gemv(layer, x.cuda()).cpu().numpy().astype(np.float64)
    ref = oracle.gemv(d, bf16_values(x))
    assert oracle.normwise_rel_err(y, ref) < TOL
    check_fx(y, ref, d, bf16_values(x))


def test_pack_meanabs_normalized_three_paths_and_zero(gpu_lib):
    out, inp = 200, 700
    say("pack meanabs normalized, three paths and a zero matrix")
    w = weight_f32(out, inp, 1700)
    layer = gpu_lib.PackedLayer.empty(out, inp, n_paths=3)
    gpu_lib.pack(w.cuda(), layer, gpu_lib.RABIT_SCALES_MEANABS_NORMALIZED)
    d = oracle.derive(w.numpy(), mode="meanabs_normalized", n_paths=3)
    words = gpu_lib.unpack(layer).cpu().numpy().view(np.uint32)
    for p, (s, g, h) in enumerate(d.paths):
        assert np.array_equal(words[p], oracle.pack_words(s)), p
        assert np.array_equal(layer.g[p].cpu().numpy().view(np.uint16), g.view(np.uint16)), p
        assert np.array_equal(layer.h[p].cpu().numpy().view(np.uint16), h.view(np.uint16)), p
    z = pack_gpu(gpu_lib, torch.zeros(64, 300), gpu_lib.RABIT_SCALES_MEANABS_NORMALIZED)
    assert not z.g.any() and not z.h.any() and not z.planes.any()


# The fp16 matrix-core path (batches 8 .. 32): ragged shapes, a chunk that
# ends inside the last range, three paths, bf16 output, outlier and tiny
# activations, zero token rows.
F16_CASES = [(65, 129, 8), (300, 1100, 31), (1024, 4096, 16), (130, 5000, 17), (4096, 14336, 32), (256, 4100, 12),
             (2048, 8192, 24)]


@pytest.mark.parametrize("case", F16_CASES)
def test_gemv_fp16_path(gpu_lib, case):
    out, inp, batch = case
    say("gemv fp16 path", case)
    w = weight_f32(out, inp, 8000 + out + batch)
    layer = pack_gpu(gpu_lib, w)
    d = oracle.derive(w.numpy())
    x = act_bf16(batch, inp, 8100 + batch)
    x[0, inp // 3] = 2000.0                 # an outlier sets token 0's exponent
    x[1, :] = 0.0                           # a zero token row
    x[2, : min(inp, 700)] = 1e-30           # tiny values in the first ranges
    xv = bf16_values(x)
    y = gpu_lib.gemv(layer, x.cuda()).cpu().numpy().astype(np.float64)
    ref = oracle.gemv(d, xv)
    err = oracle.normwise_rel_err(np.delete(y, 1, 0), np.delete(ref, 1, 0))
    say("  normwise err", err)
    assert err < TOL
    assert not y[1].any()
    check_fx(y, ref, d, xv)
    yb = gpu_lib.gemv(layer, x.cuda(), y_dtype=gpu_lib.RABIT_OUT_BF16).cpu().to(torch.float32).numpy()
    assert oracle.normwise_rel_err(np.delete(yb.astype(np.float64), 1, 0), np.delete(ref, 1, 0)) < 2 ** -8


def test_gemv_fp16_path_three_paths(gpu_lib):
    out, inp, batch = 500, 3000, 20
    say("gemv fp16 path, three paths")
    w = weight_f32(out, inp, 8200)
    layer = gpu_lib.PackedLayer.empty(out, inp, n_paths=3)
    gpu_lib.pack(w.cuda(), layer)
    d = oracle.derive(w.numpy(), n_paths=3)
    x = act_bf16(batch, inp, 8201)
    xv = bf16_values(x)
    y = gpu_lib.gemv(layer, x.cuda()).cpu().numpy().astype(np.float64)
    ref = oracle.gemv(d, xv)
    assert oracle.normwise_rel_err(y, ref) < TOL
    bound = f16_bound(d, xv) + 2.0 ** -23 * np.abs(ref)
    assert (np.abs(y - ref) <= bound).all()


def test_gemv_rows_same_for_every_batch_on_fp16_path(gpu_lib):
    # a token's result does not depend on the other tokens of the batch
    # (exponents per token, no cross-token arithmetic): batches that share a
    # launch plan (token tiles of 16 up to batch 16, of 32 above) agree bit
    # for bit
    out, inp = 1024, 4096
    say("gemv fp16 path: rows independent of the batch")
    layer = pack_gpu(gpu_lib, weight_f32(out, inp, 8300))
    x = act_bf16(32, inp, 8301).cuda()
    for lo, hi in ((9, 16), (17, 32)):
        yhi = gpu_lib.gemv(layer, x[:hi].contiguous())
        ylo = gpu_lib.gemv(layer, x[:lo].contiguous())
        assert torch.equal(yhi[:lo], ylo), (lo, hi)
