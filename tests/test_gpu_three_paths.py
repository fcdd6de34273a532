"""GPU parity of the 3-path (3-bit) variant through the C ABI against the
CPU oracle: packed words of all three planes, the device layout and the fp16
scales of every path bit-exact."""
import numpy as np
import pytest
import torch

import oracle
from synth.inputs import weight_f32, random_f16_scales

pytestmark = pytest.mark.gpu


def say(*a):
    print("[case]", *a, flush=True)


def pack3(rabit, w, mode=None, g=None, h=None):
    mode = rabit.RABIT_SCALES_MEANABS if mode is None else mode
    out, inp = w.shape
    layer = rabit.PackedLayer.empty(out, inp, n_paths=3)
    if g is not None:
        layer.g.copy_(torch.from_numpy(np.stack(g).astype(np.float16)).view(torch.int16))
        layer.h.copy_(torch.from_numpy(np.stack(h).astype(np.float16)).view(torch.int16))
    rabit.pack(torch.from_numpy(np.ascontiguousarray(w)).cuda(), layer, mode)
    torch.cuda.synchronize()
    return layer


def check3(rabit, layer, d, check_scales=True):
    out, inp = d.shape
    words = rabit.unpack(layer).cpu().numpy().view(np.uint32)
    ref = [oracle.pack_words(s) for s, _, _ in d.paths]
    for p in range(3):
        bad = np.argwhere(words[p] != ref[p])
        assert bad.size == 0, f"path {p + 1}: {len(bad)} words differ, first {bad[:3].tolist()}"
    raw = layer.planes.cpu().numpy().view(np.uint32)
    assert np.array_equal(raw, oracle.device_planes(ref[0], ref[1], out, inp, ref[2])), "device layout differs"
    if check_scales:
        g = layer.g.cpu().numpy().view(np.float16)
        h = layer.h.cpu().numpy().view(np.float16)
        for p, (_, gr, hr) in enumerate(d.paths):
            for name, got, want in ((f"g{p + 1}", g[p], gr), (f"h{p + 1}", h[p], hr)):
                bad = np.flatnonzero(got.view(np.uint16) != want.view(np.uint16))
                assert bad.size == 0, f"{name}: {bad.size} fp16 scales differ, first at {bad[:5]}"


@pytest.mark.parametrize("shape", [(4, 8), (64, 256), (100, 300), (130, 1000), (1, 1), (65, 129),
                                   (1024, 4096), (4096, 4096)])
def test_pack3_meanabs_bit_exact(gpu_lib, shape):
    out, inp = shape
    say("pack 3 paths meanabs", shape)
    w = weight_f32(out, inp, 3000 + out + inp).numpy()
    layer = pack3(gpu_lib, w)
    check3(gpu_lib, layer, oracle.derive(w, n_paths=3))


def test_pack3_given_scales_bit_exact(gpu_lib):
    out, inp = 300, 700
    say("pack 3 paths given", out, inp)
    w = weight_f32(out, inp, 3077).numpy()
    g = [random_f16_scales(out, s) for s in (31, 32, 33)]
    h = [random_f16_scales(inp, s) for s in (34, 35, 36)]
    layer = pack3(gpu_lib, w, gpu_lib.RABIT_SCALES_GIVEN, g, h)
    d = oracle.derive(w, mode="given", g1=g[0], h1=h[0], g2=g[1], h2=h[1], g3=g[2], h3=h[2], n_paths=3)
    check3(gpu_lib, layer, d, check_scales=False)


def test_pack3_residual_ties_and_zeros(gpu_lib):
    # engineered R_1 = ±e_2 (R_2 = +0, bit 0) and R_1 = ±0 (R_2 = -e_2, bit 1)
    out, inp = 64, 256
    say("pack 3 paths ties")
    g = [np.full(out, 0.5, np.float16), np.full(out, 0.25, np.float16), np.full(out, 1.0, np.float16)]
    h = [np.full(inp, 0.25, np.float16), np.full(inp, 0.25, np.float16), np.full(inp, 1.0, np.float16)]
    pattern = np.array([0.1875, 0.0625, 0.125, -0.125, -0.1875, -0.0625, 0.0, -0.0], np.float32)
    w = np.tile(pattern, (out, inp // 8))
    layer = pack3(gpu_lib, w, gpu_lib.RABIT_SCALES_GIVEN, g, h)
    d = oracle.derive(w, mode="given", g1=g[0], h1=h[0], g2=g[1], h2=h[1], g3=g[2], h3=h[2], n_paths=3)
    assert d.s3.any() and not d.s3.all()
    check3(gpu_lib, layer, d, check_scales=False)
    # mean-|.| scales on data with zero rows and columns and subnormals
    w2 = weight_f32(out, inp, 3088).numpy().copy()
    w2[3] = 0.0
    w2[:, 5] = -0.0
    w2[7, :20] = np.float32(1e-40)
    layer = pack3(gpu_lib, w2)
    check3(gpu_lib, layer, oracle.derive(w2, n_paths=3))


def test_pack3_first_two_paths_match_two_path_pack(gpu_lib):
    # the 3-path derivation extends the 2-path one: planes 1-2 and their
    # scales are the same bits as a 2-path pack of the same weight
    out, inp = 256, 1024
    say("pack 3 vs 2 paths")
    w = weight_f32(out, inp, 3099)
    l3 = pack3(gpu_lib, w.numpy())
    l2 = gpu_lib.PackedLayer.empty(out, inp)
    gpu_lib.pack(w.cuda(), l2)
    torch.cuda.synchronize()
    u3, u2 = gpu_lib.unpack(l3), gpu_lib.unpack(l2)
    assert torch.equal(u3[:2], u2)
    assert torch.equal(l3.g[:2], l2.g) and torch.equal(l3.h[:2], l2.h)


# ---- GEMV and decode with three paths -----------------------------------
from synth.inputs import act_bf16, bf16_values  # noqa: E402

TOL = 2e-3


def fx_bound(d, xv):
    """Elementwise bound of the GEMV arithmetic (rabit.h): per (batch row, path,
    512-column range) h_p*x on a grid of step 2^(ilogb(max |h_p*x|) - 18),
    exact signed sums, g_p in float64, each range's partial rounded to
    float32; summed over the paths."""
    xb = np.atleast_2d(xv)
    B, K = xb.shape
    bound = np.zeros((B, d.g1.shape[0]))
    for _, g, h in d.paths:
        u = np.abs(h.astype(np.float64)[None, :] * xb)
        tot = np.zeros(B)
        for c0 in range(0, K, 512):
            mr = u[:, c0:c0 + 512].max(axis=1)
            _, e = np.frexp(mr)
            tot += np.where(mr > 0, min(512, K - c0) * np.exp2(e - 1.0 - 19.0), 0.0)
        # the float32 rounding of every range's partial
        part = 2.0 ** -24 * (u.sum(axis=1) + tot)
        bound += np.abs(g.astype(np.float64))[None, :] * (tot + part)[:, None]
    return bound


def check_gemv3(y, ref, d, xv):
    # the bound of the arithmetic the batch size selects (fixed point below
    # the fp16 path's threshold, fp32 accumulation from it on)
    from bit_residual_binarized_amd import rabit
    from test_gpu_parity import f16_bound
    xb = np.atleast_2d(xv)
    fx = f16_bound(d, xb) if xb.shape[0] >= rabit.GEMV_FP16_MIN_BATCH else fx_bound(d, xb)
    bound = fx + 2.0 ** -23 * np.abs(ref) + 1e-300
    bad = np.argwhere(np.abs(y - ref) > bound)
    assert bad.size == 0, f"{len(bad)} outputs outside the bound, first {bad[:3].tolist()}"
    assert oracle.normwise_rel_err(y, ref) < TOL


@pytest.mark.parametrize("shape", [(64, 512), (100, 300), (130, 1000), (1, 1), (1024, 4096),
                                   (4096, 4096), (11008, 4096)])
def test_gemv3_batch1(gpu_lib, shape):
    out, inp = shape
    say("gemv 3 paths b=1", shape)
    w = weight_f32(out, inp, 3100 + out + inp).numpy()
    layer = pack3(gpu_lib, w)
    d = oracle.derive(w, n_paths=3)
    x = act_bf16(1, inp, 3101)
    y = gpu_lib.gemv(layer, x.cuda()).cpu().numpy().astype(np.float64)
    xv = bf16_values(x)
    check_gemv3(y, oracle.gemv(d, xv), d, xv)
    # repeatable bit for bit
    y2 = gpu_lib.gemv(layer, x.cuda()).cpu().numpy().astype(np.float64)
    assert np.array_equal(y, y2)


@pytest.mark.parametrize("batch", [2, 3, 17, 32])
def test_gemv3_batches(gpu_lib, batch):
    out, inp = 1024, 4096
    say("gemv 3 paths batch", batch)
    w = weight_f32(out, inp, 3200 + batch).numpy()
    layer = pack3(gpu_lib, w)
    d = oracle.derive(w, n_paths=3)
    x = act_bf16(batch, inp, 3201 + batch)
    y = gpu_lib.gemv(layer, x.cuda()).cpu().numpy().astype(np.float64)
    xv = bf16_values(x)
    check_gemv3(y, oracle.gemv(d, xv), d, xv)
    # below the fp16 path's batch threshold every batch row equals the
    # batch-1 result of that row (the same exact fixed-point arithmetic);
    # from it on the rows agree with the batch-1 result to fp32 accumulation
    for r in (0, batch - 1):
        y1 = gpu_lib.gemv(layer, x[r:r + 1].contiguous().cuda()).cpu().numpy().astype(np.float64)
        if batch < gpu_lib.GEMV_FP16_MIN_BATCH:
            assert np.array_equal(y1[0], y[r])
        else:
            assert oracle.normwise_rel_err(y[r:r + 1], y1) < 1e-5


def test_gemv3_partial_multi_equals_gemv(gpu_lib):
    inp = 2048
    say("gemv 3 paths multi")
    ws_ = [weight_f32(o, inp, 3300 + o).numpy() for o in (512, 300)]
    layers = [pack3(gpu_lib, w) for w in ws_]
    x = act_bf16(2, inp, 3301).cuda()
    parts = gpu_lib.gemv_partial_multi(layers, x, gpu_lib.gemv_multi_workspace(layers, 2))
    for L, part in zip(layers, parts):
        ref = gpu_lib.gemv(L, x)
        y = gpu_lib.gemv_reduce(L, 2, torch.empty(2, L.out_features, device="cuda"), part)
        assert torch.equal(y, ref)


@pytest.mark.parametrize("batch", [1, 40])
def test_decode3_mlp_and_attention(gpu_lib, batch):
    # batch 40 runs the prefill GEMM path
    for mlp_only in (True, False):
        say("decode 3 paths, mlp_only", mlp_only, "batch", batch)
        cfg = gpu_lib.DecoderCfg(hidden=1024, ffn=2752, n_heads=8, n_kv_heads=2, head_dim=128, n_layers=2,
                                 mlp_only=mlp_only)
        H, F, kv = cfg.hidden, cfg.ffn, cfg.n_kv_heads * cfg.head_dim
        shapes = {"q": (H, H), "k": (kv, H), "v": (kv, H), "o": (H, H), "gate": (F, H), "up": (F, H),
                  "down": (H, F)}
        names = ["gate", "up", "down"] if mlp_only else list(shapes)
        layers, dmats = [], []
        for li in range(cfg.n_layers):
            ld, dd = {}, {}
            for n in names:
                w = weight_f32(*shapes[n], 3400 + 10 * li + len(n)).numpy()
                ld[n] = pack3(gpu_lib, w)
                dd[n] = oracle.derive(w, n_paths=3)
            layers.append(ld)
            dmats.append(dd)
        x = act_bf16(batch, H, 3499)
        y = gpu_lib.decode_step(cfg, layers, x.cuda()).cpu().to(torch.float32).numpy().astype(np.float64)
        ref = bf16_values(x)
        ocfg = {"n_heads": cfg.n_heads, "n_kv_heads": cfg.n_kv_heads, "head_dim": cfg.head_dim,
                "rms_eps": cfg.rms_eps}
        for dd in dmats:
            ref = oracle.decode_layer(ref, dd, ocfg)
        a = np.abs(ref)
        ulp = np.exp2(np.floor(np.log2(np.where(a > 0, a, 1.0))) - 7)
        allow = TOL * a.max(axis=1, keepdims=True) + ulp
        assert not (np.abs(y - ref) > allow).any()


def test_mixed_path_counts_are_rejected(gpu_lib):
    say("mixed path counts")
    inp = 512
    l2 = gpu_lib.PackedLayer.empty(256, inp)
    gpu_lib.pack(weight_f32(256, inp, 3501).cuda(), l2)
    l3 = pack3(gpu_lib, weight_f32(256, inp, 3502).numpy())
    x = act_bf16(1, inp, 3503).cuda()
    with pytest.raises(gpu_lib.RabitError):
        gpu_lib.gemv_partial_multi([l2, l3], x, gpu_lib.gemv_multi_workspace([l2, l3], 1))



# (256, 4100, 64): 66 K steps over 14 split-K slices of 5, the last one of a single step
@pytest.mark.parametrize("case", [(256, 512, 64), (300, 1000, 100), (1024, 4096, 200), (4096, 4096, 512),
                                  (100, 300, 1), (256, 4100, 64), (1024, 4096, 16), (300, 1100, 31)])
def test_gemm3(gpu_lib, case):
    out, inp, m = case
    say("gemm 3 paths", case)
    w = weight_f32(out, inp, 3600 + m).numpy()
    layer = pack3(gpu_lib, w)
    d = oracle.derive(w, n_paths=3)
    xm = act_bf16(m, inp, 3700 + m)
    y = gpu_lib.gemm(layer, xm.cuda()).cpu().numpy().astype(np.float64)
    ref = oracle.gemm(d, bf16_values(xm))
    assert oracle.normwise_rel_err(y, ref) < TOL


def test_gemm3_rows_match_gemv3(gpu_lib):
    out, inp, m = 512, 2048, 70
    say("gemm 3 vs gemv 3 rows")
    layer = pack3(gpu_lib, weight_f32(out, inp, 3800).numpy())
    xm = act_bf16(m, inp, 3801).cuda()
    ym = gpu_lib.gemm(layer, xm).cpu().numpy().astype(np.float64)
    for r in (0, 33, 69):
        yv = gpu_lib.gemv(layer, xm[r:r + 1].contiguous()).cpu().numpy().astype(np.float64)
        assert oracle.normwise_rel_err(ym[r:r + 1], yv) < 1e-5
