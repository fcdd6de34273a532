"""GPU parity at the full sizes of the workloads: Llama-2-70B layer shapes
(GEMV at batch 1 and 32, a two-layer decode slice, mean-|.| derive/pack),
the Llama-3-8B decoder layer and MLP prefill GEMM, and the Llama-2-13B
shapes of the pages' kernel table (RaBiT paper Table 7).

Where the float64 oracle would take minutes over a whole layer, it computes a
documented subset that it can evaluate on its own:

* output-row subsets: with given scales the derivation of a row needs only
  that row of W and the scales (paper §4.2 steps 1-3 are elementwise), so
  the oracle derives and multiplies the sampled rows only;
* token-row subsets of the prefill GEMM (256 token rows at M = 2048, 8192);
* the mean-|.| scales at a 70B shape are checked on their own, bit for bit,
  over the whole matrix.

Bars as elsewhere: packed words and fp16 scales bit-exact; GEMV outputs
within the fixed-point bound of the arithmetic (and 2e-3 normwise); GEMM
outputs within the fp32 accumulation bound (and 2e-3 normwise); decode
outputs within 2e-3 of max|ŷ| plus one bf16 ulp elementwise.
"""
import numpy as np
import pytest
import torch

import oracle
from synth.inputs import act_bf16, bf16_values, random_f16_scales, seed_w, seed_x, weight_f32
from test_gpu_parity import TOL, bf16_close, check_fx, check_pack, pack_gpu, say

pytestmark = pytest.mark.gpu

U32 = 2.0 ** -24  # unit roundoff of float32


def given_scales(out, inp, seed, n_paths=2):
    """fp16 scales around the magnitude mean-|.| gives for W ~ 0.02 N(0,1)
    (about 0.016 per factor for path 1, 0.013 for path 2)."""
    g = [random_f16_scales(out, seed, 0.010, 0.022)]
    h = [random_f16_scales(inp, seed + 1, 0.010, 0.022)]
    for p in range(1, n_paths):
        g.append(random_f16_scales(out, seed + 2 * p, 0.008, 0.018))
        h.append(random_f16_scales(inp, seed + 2 * p + 1, 0.008, 0.018))
    return np.stack(g), np.stack(h)


def pack_given(rabit, w_cpu, g, h):
    """Derive and pack on the GPU with every path's scales given."""
    out, inp = w_cpu.shape
    P = g.shape[0]
    layer = rabit.PackedLayer.empty(out, inp, n_paths=P)
    layer.g.copy_(torch.from_numpy(g).view(torch.int16))
    layer.h.copy_(torch.from_numpy(h).view(torch.int16))
    rabit.pack(w_cpu.cuda(), layer, rabit.RABIT_SCALES_GIVEN)
    torch.cuda.synchronize()
    return layer


def derive_rows(w_np, rows, g, h):
    """Oracle derivation of the output rows `rows` with given scales."""
    kw = dict(mode="given", g1=g[0][rows], h1=h[0], g2=g[1][rows], h2=h[1])
    if g.shape[0] == 3:
        kw.update(n_paths=3, g3=g[2][rows], h3=h[2])
    d = oracle.derive(w_np[rows], **kw)
    d.r = d.r2 = None
    return d


def sample_rows(out, n=384, seed=0):
    """Rows spread over the matrix plus the edges of 64-row groups and the last row."""
    rng = np.random.default_rng(seed)
    edge = [0, 1, 15, 16, 63, 64, 127, out // 2, out - 65, out - 64, out - 2, out - 1]
    rows = np.unique(np.concatenate([rng.choice(out, n, replace=False), [r for r in edge if 0 <= r < out]]))
    return rows


def gemm_bound(d, xm, k):
    """Elementwise bound of an fp32-accumulated product: every term
    g_p B_p h_p x is exact, at most k + 64 roundings of a partial sum
    (matrix-core chains, split-K partials, the scale in the epilogue) each
    within U32 of the running sum, which is at most Σ_p |g_p| Σ_j |h_p x_j|."""
    xa = np.abs(np.atleast_2d(xm))
    tot = 0.0
    for s, g, h in d.paths:
        tot = tot + np.abs(g.astype(np.float64))[None, :] * (xa @ np.abs(h.astype(np.float64)))[:, None]
    return (k + 64) * U32 * tot


# ---------------------------------------------------------------------------
# Llama-2-70B layer shapes
# ---------------------------------------------------------------------------
@pytest.mark.timeout(600)
@pytest.mark.parametrize("shape", [(28672, 8192), (8192, 28672)], ids=["gate_up", "down"])
def test_gemv_llama2_70b_shapes_b1_b32(gpu_lib, shape):
    out, inp = shape
    say("gemv 70B shape", shape, "batches 1 and 32, oracle on sampled rows")
    w = weight_f32(out, inp, seed_w(5, 0, "gate" if out > inp else "down"))
    g, h = given_scales(out, inp, 17)
    layer = pack_given(gpu_lib, w, g, h)
    rows = sample_rows(out)
    d = derive_rows(w.numpy(), rows, g, h)
    words = gpu_lib.unpack(layer).cpu().numpy().view(np.uint32)
    assert np.array_equal(words[0][rows], oracle.pack_words(d.s1)), "path-1 words differ"
    assert np.array_equal(words[1][rows], oracle.pack_words(d.s2)), "path-2 words differ"
    del words
    for batch in (1, 32):
        x = act_bf16(batch, inp, seed_x(5, batch))
        xv = bf16_values(x)
        y = gpu_lib.gemv(layer, x.cuda()).cpu().numpy().astype(np.float64)[:, rows]
        ref = oracle.gemv(d, xv)
        err = oracle.normwise_rel_err(y, ref)
        say("  batch", batch, "normwise err", err)
        assert err < TOL
        check_fx(y, ref, d, xv)


@pytest.mark.timeout(600)
def test_pack_meanabs_llama2_70b_gate_bit_exact(gpu_lib):
    # mean-|.| scales over a whole 28672 x 8192 matrix (the canonical float64
    # sums over 28672 rows and 8192 columns), bit for bit
    out, inp = 28672, 8192
    say("pack meanabs 70B gate", out, inp)
    w = weight_f32(out, inp, seed_w(5, 0, "gate"))
    layer = pack_gpu(gpu_lib, w)
    d = oracle.derive(w.numpy())
    d.r = None
    del w
    words = gpu_lib.unpack(layer).cpu().numpy().view(np.uint32)
    assert np.array_equal(words[0], oracle.pack_words(d.s1)), "path-1 words differ"
    assert np.array_equal(words[1], oracle.pack_words(d.s2)), "path-2 words differ"
    del words
    # device layout of a few row groups (the whole layout is checked at smaller shapes)
    raw = layer.planes.cpu().numpy().view(np.uint32)
    kg = (inp + 127) // 128
    for rg in (0, 217, out // 64 - 1):
        r0 = rg * 64
        sub = oracle.device_planes(oracle.pack_words(d.s1[r0:r0 + 64]), oracle.pack_words(d.s2[r0:r0 + 64]),
                                   64, inp)
        n = kg * 2 * 64 * 4
        assert np.array_equal(raw[rg * n:(rg + 1) * n], sub), rg
    gs = layer.g.cpu().numpy().view(np.float16)
    hs = layer.h.cpu().numpy().view(np.float16)
    for name, got, ref in (("g1", gs[0], d.g1), ("h1", hs[0], d.h1), ("g2", gs[1], d.g2), ("h2", hs[1], d.h2)):
        bad = np.flatnonzero(got.view(np.uint16) != ref.view(np.uint16))
        assert bad.size == 0, f"{name}: {bad.size} fp16 scales differ, first at {bad[:5]}"


def _decode_given(gpu_lib, cfg, batch_rows, seed, n_paths=2):
    """Pack every matrix of cfg.n_layers layers with given scales and run the
    oracle's decode chain over all batch rows at once (rows are independent)."""
    H, F = cfg.hidden, cfg.ffn
    kv = cfg.n_kv_heads * cfg.head_dim
    shapes = {"q": (H, H), "k": (kv, H), "v": (kv, H), "o": (H, H), "gate": (F, H), "up": (F, H), "down": (H, F)}
    layers, dmats = [], []
    for li in range(cfg.n_layers):
        ld, dd = {}, {}
        for k, (n, (o, i)) in enumerate(shapes.items()):
            w = weight_f32(o, i, seed + 10 * li + k)
            g, h = given_scales(o, i, seed + 100 * li + 10 * k, n_paths)
            ld[n] = pack_given(gpu_lib, w, g, h)
            dd[n] = derive_rows(w.numpy(), np.arange(o), g, h)
            del w
        layers.append(ld)
        dmats.append(dd)
    ocfg = {"n_heads": cfg.n_heads, "n_kv_heads": cfg.n_kv_heads, "head_dim": cfg.head_dim, "rms_eps": cfg.rms_eps}
    x = act_bf16(sum(batch_rows), H, seed + 99)
    ref = bf16_values(x)
    for dd in dmats:
        ref = oracle.decode_layer(ref, dd, ocfg)
    del dmats
    got = []
    r0 = 0
    for b in batch_rows:
        xb = x[r0:r0 + b].contiguous().cuda()
        got.append(gpu_lib.decode_step(cfg, layers, xb).cpu().to(torch.float32).numpy().astype(np.float64))
        r0 += b
    return np.concatenate(got), ref


@pytest.mark.timeout(900)
def test_decode_llama2_70b_two_layer_slice_b1_b32(gpu_lib):
    # two consecutive Llama-2-70B layers (hidden 8192, FFN 28672, 64 query and
    # 8 key/value heads of 128) at batch 1 and batch 32
    say("decode 70B two-layer slice, batches 1 and 32")
    cfg = gpu_lib.DecoderCfg(hidden=8192, ffn=28672, n_heads=64, n_kv_heads=8, head_dim=128, n_layers=2)
    y, ref = _decode_given(gpu_lib, cfg, (1, 32), 5000)
    for name, sl in (("batch 1", slice(0, 1)), ("batch 32", slice(1, 33))):
        ok, nbad = bf16_close(y[sl], ref[sl])
        say(" ", name, "normwise err", oracle.normwise_rel_err(y[sl], ref[sl]), "outside bound", nbad)
        assert ok, name


@pytest.mark.timeout(600)
def test_decode_llama3_8b_layer_b1_b16(gpu_lib):
    # one full Llama-3-8B decoder layer with mean-|.| scales at batch 1 and 16
    say("decode Llama-3-8B layer, batches 1 and 16")
    cfg = gpu_lib.DecoderCfg(hidden=4096, ffn=14336, n_heads=32, n_kv_heads=8, head_dim=128, n_layers=1)
    H, F, kv = 4096, 14336, 1024
    shapes = {"q": (H, H), "k": (kv, H), "v": (kv, H), "o": (H, H), "gate": (F, H), "up": (F, H), "down": (H, F)}
    ld, dd = {}, {}
    for n, (o, i) in shapes.items():
        w = weight_f32(o, i, seed_w(3, 0, n))
        ld[n] = pack_gpu(gpu_lib, w)
        dd[n] = oracle.derive(w.numpy())
        dd[n].r = None
    x = act_bf16(17, H, seed_x(3, 17))
    ocfg = {"n_heads": 32, "n_kv_heads": 8, "head_dim": 128, "rms_eps": cfg.rms_eps}
    ref = oracle.decode_layer(bf16_values(x), dd, ocfg)
    y1 = gpu_lib.decode_step(cfg, [ld], x[:1].contiguous().cuda()).cpu().to(torch.float32).numpy()
    y16 = gpu_lib.decode_step(cfg, [ld], x[1:].contiguous().cuda()).cpu().to(torch.float32).numpy()
    for name, y, r in (("batch 1", y1, ref[:1]), ("batch 16", y16, ref[1:])):
        ok, nbad = bf16_close(y.astype(np.float64), r)
        say(" ", name, "normwise err", oracle.normwise_rel_err(y, r), "outside bound", nbad)
        assert ok, name


# ---------------------------------------------------------------------------
# Llama-3-8B MLP prefill GEMM (14336 x 4096 and 4096 x 14336)
# ---------------------------------------------------------------------------
@pytest.mark.timeout(600)
@pytest.mark.parametrize("shape", [(14336, 4096), (4096, 14336)], ids=["gate_up", "down"])
def test_gemm_llama3_8b_mlp(gpu_lib, shape):
    N, K = shape
    say("gemm Llama-3-8B MLP", shape, "M = 512 whole, 2048 and 8192 on 256 token rows")
    w = weight_f32(N, K, seed_w(4, 0, "gate" if N > K else "down"))
    layer = pack_gpu(gpu_lib, w)
    d = oracle.derive(w.numpy())
    d.r = None
    del w
    words = gpu_lib.unpack(layer).cpu().numpy().view(np.uint32)
    assert np.array_equal(words[0], oracle.pack_words(d.s1)) and np.array_equal(words[1], oracle.pack_words(d.s2))
    del words
    we = oracle.weff(d)
    for M in (512, 2048, 8192):
        xm = act_bf16(M, K, seed_x(4, M))
        rows = np.arange(M) if M == 512 else np.unique(np.concatenate(
            [np.random.default_rng(M).choice(M, 250, replace=False), [0, 1, 127, 128, M - 2, M - 1]]))
        y = gpu_lib.gemm(layer, xm.cuda()).cpu().numpy().astype(np.float64)[rows]
        xs = bf16_values(xm)[rows]
        ref = xs @ we.T        # the oracle's W_eff of this layer, as oracle.gemm forms it
        assert np.array_equal(ref[:4], oracle.gemm(d, bf16_values(xm), rows=rows[:4]))
        err = oracle.normwise_rel_err(y, ref)
        bound = gemm_bound(d, xs, K) + U32 * np.abs(ref)
        nbad = int((np.abs(y - ref) > bound).sum())
        say("  M", M, "rows", len(rows), "normwise err", err, "outside elementwise bound", nbad)
        assert err < TOL and nbad == 0


# ---------------------------------------------------------------------------
# Llama-2-13B projections of the pages' kernel table (5120 x 5120, 13824 x 5120)
# ---------------------------------------------------------------------------
@pytest.mark.timeout(600)
@pytest.mark.parametrize("shape", [(5120, 5120), (13824, 5120)], ids=["q_proj", "gate_proj"])
def test_gemv_llama2_13b_table_shapes(gpu_lib, shape):
    out, inp = shape
    say("gemv 13B table shape", shape)
    w = weight_f32(out, inp, seed_w(6, 1, "q" if out == inp else "gate"))
    layer = pack_gpu(gpu_lib, w)
    d = oracle.derive(w.numpy())
    d.r = None
    words = gpu_lib.unpack(layer).cpu().numpy().view(np.uint32)
    assert np.array_equal(words[0], oracle.pack_words(d.s1)) and np.array_equal(words[1], oracle.pack_words(d.s2))
    for batch in (1, 4):
        x = act_bf16(batch, inp, seed_x(6, batch))
        xv = bf16_values(x)
        y = gpu_lib.gemv(layer, x.cuda()).cpu().numpy().astype(np.float64)
        ref = oracle.gemv(d, xv)
        err = oracle.normwise_rel_err(y, ref)
        say("  batch", batch, "normwise err", err)
        assert err < TOL
        check_fx(y, ref, d, xv)
