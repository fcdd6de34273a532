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
