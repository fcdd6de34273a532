"""Boundary tests that need no GPU: the library loads, exports every symbol
include/rabit.h declares, sizes follow the documented closed forms, and every
argument error is returned before anything is enqueued (the pointers used
below are never dereferenced)."""
import ctypes
import os
import re

import pytest

from bit_residual_binarized_amd import rabit

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(rabit.LIB_PATH):
        from bit_residual_binarized_amd.build import build
        build()
    return rabit.load()


def header_symbols():
    text = open(os.path.join(ROOT, "include", "rabit.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(rabit_[a-z0-9_]+)\s*\(", text)))


def test_exports_every_header_symbol(lib):
    syms = header_symbols()
    assert len(syms) >= 12
    for s in syms:
        assert hasattr(lib, s), s
    assert sorted(rabit.EXPORTS) == syms


def test_sizes(lib):
    assert lib.rabit_planes_bytes(4096, 4096, 2) == 2 * 4096 * 4096 // 8
    assert lib.rabit_planes_bytes(11008, 4096, 2) == 2 * 11008 * 4096 // 8
    assert lib.rabit_planes_bytes(1, 1, 2) == 2048
    assert lib.rabit_planes_bytes(65, 129, 2) == 2 * 2 * 64 * 2 * 16
    assert lib.rabit_planes_bytes(0, 4, 2) == 0
    assert lib.rabit_planes_bytes(4, 4, 3) == 3 * 64 * 16          # the 3-bit variant
    assert lib.rabit_planes_bytes(65, 129, 3) == 3 * 2 * 64 * 2 * 16
    assert lib.rabit_planes_bytes(4, 4, 1) == 0
    assert lib.rabit_planes_bytes(4, 4, 4) == 0
    assert lib.rabit_planes_bytes(1 << 20, 4, 2) == 0
    assert lib.rabit_pack_workspace_bytes(4096, 4096) > 0
    assert lib.rabit_gemv_workspace_bytes(4096, 4096, 1) > 0
    assert lib.rabit_gemv_workspace_bytes(4096, 4096, 33) == 0
    assert lib.rabit_gemm_workspace_bytes(4096, 4096, 512) > 0
    assert lib.rabit_layout_version() == 1
    for code in range(-7, 1):
        assert rabit.status_string(code) != "unknown status"


FAKE = 1 << 40  # aligned, never dereferenced


def fake_layer(out=256, inp=512, version=1, paths=2, planes=FAKE, g=FAKE + (1 << 30), h=FAKE + (2 << 30)):
    return rabit.RabitLayerC(version, out, inp, paths, planes, g, h)


def gemv(lib, layer, x=FAKE + (3 << 30), batch=1, y=FAKE + (4 << 30), dtype=0, ws=FAKE + (5 << 30),
         wsb=1 << 30):
    return lib.rabit_gemv(ctypes.byref(layer) if layer is not None else None, x, batch, y, dtype, ws,
                          wsb, None)


def test_gemv_argument_errors(lib):
    L = fake_layer()
    assert gemv(lib, None) == rabit.RABIT_EINVAL
    assert gemv(lib, fake_layer(version=2)) == rabit.RABIT_EINVAL
    assert gemv(lib, fake_layer(paths=4)) == rabit.RABIT_EUNSUPPORTED
    assert gemv(lib, fake_layer(paths=1)) == rabit.RABIT_EUNSUPPORTED
    # a 3-path layer passes the path check and fails later on its workspace
    assert gemv(lib, fake_layer(paths=3), wsb=0) == rabit.RABIT_EWORKSPACE
    assert gemv(lib, fake_layer(out=0)) == rabit.RABIT_ESHAPE
    assert gemv(lib, fake_layer(inp=1 << 20)) == rabit.RABIT_ESHAPE
    assert gemv(lib, fake_layer(planes=0)) == rabit.RABIT_EINVAL
    assert gemv(lib, fake_layer(g=FAKE + 8 + (1 << 30))) == rabit.RABIT_EALIGN
    assert gemv(lib, fake_layer(h=FAKE)) == rabit.RABIT_EINVAL        # h aliases planes
    assert gemv(lib, L, x=0) == rabit.RABIT_EINVAL
    assert gemv(lib, L, x=FAKE + 2 + (3 << 30)) == rabit.RABIT_EALIGN
    assert gemv(lib, L, batch=0) == rabit.RABIT_ESHAPE
    assert gemv(lib, L, batch=33) == rabit.RABIT_ESHAPE
    assert gemv(lib, L, dtype=7) == rabit.RABIT_EINVAL
    assert gemv(lib, L, y=FAKE + (3 << 30)) == rabit.RABIT_EINVAL     # y aliases x
    assert gemv(lib, L, ws=0) == rabit.RABIT_EWORKSPACE
    assert gemv(lib, L, wsb=16) == rabit.RABIT_EWORKSPACE
    assert gemv(lib, L, ws=FAKE + 4 + (5 << 30)) == rabit.RABIT_EALIGN


def test_gemv_partial_multi_errors(lib):
    def multi(layers, n=None, x=FAKE + (3 << 30), batch=1, ws=FAKE + (5 << 30), wsb=1 << 30):
        arr = (rabit.RabitLayerC * max(1, len(layers)))(*layers)
        return lib.rabit_gemv_partial_multi(arr if layers else None, len(layers) if n is None else n,
                                            x, batch, ws, wsb, None)
    a = fake_layer()
    b = fake_layer(out=128, planes=FAKE + (6 << 30), g=FAKE + (7 << 30), h=FAKE + (8 << 30))
    assert multi([]) == rabit.RABIT_EINVAL
    assert multi([a, b], n=0) == rabit.RABIT_ESHAPE
    assert multi([a, b], n=4) == rabit.RABIT_ESHAPE
    assert multi([a, fake_layer(inp=256, planes=FAKE + (6 << 30), g=FAKE + (7 << 30), h=FAKE + (8 << 30))]) \
        == rabit.RABIT_ESHAPE                                             # in_features differ
    assert multi([a, b], batch=33) == rabit.RABIT_ESHAPE
    assert multi([a, b], x=0) == rabit.RABIT_EINVAL
    assert multi([a, fake_layer(version=3)]) == rabit.RABIT_EINVAL
    need = (lib.rabit_gemv_workspace_bytes(256, 512, 1) + lib.rabit_gemv_workspace_bytes(128, 512, 1))
    assert multi([a, b], wsb=need - 1) == rabit.RABIT_EWORKSPACE
    assert multi([a, b], ws=FAKE + 8 + (5 << 30)) == rabit.RABIT_EALIGN
    assert multi([a, b], ws=FAKE + (3 << 30)) == rabit.RABIT_EINVAL     # workspace aliases x
    assert multi([a, b], ws=FAKE + (6 << 30)) == rabit.RABIT_EINVAL     # workspace aliases planes


def test_pack_argument_errors(lib):
    L = fake_layer()
    w = FAKE + (6 << 30)
    pk = lambda w=w, mode=1, layer=L, ws=FAKE + (5 << 30), wsb=1 << 30: lib.rabit_pack(
        w, mode, ctypes.byref(layer), ws, wsb, None)
    assert pk(w=0) == rabit.RABIT_EINVAL
    assert pk(mode=5) == rabit.RABIT_EINVAL
    assert pk(mode=3) == rabit.RABIT_EINVAL
    # the normalized mean-|.| mode is accepted and needs the workspace
    assert pk(mode=rabit.RABIT_SCALES_MEANABS_NORMALIZED, wsb=8) == rabit.RABIT_EWORKSPACE
    assert pk(w=w + 4) == rabit.RABIT_EALIGN
    assert pk(w=FAKE) == rabit.RABIT_EINVAL          # W aliases the planes it would write
    assert pk(ws=0) == rabit.RABIT_EWORKSPACE
    assert pk(wsb=8) == rabit.RABIT_EWORKSPACE
    assert pk(layer=fake_layer(paths=1)) == rabit.RABIT_EUNSUPPORTED


def test_gemm_and_unpack_errors(lib):
    L = fake_layer()
    X, Y, ws = FAKE + (3 << 30), FAKE + (4 << 30), FAKE + (5 << 30)
    assert lib.rabit_gemm(ctypes.byref(L), X, 0, Y, 0, ws, 1 << 30, None) == rabit.RABIT_ESHAPE
    assert lib.rabit_gemm(ctypes.byref(L), X, 8, X, 0, ws, 1 << 30, None) == rabit.RABIT_EINVAL
    assert lib.rabit_gemm(ctypes.byref(L), X, 8, Y, 0, ws, 16, None) == rabit.RABIT_EWORKSPACE
    # a 3-path layer passes the path check and fails later on its workspace
    L3 = fake_layer(paths=3)
    assert lib.rabit_gemm(ctypes.byref(L3), X, 8, Y, 0, ws, 16, None) == rabit.RABIT_EWORKSPACE
    assert lib.rabit_gemm(ctypes.byref(fake_layer(paths=4)), X, 8, Y, 0, ws, 1 << 30, None) == \
        rabit.RABIT_EUNSUPPORTED
    assert lib.rabit_unpack(ctypes.byref(L), 0, None) == rabit.RABIT_EINVAL
    assert lib.rabit_unpack(ctypes.byref(fake_layer(version=0)), Y, None) == rabit.RABIT_EINVAL


def test_decode_cfg_errors(lib):
    cfg = rabit.DecoderCfg(hidden=64, ffn=96, n_heads=4, n_kv_heads=3, head_dim=16)
    cc = cfg.c()
    assert lib.rabit_decode_workspace_bytes(ctypes.byref(cc), 1) == 0   # 4 % 3 != 0
    cfg = rabit.DecoderCfg(hidden=64, ffn=96, n_heads=4, n_kv_heads=2, head_dim=16)
    cc = cfg.c()
    assert lib.rabit_decode_workspace_bytes(ctypes.byref(cc), 1) > 0
    arr = (rabit.RabitLayerC * 7)()
    for i in range(7):
        arr[i] = fake_layer(out=64, inp=64, planes=FAKE + i * (1 << 32), g=FAKE + i * (1 << 32) + (1 << 30),
                            h=FAKE + i * (1 << 32) + (2 << 30))
    x, out, ws = FAKE + (100 << 32), FAKE + (101 << 32), FAKE + (102 << 32)
    # k has 64 rows but n_kv_heads * head_dim = 32 -> shape error before any launch
    assert lib.rabit_decode_step(ctypes.byref(cc), arr, x, 1, out, ws, 1 << 40, None) == rabit.RABIT_ESHAPE
    mlp = rabit.DecoderCfg(hidden=64, ffn=96, mlp_only=True).c()
    assert lib.rabit_decode_step(ctypes.byref(mlp), arr, x, 1, out, ws, 1 << 40, None) == rabit.RABIT_ESHAPE


def test_stream_read_errors(lib):
    P, Q = ctypes.c_void_p(1 << 20), ctypes.c_void_p(2 << 20)
    assert lib.rabit_stream_read(None, 64, Q, None) == rabit.RABIT_EINVAL
    assert lib.rabit_stream_read(P, 64, None, None) == rabit.RABIT_EINVAL
    assert lib.rabit_stream_read(ctypes.c_void_p((1 << 20) + 8), 64, Q, None) == rabit.RABIT_EALIGN
    assert lib.rabit_stream_read(P, 64, ctypes.c_void_p((2 << 20) + 4), None) == rabit.RABIT_EALIGN
    assert lib.rabit_stream_read(P, 72, Q, None) == rabit.RABIT_EALIGN
    assert lib.rabit_stream_read(P, 0, Q, None) == rabit.RABIT_OK  # nothing runs


def test_training_sizes_and_errors(lib):
    assert lib.rabit_grad_weight_workspace_bytes(4096, 11008) > 0
    assert lib.rabit_grad_weight_workspace_bytes(0, 16) == 0
    assert lib.rabit_grad_input_workspace_bytes(4096, 11008, 2048) > \
        lib.rabit_gemm_workspace_bytes(11008, 4096, 2048)
    assert lib.rabit_grad_input_workspace_bytes(4096, 4096, 0) == 0
    L = fake_layer()
    X, dY, dW, dg, dh, ws = (FAKE + (k << 32) for k in range(3, 9))
    big = 1 << 40

    def gw(layer=L, x=X, dy=dY, m=64, dw=dW, g=dg, h=dh, flags=0, w=ws, wsb=big):
        return lib.rabit_grad_weight(ctypes.byref(layer), x, dy, m, dw, g, h, flags, w, wsb, None)
    assert gw(x=0) == rabit.RABIT_EINVAL
    assert gw(h=0) == rabit.RABIT_EINVAL
    assert gw(flags=2) == rabit.RABIT_EINVAL
    assert gw(m=0) == rabit.RABIT_ESHAPE
    assert gw(m=(1 << 20) + 1) == rabit.RABIT_ESHAPE
    assert gw(dw=dW + 4) == rabit.RABIT_EALIGN
    assert gw(dw=X) == rabit.RABIT_EINVAL                 # dW aliases X
    assert gw(g=dW + 256) == rabit.RABIT_EINVAL           # dg inside dW
    assert gw(g=FAKE + (1 << 30)) == rabit.RABIT_EINVAL   # dg aliases the layer's g
    assert gw(wsb=16) == rabit.RABIT_EWORKSPACE
    assert gw(w=0) == rabit.RABIT_EWORKSPACE
    assert gw(layer=fake_layer(paths=4)) == rabit.RABIT_EUNSUPPORTED
    assert gw(layer=fake_layer(paths=3), wsb=16) == rabit.RABIT_EWORKSPACE

    def gi(layer=L, dy=dY, m=64, dx=dW, dt=0, w=ws, wsb=big):
        return lib.rabit_grad_input(ctypes.byref(layer), dy, m, dx, dt, w, wsb, None)
    assert gi(dy=0) == rabit.RABIT_EINVAL
    assert gi(dt=3) == rabit.RABIT_EINVAL
    assert gi(m=0) == rabit.RABIT_ESHAPE
    assert gi(dx=dY) == rabit.RABIT_EINVAL                # dX aliases dY
    assert gi(dx=FAKE) == rabit.RABIT_EINVAL              # dX aliases the planes
    assert gi(wsb=16) == rabit.RABIT_EWORKSPACE
    assert gi(w=ws + 8) == rabit.RABIT_EALIGN

    assert lib.rabit_transpose_planes(ctypes.byref(L), 0, None) == rabit.RABIT_EINVAL
    assert lib.rabit_transpose_planes(ctypes.byref(L), FAKE + 16, None) == rabit.RABIT_EINVAL
    assert lib.rabit_transpose_planes(ctypes.byref(L), dW + 8, None) == rabit.RABIT_EALIGN
    assert lib.rabit_transpose_planes(ctypes.byref(fake_layer(version=0)), dW, None) == \
        rabit.RABIT_EINVAL


def test_svid_errors(lib):
    assert lib.rabit_svid_workspace_bytes(4096, 11008) > 0
    assert lib.rabit_svid_workspace_bytes(0, 8) == 0
    W, g, h, pl, ws = (FAKE + (k << 32) for k in range(10, 15))
    big = 1 << 40

    def sv(w=W, out=256, inp=512, P=2, sweeps=20, passes=3, fo=None, fi=None, flags=0, G=g, H=h,
           planes=pl, wsp=ws, wsb=big):
        return lib.rabit_svid_init(w, out, inp, P, sweeps, passes, fo, fi, flags, G, H, planes, wsp,
                                   wsb, None)
    assert sv(P=4) == rabit.RABIT_EUNSUPPORTED
    assert sv(P=1) == rabit.RABIT_EUNSUPPORTED
    assert sv(out=0) == rabit.RABIT_ESHAPE
    assert sv(sweeps=0) == rabit.RABIT_ESHAPE
    assert sv(passes=2) == rabit.RABIT_ESHAPE
    assert sv(passes=65) == rabit.RABIT_ESHAPE
    assert sv(w=0) == rabit.RABIT_EINVAL
    assert sv(planes=0) == rabit.RABIT_EINVAL
    assert sv(flags=2) == rabit.RABIT_EINVAL
    assert sv(G=W) == rabit.RABIT_EINVAL                 # g aliases W
    assert sv(H=g + 512) == rabit.RABIT_EINVAL           # h inside g
    assert sv(fo=g) == rabit.RABIT_EINVAL                # f_out aliases g
    assert sv(fi=FAKE + (20 << 32) + 4) == rabit.RABIT_EALIGN
    assert sv(wsb=16) == rabit.RABIT_EWORKSPACE
    assert sv(P=3, wsb=16) == rabit.RABIT_EWORKSPACE


def test_gemm_plane_size_limit(lib):
    # 2^17 x 2^17 with two paths: 4 GiB of planes, beyond the GEMM's 32-bit
    # offsets (the layer's buffers are placed apart so that only the size fails)
    big = 1 << 17
    L = fake_layer(out=big, inp=big, planes=FAKE, g=FAKE + (8 << 30), h=FAKE + (9 << 30))
    X, Y, ws = FAKE + (10 << 30), FAKE + (11 << 30), FAKE + (12 << 30)
    assert lib.rabit_planes_bytes(big, big, 2) == 1 << 32
    assert lib.rabit_gemm(ctypes.byref(L), X, 8, Y, 0, ws, 1 << 40, None) == rabit.RABIT_ESHAPE
    assert lib.rabit_gemm_ex(ctypes.byref(L), X, 8, Y, 0, 1, ws, 1 << 40, None) == rabit.RABIT_ESHAPE
    assert lib.rabit_grad_input(ctypes.byref(L), X, 8, Y, 0, ws, 1 << 40, None) == rabit.RABIT_ESHAPE
    # just below the limit the size check passes (the workspace check fails next)
    L2 = fake_layer(out=big - 64, inp=big, planes=FAKE, g=FAKE + (8 << 30), h=FAKE + (9 << 30))
    assert lib.rabit_gemm(ctypes.byref(L2), X, 8, Y, 0, ws, 16, None) == rabit.RABIT_EWORKSPACE


def test_gemm_ex_flags(lib):
    L = fake_layer()
    X, Y, ws = FAKE + (3 << 30), FAKE + (4 << 30), FAKE + (5 << 30)
    assert lib.rabit_gemm_ex(ctypes.byref(L), X, 8, Y, 0, 2, ws, 1 << 30, None) == rabit.RABIT_EINVAL
    assert lib.rabit_gemm_ex(ctypes.byref(L), X, 0, Y, 0, 1, ws, 1 << 30, None) == rabit.RABIT_ESHAPE
    assert lib.rabit_grad_input_ex(ctypes.byref(L), X, 8, Y, 0, 4, ws, 1 << 30, None) == rabit.RABIT_EINVAL
    assert lib.rabit_grad_input_ex(ctypes.byref(L), X, 8, Y, 0, 1, ws, 16, None) == rabit.RABIT_EWORKSPACE


def test_three_path_layer_aliasing(lib):
    # A 3-path layer's third plane, g_3 and h_3 lie beyond what a 2-path layer
    # of the same shape occupies; outputs and workspaces that overlap only
    # them must still be rejected.
    out, inp = 256, 512
    pb2, pb3 = lib.rabit_planes_bytes(out, inp, 2), lib.rabit_planes_bytes(out, inp, 3)
    assert pb3 > pb2
    G, H = FAKE + (1 << 30), FAKE + (2 << 30)
    L3 = fake_layer(out, inp, paths=3, planes=FAKE, g=G, h=H)
    third_plane = FAKE + (pb2 + pb3) // 2 // 16 * 16
    g3 = G + 2 * 2 * out          # g of path 3
    h3 = H + 2 * 2 * inp          # h of path 3
    x, ws = FAKE + (3 << 30), FAKE + (5 << 30)
    big = 1 << 30
    # rabit_gemv: y or the workspace on the third plane, g_3 or h_3
    for y in (third_plane, g3, h3):
        assert gemv(lib, L3, y=y) == rabit.RABIT_EINVAL, hex(y)
        assert gemv(lib, L3, ws=y) == rabit.RABIT_EINVAL, hex(y)
    # rabit_gemv_partial: the workspace on any of them
    for w in (third_plane, g3, h3):
        assert lib.rabit_gemv_partial(ctypes.byref(L3), x, 1, w, big, None) == rabit.RABIT_EINVAL
    # rabit_gemv_reduce: y or the workspace on any of them
    for p in (third_plane, g3, h3):
        assert lib.rabit_gemv_reduce(ctypes.byref(L3), 1, p, 0, ws, big, None) == rabit.RABIT_EINVAL
        assert lib.rabit_gemv_reduce(ctypes.byref(L3), 1, FAKE + (4 << 30), 0, p, big, None) == \
            rabit.RABIT_EINVAL
    # rabit_gemv_partial_multi: the workspace on the second layer's third plane or scales
    a = fake_layer(out, inp, paths=3, planes=FAKE + (6 << 30), g=FAKE + (7 << 30), h=FAKE + (8 << 30))
    for w in (third_plane, g3, h3):
        arr = (rabit.RabitLayerC * 2)(a, L3)
        assert lib.rabit_gemv_partial_multi(arr, 2, x, 1, w, big, None) == rabit.RABIT_EINVAL


def test_gemv_noalloc_argument_errors(lib):
    # every error is returned before the scratch address is looked up or
    # anything is enqueued
    def na(layer, x=FAKE + (3 << 30), batch=1, y=FAKE + (4 << 30), dtype=0):
        return lib.rabit_gemv_noalloc(ctypes.byref(layer) if layer is not None else None, x, batch, y,
                                      dtype, None)
    L = fake_layer()
    assert na(None) == rabit.RABIT_EINVAL
    assert na(fake_layer(paths=4)) == rabit.RABIT_EUNSUPPORTED
    assert na(L, x=0) == rabit.RABIT_EINVAL
    assert na(L, dtype=5) == rabit.RABIT_EINVAL
    assert na(L, batch=0) == rabit.RABIT_ESHAPE
    assert na(L, batch=33) == rabit.RABIT_ESHAPE
    assert na(L, y=FAKE + (3 << 30)) == rabit.RABIT_EINVAL            # y aliases x
    assert na(L, y=FAKE + 8 + (4 << 30)) == rabit.RABIT_EALIGN
    L3 = fake_layer(paths=3)
    assert na(L3, y=FAKE + 32768) == rabit.RABIT_EINVAL               # y on the third plane
    # partials beyond the fixed scratch buffer
    big = fake_layer(28672, 8192, planes=FAKE, g=FAKE + (1 << 30), h=FAKE + (2 << 30))
    need = lib.rabit_gemv_workspace_bytes(28672, 8192, 9)
    assert need > rabit.NOALLOC_SCRATCH_BYTES
    assert na(big, batch=9, x=FAKE + (3 << 32), y=FAKE + (4 << 32)) == rabit.RABIT_ESCRATCH
    assert lib.rabit_gemv_workspace_bytes(28672, 8192, 8) <= rabit.NOALLOC_SCRATCH_BYTES
