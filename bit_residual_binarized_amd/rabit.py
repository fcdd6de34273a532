"""Thin ctypes binding of librabit (include/rabit.h).

Argument marshalling only: every step of the hot path runs in the HIP
kernels of librabit.so. torch supplies device memory and the current stream.
There is no fallback: if the library is missing, load() raises.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "librabit.so")

RABIT_OK = 0
RABIT_EINVAL = -1
RABIT_ESHAPE = -2
RABIT_EALIGN = -3
RABIT_EUNSUPPORTED = -4
RABIT_EDEVICE = -5
RABIT_EWORKSPACE = -6
RABIT_ESCRATCH = -7
NOALLOC_SCRATCH_BYTES = 16 << 20
RABIT_SCALES_GIVEN = 0
RABIT_SCALES_MEANABS = 1
RABIT_SCALES_MEANABS_NORMALIZED = 2
RABIT_OUT_F32 = 0
RABIT_OUT_BF16 = 1
RABIT_LAYOUT_V1 = 1
MAX_GEMV_BATCH = 32
GEMV_FP16_MIN_BATCH = 8   # RABIT_GEMV_FP16_MIN_BATCH: batches from here on use the fp16 matrix-core path

# every symbol include/rabit.h declares
EXPORTS = [
    "rabit_planes_bytes", "rabit_pack_workspace_bytes", "rabit_gemv_workspace_bytes",
    "rabit_gemm_workspace_bytes", "rabit_pack", "rabit_unpack", "rabit_gemv", "rabit_gemm",
    "rabit_decode_workspace_bytes", "rabit_decode_step", "rabit_status_string",
    "rabit_layout_version", "rabit_test_f64_to_16", "rabit_gemv_partial", "rabit_gemv_reduce",
    "rabit_gemv_partial_multi", "rabit_stream_read", "rabit_grad_input_workspace_bytes",
    "rabit_grad_weight_workspace_bytes", "rabit_transpose_planes", "rabit_grad_input",
    "rabit_grad_weight", "rabit_svid_workspace_bytes", "rabit_svid_init", "rabit_gemm_ex",
    "rabit_grad_input_ex", "rabit_gemv_noalloc",
]


class RabitLayerC(ctypes.Structure):
    _fields_ = [
        ("layout_version", ctypes.c_int32),
        ("out_features", ctypes.c_int32),
        ("in_features", ctypes.c_int32),
        ("n_paths", ctypes.c_int32),
        ("planes", ctypes.c_void_p),
        ("g", ctypes.c_void_p),
        ("h", ctypes.c_void_p),
    ]


class DecoderCfgC(ctypes.Structure):
    _fields_ = [
        ("hidden", ctypes.c_int32),
        ("ffn", ctypes.c_int32),
        ("n_heads", ctypes.c_int32),
        ("n_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("n_layers", ctypes.c_int32),
        ("rms_eps", ctypes.c_float),
        ("mlp_only", ctypes.c_int32),
    ]


class RabitError(RuntimeError):
    def __init__(self, code: int, what: str):
        self.code = code
        super().__init__(f"{what}: {status_string(code)} ({code})")


_lib = None


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load librabit.so (built by bit_residual_binarized_amd.build); raise if absent."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"librabit.so not found at {path}; run "
                           "`python -m bit_residual_binarized_amd.build` first")
    lib = ctypes.CDLL(path)
    vp, sz, i32, u32 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int32, ctypes.c_uint32
    lp = ctypes.POINTER(RabitLayerC)
    sig = {
        "rabit_planes_bytes": (sz, [i32, i32, i32]),
        "rabit_pack_workspace_bytes": (sz, [i32, i32]),
        "rabit_gemv_workspace_bytes": (sz, [i32, i32, i32]),
        "rabit_gemm_workspace_bytes": (sz, [i32, i32, i32]),
        "rabit_pack": (ctypes.c_int, [vp, u32, lp, vp, sz, vp]),
        "rabit_unpack": (ctypes.c_int, [lp, vp, vp]),
        "rabit_gemv": (ctypes.c_int, [lp, vp, i32, vp, i32, vp, sz, vp]),
        "rabit_gemv_noalloc": (ctypes.c_int, [lp, vp, i32, vp, i32, vp]),
        "rabit_gemm": (ctypes.c_int, [lp, vp, i32, vp, i32, vp, sz, vp]),
        "rabit_gemv_partial": (ctypes.c_int, [lp, vp, i32, vp, sz, vp]),
        "rabit_gemv_reduce": (ctypes.c_int, [lp, i32, vp, i32, vp, sz, vp]),
        "rabit_gemv_partial_multi": (ctypes.c_int, [lp, i32, vp, i32, vp, sz, vp]),
        "rabit_decode_workspace_bytes": (sz, [ctypes.POINTER(DecoderCfgC), i32]),
        "rabit_decode_step": (ctypes.c_int, [ctypes.POINTER(DecoderCfgC), lp, vp, i32, vp, vp, sz, vp]),
        "rabit_status_string": (ctypes.c_char_p, [ctypes.c_int]),
        "rabit_layout_version": (i32, []),
        "rabit_test_f64_to_16": (ctypes.c_int, [vp, vp, i32, i32, vp]),
        "rabit_stream_read": (ctypes.c_int, [vp, sz, vp, vp]),
        "rabit_grad_input_workspace_bytes": (sz, [i32, i32, i32]),
        "rabit_grad_weight_workspace_bytes": (sz, [i32, i32]),
        "rabit_transpose_planes": (ctypes.c_int, [lp, vp, vp]),
        "rabit_grad_input": (ctypes.c_int, [lp, vp, i32, vp, i32, vp, sz, vp]),
        "rabit_grad_weight": (ctypes.c_int, [lp, vp, vp, i32, vp, vp, vp, u32, vp, sz, vp]),
        "rabit_svid_workspace_bytes": (sz, [i32, i32]),
        "rabit_gemm_ex": (ctypes.c_int, [lp, vp, i32, vp, i32, u32, vp, sz, vp]),
        "rabit_grad_input_ex": (ctypes.c_int, [lp, vp, i32, vp, i32, u32, vp, sz, vp]),
        "rabit_svid_init": (ctypes.c_int, [vp, i32, i32, i32, i32, i32, vp, vp, u32, vp, vp, vp, vp,
                                           sz, vp]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def status_string(code: int) -> str:
    return load().rabit_status_string(code).decode()


def _check(code: int, what: str) -> None:
    if code != RABIT_OK:
        raise RabitError(code, what)


def _stream(stream=None):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _ptr(t: torch.Tensor | None):
    return ctypes.c_void_p(0 if t is None else t.data_ptr())


def planes_bytes(out: int, inp: int, n_paths: int = 2) -> int:
    return int(load().rabit_planes_bytes(out, inp, n_paths))


@dataclass
class PackedLayer:
    """Device buffers of one frozen layer of n_paths (2 or 3) binary paths
    (see rabit_layer in rabit.h)."""
    out_features: int
    in_features: int
    planes: torch.Tensor  # uint8 [planes_bytes]
    g: torch.Tensor       # int16 fp16 bits [n_paths, out]
    h: torch.Tensor       # int16 fp16 bits [n_paths, in]
    n_paths: int = 2

    @staticmethod
    def empty(out: int, inp: int, device="cuda", n_paths: int = 2) -> "PackedLayer":
        pb = planes_bytes(out, inp, n_paths)
        if pb == 0:
            raise RabitError(RABIT_ESHAPE, "planes_bytes")
        return PackedLayer(out, inp,
                           torch.empty(pb, dtype=torch.uint8, device=device),
                           torch.empty(n_paths, out, dtype=torch.int16, device=device),
                           torch.empty(n_paths, inp, dtype=torch.int16, device=device),
                           n_paths)

    def c(self) -> RabitLayerC:
        return RabitLayerC(RABIT_LAYOUT_V1, self.out_features, self.in_features, self.n_paths,
                           self.planes.data_ptr(), self.g.data_ptr(), self.h.data_ptr())

    def scales_f16(self):
        return self.g.view(torch.float16), self.h.view(torch.float16)


def _ws(nbytes: int, device) -> torch.Tensor:
    return torch.empty(max(int(nbytes), 16), dtype=torch.uint8, device=device)


def pack(w: torch.Tensor, layer: PackedLayer, mode: int = RABIT_SCALES_MEANABS,
         workspace: torch.Tensor | None = None, stream=None) -> PackedLayer:
    """Derive and pack every path of `w` (float32 [out, in], cuda) into `layer`."""
    lib = load()
    assert w.dtype == torch.float32 and w.is_contiguous()
    nb = lib.rabit_pack_workspace_bytes(layer.out_features, layer.in_features)
    if workspace is None and mode != RABIT_SCALES_GIVEN:
        workspace = _ws(nb, w.device)
    lc = layer.c()
    _check(lib.rabit_pack(_ptr(w), mode, ctypes.byref(lc), _ptr(workspace),
                          0 if workspace is None else workspace.numel(), _stream(stream)),
           "rabit_pack")
    return layer


def unpack(layer: PackedLayer, stream=None) -> torch.Tensor:
    lib = load()
    nw = (layer.in_features + 31) // 32
    words = torch.empty(layer.n_paths, layer.out_features, nw, dtype=torch.int32, device=layer.planes.device)
    lc = layer.c()
    _check(lib.rabit_unpack(ctypes.byref(lc), _ptr(words), _stream(stream)), "rabit_unpack")
    return words


def gemv_workspace(layer: PackedLayer, batch: int) -> torch.Tensor:
    nb = load().rabit_gemv_workspace_bytes(layer.out_features, layer.in_features, batch)
    return _ws(nb, layer.planes.device)


def gemv(layer: PackedLayer, x: torch.Tensor, y_dtype: int = RABIT_OUT_F32,
         y: torch.Tensor | None = None, workspace: torch.Tensor | None = None,
         stream=None) -> torch.Tensor:
    """y[b] = Σ_p g_p ⊙ (B_p (h_p ⊙ x[b])); x bfloat16 [batch, in] on cuda."""
    lib = load()
    assert x.dtype == torch.bfloat16 and x.is_contiguous()
    batch = x.shape[0]
    if y is None:
        dt = torch.float32 if y_dtype == RABIT_OUT_F32 else torch.bfloat16
        y = torch.empty(batch, layer.out_features, dtype=dt, device=x.device)
    if workspace is None:
        workspace = gemv_workspace(layer, batch)
    lc = layer.c()
    _check(lib.rabit_gemv(ctypes.byref(lc), _ptr(x), batch, _ptr(y), y_dtype, _ptr(workspace),
                          workspace.numel(), _stream(stream)), "rabit_gemv")
    return y


def gemv_noalloc(layer: PackedLayer, x: torch.Tensor, y: torch.Tensor, y_dtype: int = RABIT_OUT_F32,
                 stream=None) -> torch.Tensor:
    """rabit_gemv_noalloc: the GEMV with the library's fixed scratch buffer
    (no workspace); y must be preallocated [batch, out]."""
    assert x.dtype == torch.bfloat16 and x.is_contiguous() and y.is_contiguous()
    lc = layer.c()
    _check(load().rabit_gemv_noalloc(ctypes.byref(lc), _ptr(x), x.shape[0], _ptr(y), y_dtype,
                                     _stream(stream)), "rabit_gemv_noalloc")
    return y


def gemv_partial(layer: PackedLayer, x: torch.Tensor, workspace: torch.Tensor, stream=None) -> None:
    """rabit_gemv_partial: one launch over every plane byte; partials stay in workspace."""
    assert x.dtype == torch.bfloat16 and x.is_contiguous()
    lc = layer.c()
    _check(load().rabit_gemv_partial(ctypes.byref(lc), _ptr(x), x.shape[0], _ptr(workspace),
                                     workspace.numel(), _stream(stream)), "rabit_gemv_partial")


def gemv_partial_multi(layers: list, x: torch.Tensor, workspace: torch.Tensor, stream=None) -> list:
    """rabit_gemv_partial_multi: partials of 1..3 layers sharing x in one launch.
    Returns each layer's view of the workspace (pass it to gemv_reduce)."""
    assert x.dtype == torch.bfloat16 and x.is_contiguous()
    lib = load()
    arr = (RabitLayerC * len(layers))(*[L.c() for L in layers])
    _check(lib.rabit_gemv_partial_multi(arr, len(layers), _ptr(x), x.shape[0], _ptr(workspace),
                                        workspace.numel(), _stream(stream)), "rabit_gemv_partial_multi")
    views, off = [], 0
    for L in layers:
        nb = lib.rabit_gemv_workspace_bytes(L.out_features, L.in_features, x.shape[0])
        views.append(workspace[off:off + nb])
        off += nb
    return views


def gemv_multi_workspace(layers: list, batch: int) -> torch.Tensor:
    lib = load()
    nb = sum(lib.rabit_gemv_workspace_bytes(L.out_features, L.in_features, batch) for L in layers)
    return _ws(nb, layers[0].planes.device)


def gemv_reduce(layer: PackedLayer, batch: int, y: torch.Tensor, workspace: torch.Tensor,
                y_dtype: int = RABIT_OUT_F32, stream=None) -> torch.Tensor:
    """rabit_gemv_reduce: sums the partials of the last gemv_partial into y."""
    lc = layer.c()
    _check(load().rabit_gemv_reduce(ctypes.byref(lc), batch, _ptr(y), y_dtype, _ptr(workspace),
                                    workspace.numel(), _stream(stream)), "rabit_gemv_reduce")
    return y


def gemm_workspace(layer: PackedLayer, m: int) -> torch.Tensor:
    nb = load().rabit_gemm_workspace_bytes(layer.out_features, layer.in_features, m)
    return _ws(nb, layer.planes.device)


RABIT_GEMM_WEFF = 1


def gemm(layer: PackedLayer, xm: torch.Tensor, y_dtype: int = RABIT_OUT_F32,
         y: torch.Tensor | None = None, workspace: torch.Tensor | None = None,
         stream=None, weff: bool = False) -> torch.Tensor:
    """Y = X W_hatᵀ; weff=True forms the effective weight per tile in fp16
    (rabit_gemm_ex with RABIT_GEMM_WEFF)."""
    lib = load()
    assert xm.dtype == torch.bfloat16 and xm.is_contiguous()
    m = xm.shape[0]
    if y is None:
        dt = torch.float32 if y_dtype == RABIT_OUT_F32 else torch.bfloat16
        y = torch.empty(m, layer.out_features, dtype=dt, device=xm.device)
    if workspace is None:
        workspace = gemm_workspace(layer, m)
    lc = layer.c()
    if weff:
        _check(lib.rabit_gemm_ex(ctypes.byref(lc), _ptr(xm), m, _ptr(y), y_dtype, RABIT_GEMM_WEFF,
                                 _ptr(workspace), workspace.numel(), _stream(stream)), "rabit_gemm_ex")
    else:
        _check(lib.rabit_gemm(ctypes.byref(lc), _ptr(xm), m, _ptr(y), y_dtype, _ptr(workspace),
                              workspace.numel(), _stream(stream)), "rabit_gemm")
    return y


# --- training side (rabit_grad_* in rabit.h) ---
RABIT_GRAD_ACCUMULATE = 1


def transpose_planes(layer: PackedLayer, out: torch.Tensor | None = None,
                     stream=None) -> torch.Tensor:
    """Planes of the layer W_hatᵀ (uint8 buffer in layout V1)."""
    nb = planes_bytes(layer.in_features, layer.out_features, layer.n_paths)
    if out is None:
        out = torch.empty(nb, dtype=torch.uint8, device=layer.planes.device)
    lc = layer.c()
    _check(load().rabit_transpose_planes(ctypes.byref(lc), _ptr(out), _stream(stream)),
           "rabit_transpose_planes")
    return out


def grad_input_workspace(layer: PackedLayer, m: int) -> torch.Tensor:
    nb = load().rabit_grad_input_workspace_bytes(layer.out_features, layer.in_features, m)
    return _ws(nb, layer.planes.device)


def grad_weight_workspace(layer: PackedLayer) -> torch.Tensor:
    nb = load().rabit_grad_weight_workspace_bytes(layer.out_features, layer.in_features)
    return _ws(nb, layer.planes.device)


def grad_input(layer: PackedLayer, dy: torch.Tensor, dx_dtype: int = RABIT_OUT_F32,
               dx: torch.Tensor | None = None, workspace: torch.Tensor | None = None,
               stream=None, weff: bool = False) -> torch.Tensor:
    """dX = dY W_hat for dY [M][out] bf16."""
    lib = load()
    assert dy.dtype == torch.bfloat16 and dy.is_contiguous()
    m = dy.shape[0]
    if dx is None:
        dt = torch.float32 if dx_dtype == RABIT_OUT_F32 else torch.bfloat16
        dx = torch.empty(m, layer.in_features, dtype=dt, device=dy.device)
    if workspace is None:
        workspace = grad_input_workspace(layer, m)
    lc = layer.c()
    _check(lib.rabit_grad_input_ex(ctypes.byref(lc), _ptr(dy), m, _ptr(dx), dx_dtype,
                                   RABIT_GEMM_WEFF if weff else 0, _ptr(workspace),
                                   workspace.numel(), _stream(stream)), "rabit_grad_input_ex")
    return dx


def grad_weight(layer: PackedLayer, x: torch.Tensor, dy: torch.Tensor, dw=None, dg=None, dh=None,
                accumulate: bool = False, workspace: torch.Tensor | None = None, stream=None):
    """(dW [out][in], dg [P][out], dh [P][in]) in float32 for X [M][in] and
    dY [M][out] (bf16)."""
    lib = load()
    assert x.dtype == torch.bfloat16 and dy.dtype == torch.bfloat16
    assert x.is_contiguous() and dy.is_contiguous() and x.shape[0] == dy.shape[0]
    m, dev, P = x.shape[0], x.device, layer.n_paths
    if dw is None:
        dw = torch.empty(layer.out_features, layer.in_features, dtype=torch.float32, device=dev)
    if dg is None:
        dg = torch.empty(P, layer.out_features, dtype=torch.float32, device=dev)
    if dh is None:
        dh = torch.empty(P, layer.in_features, dtype=torch.float32, device=dev)
    if workspace is None:
        workspace = grad_weight_workspace(layer)
    lc = layer.c()
    _check(lib.rabit_grad_weight(ctypes.byref(lc), _ptr(x), _ptr(dy), m, _ptr(dw), _ptr(dg),
                                 _ptr(dh), RABIT_GRAD_ACCUMULATE if accumulate else 0,
                                 _ptr(workspace), workspace.numel(), _stream(stream)),
           "rabit_grad_weight")
    return dw, dg, dh


# --- initialisation (rabit_svid_init in rabit.h) ---
RABIT_SVID_CONTINUE = 1


def svid_workspace(out: int, inp: int, device="cuda") -> torch.Tensor:
    return _ws(load().rabit_svid_workspace_bytes(out, inp), device)


def svid_init(w: torch.Tensor, n_paths: int = 2, sweeps: int = 20, power_passes: int = 5,
              f_out: torch.Tensor | None = None, f_in: torch.Tensor | None = None,
              g: torch.Tensor | None = None, h: torch.Tensor | None = None,
              planes: torch.Tensor | None = None, cont: bool = False,
              workspace: torch.Tensor | None = None, stream=None):
    """Iterative residual SVID of w (float32 [out, in], cuda): returns
    (g [P][out], h [P][in] float32, planes uint8 in layout V1)."""
    lib = load()
    assert w.dtype == torch.float32 and w.is_contiguous()
    out, inp = w.shape
    dev = w.device
    if g is None:
        g = torch.zeros(n_paths, out, dtype=torch.float32, device=dev)
    if h is None:
        h = torch.zeros(n_paths, inp, dtype=torch.float32, device=dev)
    if planes is None:
        planes = torch.zeros(planes_bytes(out, inp, n_paths), dtype=torch.uint8, device=dev)
    if workspace is None:
        workspace = svid_workspace(out, inp, dev)
    _check(lib.rabit_svid_init(_ptr(w), out, inp, n_paths, sweeps, power_passes, _ptr(f_out),
                               _ptr(f_in), RABIT_SVID_CONTINUE if cont else 0, _ptr(g), _ptr(h),
                               _ptr(planes), _ptr(workspace), workspace.numel(), _stream(stream)),
           "rabit_svid_init")
    return g, h, planes


MATRICES = ("q", "k", "v", "o", "gate", "up", "down")


@dataclass
class DecoderCfg:
    hidden: int
    ffn: int
    n_heads: int = 1
    n_kv_heads: int = 1
    head_dim: int = 1
    n_layers: int = 1
    rms_eps: float = 1e-5
    mlp_only: bool = False

    def c(self) -> DecoderCfgC:
        return DecoderCfgC(self.hidden, self.ffn, self.n_heads, self.n_kv_heads, self.head_dim,
                           self.n_layers, self.rms_eps, int(self.mlp_only))


def decode_workspace(cfg: DecoderCfg, batch: int, device="cuda") -> torch.Tensor:
    cc = cfg.c()
    nb = load().rabit_decode_workspace_bytes(ctypes.byref(cc), batch)
    if nb == 0:
        raise RabitError(RABIT_ESHAPE, "rabit_decode_workspace_bytes")
    return _ws(nb, device)


def layer_array(cfg: DecoderCfg, layers: list[dict]):
    """ctypes array [n_layers * 7] in q,k,v,o,gate,up,down order."""
    arr = (RabitLayerC * (7 * cfg.n_layers))()
    for li, mats in enumerate(layers):
        for mi, name in enumerate(MATRICES):
            pl = mats.get(name)
            if pl is not None:
                arr[li * 7 + mi] = pl.c()
    return arr


def decode_step(cfg: DecoderCfg, layers, x: torch.Tensor, out: torch.Tensor | None = None,
                workspace: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """One decode step through cfg.n_layers blocks; layers is a list of dicts
    name -> PackedLayer, or a prebuilt layer_array."""
    lib = load()
    assert x.dtype == torch.bfloat16 and x.is_contiguous()
    batch = x.shape[0]
    if out is None:
        out = torch.empty_like(x)
    if workspace is None:
        workspace = decode_workspace(cfg, batch, x.device)
    arr = layers if isinstance(layers, ctypes.Array) else layer_array(cfg, layers)
    cc = cfg.c()
    _check(lib.rabit_decode_step(ctypes.byref(cc), arr, _ptr(x), batch, _ptr(out),
                                 _ptr(workspace), workspace.numel(), _stream(stream)),
           "rabit_decode_step")
    return out


def stream_read(t: torch.Tensor, sink: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """Measurement hook: read all bytes of the device tensor t once (see
    rabit_stream_read); returns the sink buffer."""
    lib = load()
    assert t.is_cuda and t.is_contiguous()
    if sink is None:
        sink = torch.empty(4, dtype=torch.int32, device=t.device)
    _check(lib.rabit_stream_read(_ptr(t), t.numel() * t.element_size(), _ptr(sink), _stream(stream)),
           "rabit_stream_read")
    return sink


def test_f64_to_16(v: torch.Tensor, bf16: int, stream=None) -> torch.Tensor:
    """bf16: 0 fp16, 1 bfloat16, 2 the short bfloat16 path of the RMSNorm prologues."""
    lib = load()
    assert v.dtype == torch.float64 and v.is_cuda
    out = torch.empty(v.numel(), dtype=torch.int16, device=v.device)
    _check(lib.rabit_test_f64_to_16(_ptr(v), _ptr(out), v.numel(), int(bf16), _stream(stream)),
           "rabit_test_f64_to_16")
    return out
