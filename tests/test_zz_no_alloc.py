"""The allocation-free GEMV (rabit_gemv_noalloc, through the C ABI) against
rabit_gemv with a caller workspace: the same kernels, so the outputs must be
bit-identical; two calls in a row share the library's scratch, the second
with a smaller input, and the last call's partials must not leak into the
next."""
import sys

import numpy as np
import pytest
import torch

from synth.inputs import act_bf16, weight_f32

pytestmark = pytest.mark.gpu


def say(*a):
    print("[case]", *a, flush=True)
    sys.stdout.flush()


def _layer(rabit, out, inp, seed, n_paths=2):
    w = weight_f32(out, inp, seed)
    L = rabit.PackedLayer.empty(out, inp, n_paths=n_paths)
    rabit.pack(w.cuda(), L)
    return L


def test_gemv_noalloc_matches_gemv(gpu_lib):
    rabit = gpu_lib
    cases = [(4096, 11008, 4, 2), (1000, 3000, 1, 2), (8192, 28672, 1, 2), (300, 1100, 3, 3),
             (2048, 4096, 12, 2), (300, 1100, 3, 2)]
    prev = None
    for out, inp, batch, P in cases:
        say("gemv_noalloc", out, inp, "batch", batch, "paths", P)
        L = _layer(rabit, out, inp, out + inp + P, P)
        x = act_bf16(batch, inp, 7 * batch + inp).cuda()
        for dtype, tdt in ((rabit.RABIT_OUT_F32, torch.float32), (rabit.RABIT_OUT_BF16, torch.bfloat16)):
            ref = rabit.gemv(L, x, y_dtype=dtype)
            y = torch.full((batch, out), float("nan"), dtype=tdt, device="cuda")
            rabit.gemv_noalloc(L, x, y, dtype)
            torch.cuda.synchronize()
            assert torch.equal(y.view(torch.int16) if tdt == torch.bfloat16 else y.view(torch.int32),
                               ref.view(torch.int16) if tdt == torch.bfloat16 else ref.view(torch.int32))
        prev = (L, x)
    # a second call right after a larger one, repeated: identical bits
    L, x = prev
    y1 = torch.empty(x.shape[0], L.out_features, device="cuda")
    y2 = torch.empty_like(y1)
    rabit.gemv_noalloc(L, x, y1)
    big = _layer(rabit, 4096, 11008, 5)
    yb = torch.empty(4, 4096, device="cuda")
    rabit.gemv_noalloc(big, act_bf16(4, 11008, 3).cuda(), yb)
    rabit.gemv_noalloc(L, x, y2)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2)


def test_gemv_noalloc_too_large_is_rejected(gpu_lib):
    rabit = gpu_lib
    L = _layer(rabit, 28672, 8192, 11)
    x = act_bf16(9, 8192, 12).cuda()
    y = torch.empty(9, 28672, device="cuda")
    with pytest.raises(rabit.RabitError) as e:
        rabit.gemv_noalloc(L, x, y)
    assert e.value.code == rabit.RABIT_ESCRATCH
    # at the limit's largest batch it runs and matches
    x8 = x[:8].contiguous()
    y8 = torch.empty(8, 28672, device="cuda")
    rabit.gemv_noalloc(L, x8, y8)
    assert torch.equal(y8, rabit.gemv(L, x8))
