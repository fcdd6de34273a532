"""HIP graph replay of the library's launch sequences (the decode benchmark
replays the decode step from a graph). Every replay, with eager work and
synchronisations between the replays, must give the eager result bit for
bit: the kernels keep no state between calls and the library records no
memset or copy nodes. Inputs changed in place between replays are picked up.
"""
import pytest
import torch

from synth.inputs import weight_f32, act_bf16

pytestmark = pytest.mark.gpu


def say(*a):
    print("[case]", *a, flush=True)


def pack(rabit, out, inp, seed, paths=2):
    layer = rabit.PackedLayer.empty(out, inp, n_paths=paths)
    rabit.pack(weight_f32(out, inp, seed).cuda(), layer)
    return layer


def capture(fn):
    """Warm fn up on a side stream, then capture it into a graph (as torch
    requires for capture)."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def eager_noise():
    # unrelated eager kernels between replays
    a = torch.randn(512, 512, device="cuda")
    (a @ a).sum().item()


def same_bits(a, b):
    return torch.equal(a.view(torch.int16) if a.dtype == torch.bfloat16 else a.view(torch.int32),
                       b.view(torch.int16) if b.dtype == torch.bfloat16 else b.view(torch.int32))


@pytest.mark.parametrize("mlp_only,batch", [(True, 1), (False, 1), (False, 4), (False, 12), (True, 9), (True, 40)])
def test_decode_step_graph_replays(gpu_lib, mlp_only, batch):
    say("decode step graph replay, mlp_only", mlp_only, "batch", batch)
    cfg = gpu_lib.DecoderCfg(hidden=1024, ffn=2752, n_heads=8, n_kv_heads=2, head_dim=128, n_layers=2,
                             mlp_only=mlp_only)
    H, F, kv = cfg.hidden, cfg.ffn, cfg.n_kv_heads * cfg.head_dim
    shapes = {"q": (H, H), "k": (kv, H), "v": (kv, H), "o": (H, H), "gate": (F, H), "up": (F, H), "down": (H, F)}
    names = ["gate", "up", "down"] if mlp_only else list(shapes)
    layers = [{n: pack(gpu_lib, *shapes[n], 1300 + 10 * li + len(n)) for n in names}
              for li in range(cfg.n_layers)]
    x = act_bf16(batch, H, 1390 + batch).cuda()
    out = torch.empty_like(x)
    ws = gpu_lib.decode_workspace(cfg, batch, x.device)
    step = lambda: gpu_lib.decode_step(cfg, layers, x, out=out, workspace=ws)  # noqa: E731
    step()
    torch.cuda.synchronize()
    ref = out.clone()
    g = capture(step)
    for rep in range(3):
        out.zero_()
        eager_noise()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert same_bits(out, ref), rep
    # a new input written in place is picked up by the next replay
    x.copy_(act_bf16(batch, H, 1490 + batch).cuda())
    step()
    torch.cuda.synchronize()
    ref2 = out.clone()
    assert not same_bits(ref2, ref)
    out.zero_()
    g.replay()
    torch.cuda.synchronize()
    assert same_bits(out, ref2)
    del g


@pytest.mark.parametrize("weff", [False, True])
@pytest.mark.parametrize("shape", [(1024, 4096, 512), (4096, 1024, 300)])
def test_gemm_graph_replays(gpu_lib, shape, weff):
    # (1024, 4096, 512): split-K with the ordered reduce; (4096, 1024, 300): one slice
    out_f, inp, m = shape
    say("gemm graph replay", shape, "weff", weff)
    layer = pack(gpu_lib, out_f, inp, 1500 + m)
    X = act_bf16(m, inp, 1600 + m).cuda()
    y = torch.empty(m, out_f, dtype=torch.float32, device="cuda")
    ws = gpu_lib.gemm_workspace(layer, m)
    call = lambda: gpu_lib.gemm(layer, X, y=y, workspace=ws, weff=weff)  # noqa: E731
    call()
    torch.cuda.synchronize()
    ref = y.clone()
    g = capture(call)
    for rep in range(3):
        y.fill_(float("nan"))
        eager_noise()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert same_bits(y, ref), rep
    X.copy_(act_bf16(m, inp, 1700 + m).cuda())
    call()
    torch.cuda.synchronize()
    ref2 = y.clone()
    y.zero_()
    g.replay()
    torch.cuda.synchronize()
    assert same_bits(y, ref2)
    del g
