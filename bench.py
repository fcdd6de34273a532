#!/usr/bin/env python3
"""Benchmark of the RaBiT 2-path residual-binary hot path on one MI355X.

Metric: W2 residual-binary GEMV packed-weight GB/s (% HBM peak) + decode
tokens/s. Default workload: the Llama-2-70B-shaped stack on one GPU (80
layers, hidden 8192, FFN 28672, 64 query and 8 key/value heads of 128; every
linear layer 2-path packed, 17.1 GB of planes), decode at batch 1 (the timed
steps) and batch 32 (reported alongside). Weights are random-init
W ~ 0.02 N(0,1) packed by rabit_pack (mean-|.| scales; the derive/pack of all
weights is timed too); activations are bf16 N(0,1).

A step is one rabit_decode_step through the 80 layers, replayed from a HIP
graph. Per layer the library runs: [q,k,v] GEMV on RMSNorm(x) in one launch,
q/k/v range sums + one-token attention, o GEMV, x + o with its x^2
statistics, [gate,up] GEMV on RMSNorm in one launch, SiLU(gate)*up, down
GEMV, x + down with its statistics.

value = plane bytes per step / whole-step time (every kernel of the step).
linear_only: the step's GEMV launches alone (the plane-streaming kernels of
the linear layers), captured back to back in a HIP graph and replayed between
HIP events on the launch stream: tokens/s and plane GB/s from their time.
roofline: the dominant kernel, k_gemv (the plane-streaming GEMV), over the
step's four launch shapes: algorithmic bytes of all of them / their total
time (so avg bytes per launch / avg launch duration). traffic comes from the
committed rocprofv3 counter summary when it was taken on the current GEMV
source, else null. stream_ceiling: a plain read-only stream of the same plane
bytes as each launch shape, measured in the same run.

Printed: one JSON line (stdout). Diagnostics go to stderr. The other
configurations (--workload ...) print one JSON line each.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X published HBM3E bandwidth
GEMV_SRC = os.path.join(ROOT, "bit_residual_binarized_amd", "csrc", "gemv.hip")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "k_gemv_llama2_70b_decode_b1_traffic.txt")

L70 = dict(H=8192, F=28672, KV=1024, L=80, n_heads=64, n_kv_heads=8, head_dim=128)


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def mlp_shapes(hidden=4096, ffn=11008):
    return {"gate": (ffn, hidden), "up": (ffn, hidden), "down": (hidden, ffn)}


def layer_shapes(H, F, KV):
    return {"q": (H, H), "k": (KV, H), "v": (KV, H), "o": (H, H), "gate": (F, H), "up": (F, H),
            "down": (H, F)}


def gemv_alg_bytes(out, inp, b=1):
    """Algorithmic bytes of one GEMV: planes (0.25 B/weight), fp16 g and h of
    both paths, bf16 x, fp32 y."""
    return out * inp // 4 + 4 * (out + inp) + 2 * b * inp + 4 * b * out


def launch_alg_bytes(outs, inp, b=1):
    """One launch over several matrices that read the same x (x counted once)."""
    return sum(gemv_alg_bytes(o, inp, b) for o in outs) - (len(outs) - 1) * 2 * b * inp


def gemv_source_sha():
    with open(GEMV_SRC, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def committed_traffic(path=TRAFFIC_FILE):
    """HBM bytes per k_gemv launch from the committed counter summary, or
    None when it is missing or was taken on another GEMV source."""
    try:
        kv = {}
        with open(path) as f:
            for line in f:
                if ":" in line and not line.startswith("#"):
                    k, v = line.split(":", 1)
                    kv[k.strip()] = v.strip()
        if kv.get("gemv_source_sha256") != gemv_source_sha():
            return None
        return float(kv["traffic_bytes_per_launch"])
    except (OSError, KeyError, ValueError):
        return None


def build_copies(rabit, torch, copies, shapes, cfg_id=2):
    """Generate and pack `copies` distinct copies of the matrices in `shapes`."""
    from synth.inputs import weight_f32, seed_w
    layers, pack_ms = [], []
    ws = None
    for c in range(copies):
        d = {}
        for name, (o, i) in shapes.items():
            w = weight_f32(o, i, seed_w(cfg_id, c, name), device="cuda")
            pl = rabit.PackedLayer.empty(o, i)
            need = rabit.load().rabit_pack_workspace_bytes(o, i)
            if ws is None or ws.numel() < need:
                ws = torch.empty(need, dtype=torch.uint8, device="cuda")
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            rabit.pack(w, pl, workspace=ws)
            e1.record()
            e1.synchronize()
            pack_ms.append((name, o, i, e0.elapsed_time(e1)))
            del w
            d[name] = pl
        layers.append(d)
    return layers, pack_ms


def cpu_baseline_mlp(shapes, budget_s):
    """The oracle (float64 numpy) on the host: derive one copy of the block,
    then time its GEMV path (W_eff reconstruction + matmul) for the three
    matrices, repeated until about `budget_s` seconds of work."""
    import oracle
    from synth.inputs import weight_f32, act_bf16, bf16_values, seed_w, seed_x
    try:
        from threadpoolctl import threadpool_info
        blas = [(t.get("internal_api"), t.get("num_threads")) for t in threadpool_info()]
    except Exception:  # pragma: no cover
        blas = []
    ds = {}
    t0 = time.perf_counter()
    for name, (o, i) in shapes.items():
        ds[name] = oracle.derive(weight_f32(o, i, seed_w(2, 0, name)).numpy())
    t_derive = time.perf_counter() - t0
    weights = sum(o * i for o, i in shapes.values())
    x = bf16_values(act_bf16(1, shapes["gate"][1], seed_x(2, 1)))
    reps, t_gemv = 0, 0.0
    while t_gemv < budget_s and reps < 20:
        t1 = time.perf_counter()
        oracle.mlp_block(x, ds["gate"], ds["up"], ds["down"])
        t_gemv += time.perf_counter() - t1
        reps += 1
    plane_bytes = sum(oracle.planes_bytes(o, i) for o, i in shapes.values())
    return {
        "value": round(plane_bytes * reps / t_gemv / 1e9, 4),
        "unit": "GB/s",
        "cores": len(os.sched_getaffinity(0)),
        "kind": "oracle",
        "sample": (f"{reps} x one MLP block (gate/up 11008x4096, down 4096x11008) at batch 1: "
                   "oracle float64 W_eff reconstruction + matmul; GB/s of packed-plane bytes"),
        "blas_threads": blas,
        "ms_per_block": round(1e3 * t_gemv / reps, 3),
        "derive_pack_s": round(t_derive, 3),
        "derive_pack_gbs_w_read": round(8 * weights / t_derive / 1e9, 4),
    }


def graph_ms(torch, fn, reps):
    """fn() enqueues a sequence of launches on the current stream; it is
    captured once into a HIP graph and replayed `reps` times between two
    events, so that the launches run back to back on the GPU (Python-side
    launch overhead would otherwise leave gaps). Returns ms per replay."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()  # eager warm-up
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    del g
    return e0.elapsed_time(e1) / reps


def dist_summary(vals):
    """Median, p10 and p90 of a list of timings (nearest-rank percentiles)."""
    v = sorted(vals)
    pick = lambda q: v[min(len(v) - 1, max(0, int(round(q * (len(v) - 1)))))]
    return {"median": pick(0.5), "p10": pick(0.1), "p90": pick(0.9), "n": len(v)}


def graph_ms_dist(torch, fn, reps):
    """As graph_ms, but one event after every replay: the list of per-replay
    times (ms), for the distribution over repetitions."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    g.replay()
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
    ev[0].record()
    for k in range(reps):
        g.replay()
        ev[k + 1].record()
    torch.cuda.synchronize()
    del g
    return [ev[k].elapsed_time(ev[k + 1]) for k in range(reps)]


def stream_read_ms(rabit, torch, nbytes, reps=8):
    """Practical ceiling: a plain read-only stream of nbytes (rabit_stream_read,
    16-byte loads like the GEMV's plane loads) over rotating cold buffers
    (>= 512 MiB in total), graph-replayed back to back; ms per call."""
    n = max(16, nbytes // 16 * 16)
    copies = max(2, -(-(512 << 20) // n))
    bufs = [torch.ones(n, dtype=torch.uint8, device="cuda") for _ in range(copies)]
    sink = torch.empty(4, dtype=torch.int32, device="cuda")

    def run():
        for b in bufs:
            rabit.stream_read(b, sink)
    ms = graph_ms(torch, run, reps) / copies
    del bufs
    return ms


def time_gemv_launches(rabit, torch, layers, hidden, ffn, reps=5):
    """Average duration of the step's two k_gemv<1> launch shapes, each timed
    as `len(layers)` back-to-back launches (one per layer, cold planes),
    captured in a HIP graph and replayed `reps` times between two events on
    the launch stream."""
    x_h = torch.randn(1, hidden, device="cuda").to(torch.bfloat16)
    x_f = torch.randn(1, ffn, device="cuda").to(torch.bfloat16)
    ws_gu = rabit.gemv_multi_workspace([layers[0]["gate"], layers[0]["up"]], 1)
    ws_d = rabit.gemv_workspace(layers[0]["down"], 1)

    def gate_up():
        for L in layers:
            rabit.gemv_partial_multi([L["gate"], L["up"]], x_h, ws_gu)

    def down():
        for L in layers:
            rabit.gemv_partial(L["down"], x_f, ws_d)
    med = {kind: graph_ms(torch, fn, reps) / len(layers) for kind, fn in (("gate+up", gate_up), ("down", down))}
    return med, dict(med)


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--layers", type=int, default=None,
                    help="layers of the stack (default: 80 for llama70b, 32 for mlp7b)")
    ap.add_argument("--cpu-budget-s", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-graph", action="store_true", help="launch eagerly instead of graph replay")
    ap.add_argument("--workload", default="llama70b",
                    choices=["llama70b", "mlp7b", "layer4096", "llama3-8b", "gemm", "table7", "train",
                             "init", "crossover"],
                    help="llama70b (default): the headline decode workload; the others measure the "
                         "remaining configurations (one JSON line each)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the library and every kernel run on a single device, and "
              "the multi-GPU split is a design only. Run it with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch
    from bit_residual_binarized_amd import rabit

    rabit.load()
    torch.cuda.set_device(0)
    fn = {"llama70b": bench_llama70b, "mlp7b": bench_mlp7b, "layer4096": bench_layer4096,
          "llama3-8b": bench_llama3_8b, "gemm": bench_gemm, "table7": bench_table7, "train": bench_train,
          "init": bench_init, "crossover": bench_crossover}[args.workload]
    print(json.dumps(fn(args, rabit, torch)), flush=True)


def bench_mlp7b(args, rabit, torch):
    """32 Llama-2-7B MLP blocks per decode step at batch 1 (gate and up
    11008x4096, down 4096x11008, SiLU gating), graph replay."""
    from synth.inputs import act_bf16, seed_x
    args.layers = args.layers or 32
    hidden, ffn = 4096, 11008
    shapes = mlp_shapes(hidden, ffn)
    cfg = rabit.DecoderCfg(hidden=hidden, ffn=ffn, n_layers=args.layers, mlp_only=True)

    t0 = time.time()
    log(f"packing {args.layers} MLP blocks ...")
    layers, pack_ms = build_copies(rabit, torch, args.layers, shapes)
    torch.cuda.synchronize()
    log(f"packed in {time.time() - t0:.1f} s")
    plane_bytes_block = sum(rabit.planes_bytes(o, i) for o, i in shapes.values())
    plane_bytes_step = plane_bytes_block * args.layers

    arr = rabit.layer_array(cfg, layers)
    x0 = act_bf16(1, hidden, seed_x(2, 1)).cuda()
    bufs = [x0.clone(), torch.empty_like(x0)]
    ws = rabit.decode_workspace(cfg, 1)

    def step(i):
        rabit.decode_step(cfg, arr, bufs[i % 2], out=bufs[(i + 1) % 2], workspace=ws)

    # eager reference of two steps, then the graph of one step
    bufs[0].copy_(x0)
    step(0)
    step(1)
    torch.cuda.synchronize()
    eager_out = bufs[0].clone()
    graphs = None
    if not args.no_graph:
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            step(0)  # warm the capture path
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        graphs = []
        for par in (0, 1):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                step(par)
            graphs.append(g)
        torch.cuda.synchronize()
        # graph replays must reproduce the eager steps
        bufs[0].copy_(x0)
        graphs[0].replay()
        graphs[1].replay()
        torch.cuda.synchronize()
        assert torch.equal(bufs[0], eager_out), "graph replay differs from eager run"

    def run_steps(n, start=0):
        for k in range(start, start + n):
            if graphs is not None:
                graphs[k % 2].replay()
            else:
                step(k)
        return start + n

    bufs[0].copy_(x0)
    nxt = run_steps(args.warmup)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    run_steps(args.steps, nxt)
    e1.record()
    torch.cuda.synchronize()
    total_ms = e0.elapsed_time(e1)
    ms_step = total_ms / args.steps
    gbs = plane_bytes_step * args.steps / (total_ms * 1e-3) / 1e9
    log(f"{args.steps} steps of {args.layers} MLP blocks in {total_ms:.3f} ms: {ms_step * 1e3:.1f} us/step, "
        f"{ms_step * 1e3 / args.layers:.2f} us/block, {gbs:.1f} GB/s of planes")

    # dominant kernel: k_gemv<1>, both launch shapes of the step
    med, raw = time_gemv_launches(rabit, torch, layers, hidden, ffn)
    gu_bytes = gemv_alg_bytes(*shapes["gate"]) + gemv_alg_bytes(*shapes["up"]) - 2 * hidden
    d_bytes = gemv_alg_bytes(*shapes["down"])
    kavg_ms = (med["gate+up"] + med["down"]) / 2
    alg_bytes = (gu_bytes + d_bytes) / 2
    achieved = alg_bytes / (kavg_ms * 1e-3) / 1e9
    log(f"k_gemv<1>: gate+up {med['gate+up'] * 1e3:.2f} us, down {med['down'] * 1e3:.2f} us per launch "
        f"-> {achieved:.1f} GB/s algorithmic")
    traffic = committed_traffic(os.path.join(ROOT, "profiles", "k_gemv_llama2_7b_mlp_b1_traffic.txt"))
    # practical ceilings at the two launch sizes (planes only) and for a large copy
    gu_planes = 2 * shapes["gate"][0] * shapes["gate"][1] // 4
    d_planes = shapes["down"][0] * shapes["down"][1] // 4
    st_gu, st_d = stream_read_ms(rabit, torch, gu_planes), stream_read_ms(rabit, torch, d_planes)
    big_a = torch.empty(256 << 20, dtype=torch.uint8, device="cuda").fill_(1)
    big_b = torch.empty_like(big_a)
    big_b.copy_(big_a)
    torch.cuda.synchronize()
    c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    c0.record()
    for _ in range(10):
        big_b.copy_(big_a)
    c1.record()
    torch.cuda.synchronize()
    copy_gbs = 2 * (256 << 20) * 10 / (c0.elapsed_time(c1) * 1e-3) / 1e9
    del big_a, big_b
    stream = {
        "read_only_us": {"gate+up planes": round(st_gu * 1e3, 2), "down planes": round(st_d * 1e3, 2)},
        "read_only_gbs": {"gate+up planes": round(gu_planes / (st_gu * 1e-3) / 1e9, 1),
                          "down planes": round(d_planes / (st_d * 1e-3) / 1e9, 1)},
        "copy_256MiB_gbs_read_plus_write": round(copy_gbs, 1),
        "gemv_launch_over_read_only": {"gate+up": round(med["gate+up"] / st_gu, 3),
                                       "down": round(med["down"] / st_d, 3)},
        "note": "rabit_stream_read (16-byte loads) over cold rotating buffers of the same byte size as each "
                "launch's planes; copy is torch copy_ (read + write bytes)",
    }
    log(f"streaming ceiling: {stream}")

    pk = pack_ms[3:] or pack_ms
    pk_ms = sum(p[3] for p in pk) / len(pk)
    pk_weights = sum(p[1] * p[2] for p in pk) / len(pk)
    derive = {
        "ms_per_matrix": round(pk_ms, 4),
        "alg_bytes_per_weight": 8.25,
        "gbs": round(8.25 * pk_weights / (pk_ms * 1e-3) / 1e9, 1),
        "frac_hbm": round(8.25 * pk_weights / (pk_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        "note": "rabit_pack MEANABS: 2 reads of W fp32 + planes; event-timed per matrix",
    }

    # plain device copy of a known size: the counter summaries use it to
    # calibrate FETCH_SIZE / WRITE_SIZE
    cal_a = torch.empty(256 << 20, dtype=torch.uint8, device="cuda").fill_(1)
    cal_b = torch.empty_like(cal_a)
    cal_b.copy_(cal_a)
    torch.cuda.synchronize()
    del cal_a, cal_b

    cpu = None
    if not args.no_cpu_baseline:
        log("timing the CPU oracle baseline ...")
        cpu = cpu_baseline_mlp(shapes, args.cpu_budget_s)
        log(f"cpu oracle: {cpu}")

    res = {
        "metric": "W2 residual-binary GEMV packed-weight GB/s (% HBM peak) + decode tokens/s",
        "value": round(gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp4xfp6",
        "data": "synthetic",
        "config": {"workload": "llama2-7b-mlp-block-decode-b1", "hidden": hidden, "ffn": ffn,
                   "batch": 1, "blocks_per_step": args.layers, "graph_replay": graphs is not None,
                   "plane_bytes_per_step": plane_bytes_step},
        "pct_hbm_peak": round(100.0 * gbs / HBM_PEAK_GBS, 2),
        "us_per_block": round(ms_step * 1e3 / args.layers, 3),
        "decode_tokens_per_s": round(1e3 / ms_step, 1),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": None if traffic is None else int(traffic),
                     "kernel": "k_gemv<1>", "avg_launch_us": round(kavg_ms * 1e3, 3),
                     "launch_us": {k: round(v * 1e3, 3) for k, v in med.items()},
                     "alg_bytes_per_launch": int(alg_bytes)},
        "stream_ceiling": stream,
        "derive_pack": derive,
        "cpu_baseline": cpu,
    }
    return res


# ---------------------------------------------------------------------------
# The other configurations (not the headline line; one JSON line each)
# ---------------------------------------------------------------------------
def _pack_layer(rabit, torch, out, inp, seed, ws_holder):
    from synth.inputs import weight_f32
    w = weight_f32(out, inp, seed, device="cuda")
    pl = rabit.PackedLayer.empty(out, inp)
    need = rabit.load().rabit_pack_workspace_bytes(out, inp)
    if ws_holder[0] is None or ws_holder[0].numel() < need:
        ws_holder[0] = torch.empty(need, dtype=torch.uint8, device="cuda")
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    rabit.pack(w, pl, workspace=ws_holder[0])
    e1.record()
    e1.synchronize()
    del w
    return pl, e0.elapsed_time(e1)


def pack_graph_ms(rabit, torch, out, inp, seed, reps=5):
    """GPU time of one rabit_pack (MEANABS) of an out x inp fp32 matrix,
    captured in a HIP graph and replayed back to back (ms per call; the
    host-side call overhead, which a per-call event pair around the Python
    call also measures, is excluded)."""
    from synth.inputs import weight_f32
    w = weight_f32(out, inp, seed, device="cuda")
    pl = rabit.PackedLayer.empty(out, inp)
    ws = torch.empty(rabit.load().rabit_pack_workspace_bytes(out, inp), dtype=torch.uint8, device="cuda")
    ms = graph_ms(torch, lambda: rabit.pack(w, pl, workspace=ws), reps)
    del w, pl, ws
    return ms


def _events_ms(torch, fn, n, reps=3):
    """ms per call of fn(i), i = 0..n-1, captured in a HIP graph and replayed
    back to back (Python launch overhead excluded)."""
    def run():
        for i in range(n):
            fn(i)
    return graph_ms(torch, run, reps) / n


def _line(metric, value, unit, config, higher=True, **kw):
    d = {"metric": metric, "value": value, "unit": unit, "n_gpus": 1, "higher_is_better": higher,
         "vs_baseline": None, "data": "synthetic", "config": config}
    d.update(kw)
    return d


def _blas_info():
    try:
        from threadpoolctl import threadpool_info
        return [(t.get("internal_api"), t.get("num_threads")) for t in threadpool_info()]
    except Exception:  # pragma: no cover
        return []


def cpu_baseline_layers(rabit, shapes, cfg_id, batches=(1,)):
    """The oracle (float64 numpy) on the host over whole matrices: derive with
    mean-|.| scales and pack each matrix (timed), then its GEMV (W_eff
    reconstruction + product) at each batch. value = plane bytes / GEMV time
    at batch 1 (all matrices)."""
    import numpy as np
    import oracle
    from synth.inputs import act_bf16, bf16_values, seed_w, seed_x, weight_f32
    t_derive, t_gemv = 0.0, {b: 0.0 for b in batches}
    weights = 0
    for k, (name, (o, i)) in enumerate(shapes.items()):
        w = weight_f32(o, i, seed_w(cfg_id, 0, name)).numpy()
        t0 = time.perf_counter()
        d = oracle.derive(w)
        oracle.pack_words(d.s1), oracle.pack_words(d.s2)
        t_derive += time.perf_counter() - t0
        d.r = None
        weights += o * i
        del w
        for b in batches:
            x = bf16_values(act_bf16(b, i, seed_x(cfg_id, b)))
            t0 = time.perf_counter()
            oracle.gemv(d, x)
            t_gemv[b] += time.perf_counter() - t0
        del d
    planes = sum(rabit.planes_bytes(o, i) for o, i in shapes.values())
    return {
        "value": round(planes / t_gemv[batches[0]] / 1e9, 5), "unit": "GB/s",
        "cores": len(os.sched_getaffinity(0)), "kind": "oracle",
        "sample": (f"the whole workload ({weights / 1e6:.0f} M weights): oracle mean-|.| derive + pack of every "
                   "matrix, then its float64 GEMV (W_eff reconstruction + product) at batch "
                   + ", ".join(str(b) for b in batches) + "; GB/s of packed-plane bytes at batch "
                   + str(batches[0])),
        "derive_pack_s": round(t_derive, 3),
        "gemv_s": {str(b): round(v, 3) for b, v in t_gemv.items()},
        "blas_threads": _blas_info(),
    }


def cpu_baseline_gemm(rabit, NK, Ms=(512, 2048, 8192), rows=256):
    """The oracle's prefill GEMM (W_eff in float64, then X W_eff^T): M = 512 in
    full, larger M on `rows` token rows, extrapolated linearly in M."""
    import oracle
    from synth.inputs import act_bf16, bf16_values, seed_w, seed_x, weight_f32
    res, tot_flop, tot_s = {}, 0.0, 0.0
    for (N, K) in NK:
        w = weight_f32(N, K, seed_w(4, 0, "gate" if N > K else "down")).numpy()
        t0 = time.perf_counter()
        d = oracle.derive(w)
        t_derive = time.perf_counter() - t0
        d.r = None
        del w
        for M in Ms:
            xm = bf16_values(act_bf16(M, K, seed_x(4, M)))
            sub = None if M <= 512 else list(range(0, M, max(1, M // rows)))[:rows]
            n = M if sub is None else len(sub)
            t0 = time.perf_counter()
            oracle.gemm(d, xm, rows=sub)
            dt = time.perf_counter() - t0
            full = dt * M / n
            res[f"{N}x{K}_M{M}"] = {"s": round(full, 3), "extrapolated": sub is not None,
                                    "tflops": round(4.0 * M * N * K / full / 1e12, 5)}
            tot_flop += 4.0 * M * N * K
            tot_s += full
        res[f"{N}x{K}_derive_s"] = round(t_derive, 3)
    return {"value": round(tot_flop / tot_s / 1e12, 5), "unit": "TFLOP/s", "cores": len(os.sched_getaffinity(0)),
            "kind": "oracle",
            "sample": (f"Llama-3-8B MLP shapes, M = 512 whole and {rows} token rows at M = 2048, 8192 "
                       "(extrapolated linearly in M, labelled): oracle W_eff reconstruction + float64 product"),
            "runs": res, "blas_threads": _blas_info()}


def bench_layer4096(args, rabit, torch):
    """One 4096x4096 layer: derive+pack then batch-1 GEMV, over 128 cold copies."""
    from synth.inputs import act_bf16, seed_w, seed_x
    n, wsh, packs = 128, [None], []
    layers = []
    for c in range(n):
        pl, ms = _pack_layer(rabit, torch, 4096, 4096, seed_w(1, c, "q"), wsh)
        layers.append(pl)
        packs.append(ms)
    x = act_bf16(1, 4096, seed_x(1, 1)).cuda()
    ws = rabit.gemv_workspace(layers[0], 1)
    y = torch.empty(1, 4096, device="cuda")
    for i in range(n):
        rabit.gemv(layers[i], x, y=y, workspace=ws)
    full = _events_ms(torch, lambda i: rabit.gemv(layers[i % n], x, y=y, workspace=ws), 4 * n)
    part = _events_ms(torch, lambda i: rabit.gemv_partial(layers[i % n], x, ws), 4 * n)
    pb = rabit.planes_bytes(4096, 4096)
    pk = sorted(packs[2:])[len(packs[2:]) // 2]
    alg = gemv_alg_bytes(4096, 4096)
    cpu = None if args.no_cpu_baseline else cpu_baseline_layers(rabit, {"q": (4096, 4096)}, 1)
    return _line("4096x4096 residual-binary GEMV packed-weight GB/s (batch 1, cold)",
                 round(pb / (full * 1e-3) / 1e9, 1), "GB/s",
                 {"workload": "single-layer-4096x4096-b1", "copies": n}, dtype="fp4xfp6",
                 us_per_gemv=round(full * 1e3, 2), us_per_partial_kernel=round(part * 1e3, 2),
                 roofline={"bound": "hbm", "achieved": round(alg / (part * 1e-3) / 1e9, 1),
                           "peak": HBM_PEAK_GBS, "unit": "GB/s",
                           "frac": round(alg / (part * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                           "kernel": "k_gemv<1>"},
                 derive_pack={"ms": round(pk, 4), "gbs": round(8.25 * 4096 * 4096 / (pk * 1e-3) / 1e9, 1)},
                 cpu_baseline=cpu)


def bench_table7(args, rabit, torch):
    """The shapes of the pages' kernel-latency table (Llama-2 7B and 13B
    projections) at batch 1: the residual-binary GEMV (rabit_gemv, both
    launches; 2-bit, and the 3-bit variant with three planes) against a dense
    bf16 GEMV (torch.mm on a contiguous [in][out]
    bf16 weight, hipBLASLt), each cold (rotating copies over >= 512 MiB) and
    warm (one copy, as the pages measured). Context only: the pages' figures
    are from another GPU."""
    from synth.inputs import act_bf16, seed_w, seed_x
    shapes = [(4096, 4096, "q_proj 7B"), (11008, 4096, "gate_proj 7B"), (5120, 5120, "q_proj 13B"),
              (13824, 5120, "gate_proj 13B")]
    runs, wsh, speed = {}, [None], []
    for si, (out, inp, name) in enumerate(shapes):
        pl, _ = _pack_layer(rabit, torch, out, inp, seed_w(6, si, "q"), wsh)
        pb = rabit.planes_bytes(out, inp)
        n = max(2, -(-(512 << 20) // pb))
        layers = [pl]
        for _ in range(n - 1):
            c = rabit.PackedLayer.empty(out, inp)
            c.planes.copy_(pl.planes)
            c.g.copy_(pl.g)
            c.h.copy_(pl.h)
            layers.append(c)
        x = act_bf16(1, inp, seed_x(6, 1)).cuda()
        ws = rabit.gemv_workspace(pl, 1)
        y = torch.empty(1, out, device="cuda")
        ours_cold = _events_ms(torch, lambda i: rabit.gemv(layers[i % n], x, y=y, workspace=ws), n)
        ours_warm = _events_ms(torch, lambda i: rabit.gemv(layers[0], x, y=y, workspace=ws), 64)
        del layers
        # the 3-bit variant (three planes) on the same shape
        from synth.inputs import weight_f32
        l3 = rabit.PackedLayer.empty(out, inp, n_paths=3)
        w = weight_f32(out, inp, seed_w(6, si, "q"), device="cuda")
        rabit.pack(w, l3, workspace=wsh[0])
        del w
        pb3 = rabit.planes_bytes(out, inp, 3)
        n3 = max(2, -(-(512 << 20) // pb3))
        layers3 = [l3]
        for _ in range(n3 - 1):
            c = rabit.PackedLayer.empty(out, inp, n_paths=3)
            c.planes.copy_(l3.planes)
            c.g.copy_(l3.g)
            c.h.copy_(l3.h)
            layers3.append(c)
        ours3_cold = _events_ms(torch, lambda i: rabit.gemv(layers3[i % n3], x, y=y, workspace=ws), n3)
        ours3_warm = _events_ms(torch, lambda i: rabit.gemv(layers3[0], x, y=y, workspace=ws), 64)
        del layers3
        wb = out * inp * 2
        nd = max(2, -(-(512 << 20) // wb))
        dense = [torch.randn(inp, out, device="cuda").mul_(0.02).to(torch.bfloat16) for _ in range(nd)]
        yd = torch.empty(1, out, device="cuda", dtype=torch.bfloat16)
        dense_cold = _events_ms(torch, lambda i: torch.mm(x, dense[i % nd], out=yd), nd)
        dense_warm = _events_ms(torch, lambda i: torch.mm(x, dense[0], out=yd), 64)
        del dense
        sp = dense_cold / ours_cold
        speed.append(sp)
        runs[f"{out}x{inp} {name}"] = {
            "rabit_us_cold": round(ours_cold * 1e3, 2), "rabit_us_warm": round(ours_warm * 1e3, 2),
            "dense_bf16_us_cold": round(dense_cold * 1e3, 2), "dense_bf16_us_warm": round(dense_warm * 1e3, 2),
            "speedup_cold": round(sp, 2), "speedup_warm": round(dense_warm / ours_warm, 2),
            "rabit_plane_gbs_cold": round(pb / (ours_cold * 1e-3) / 1e9, 1),
            "rabit3_us_cold": round(ours3_cold * 1e3, 2), "rabit3_us_warm": round(ours3_warm * 1e3, 2),
            "rabit3_speedup_cold": round(dense_cold / ours3_cold, 2),
            "dense_gbs_cold": round(wb / (dense_cold * 1e-3) / 1e9, 1)}
        log(f"{name} {out}x{inp}: {runs[f'{out}x{inp} {name}']}")
    gm = 1.0
    for v in speed:
        gm *= v
    gm **= 1.0 / len(speed)
    return _line("Residual-binary GEMV speed-up over dense bf16 GEMV, batch 1, cold (geometric mean over the "
                 "pages' 7B/13B shapes)", round(gm, 3), "x", {"workload": "table7-shapes-b1"},
                 dtype="fp4xfp6 vs bf16", runs=runs)


def bench_crossover(args, rabit, torch):
    """The GEMV (rabit_gemv) against the prefill GEMM (rabit_gemm, small-token
    tiles up to M = 32) at batch / M = 2 .. 32 on the Llama-3-8B layer shapes:
    microseconds per call, four calls per graph replay. The value is the
    smallest batch from which the GEMM is faster on every MLP shape."""
    from synth.inputs import act_bf16, seed_w, seed_x
    shapes = [(14336, 4096, "gate/up"), (4096, 14336, "down"), (4096, 4096, "q/o"), (1024, 4096, "k/v")]
    batches = (2, 4, 8, 16, 32)
    runs, wsh = {}, [None]
    first = {}
    for si, (out, inp, name) in enumerate(shapes):
        pl, _ = _pack_layer(rabit, torch, out, inp, seed_w(7, si, "q"), wsh)
        row = {}
        for b in batches:
            x = act_bf16(b, inp, seed_x(7, b)).cuda()
            y = torch.empty(b, out, device="cuda")
            wsv, wsm = rabit.gemv_workspace(pl, b), rabit.gemm_workspace(pl, b)

            def gv():
                for _ in range(4):
                    rabit.gemv(pl, x, y=y, workspace=wsv)

            def gm():
                for _ in range(4):
                    rabit.gemm(pl, x, y=y, workspace=wsm)
            tv = graph_ms(torch, gv, 20) * 1e3 / 4
            tm = graph_ms(torch, gm, 20) * 1e3 / 4
            row[str(b)] = {"gemv_us": round(tv, 1), "gemm_us": round(tm, 1), "gemv_over_gemm": round(tv / tm, 2)}
            if tm < tv and name in ("gate/up", "down"):
                first.setdefault(name, b)
            log(f"crossover {name} {out}x{inp} batch {b}: gemv {tv:.1f} us, gemm {tm:.1f} us")
        runs[f"{out}x{inp} {name}"] = row
    value = max(first.values()) if len(first) == 2 else None
    return _line("Smallest batch from which the prefill GEMM beats the GEMV on the Llama-3-8B MLP shapes",
                 value, "batch", {"workload": "llama3-8b-shapes-gemv-vs-gemm", "batches": list(batches)},
                 higher=False, dtype="fp4xfp6 vs fp16", runs=runs)


def _decoder_layers(rabit, torch, cfg_id, H, F, kv, n_layers):
    names = {"q": (H, H), "k": (kv, H), "v": (kv, H), "o": (H, H), "gate": (F, H), "up": (F, H),
             "down": (H, F)}
    from synth.inputs import seed_w
    wsh, layers, pack = [None], [], []
    for li in range(n_layers):
        d = {}
        for nm, (o, i) in names.items():
            d[nm], ms = _pack_layer(rabit, torch, o, i, seed_w(cfg_id, li, nm), wsh)
            pack.append((o * i, ms))
        layers.append(d)
    wsh[0] = None
    torch.cuda.empty_cache()
    planes = sum(rabit.planes_bytes(o, i) for o, i in names.values()) * n_layers
    return layers, planes, pack


def _time_decode(rabit, torch, cfg, layers, batch, steps):
    """ms per decode step: `steps` steps ping-ponging between two activation
    buffers, captured in one HIP graph and replayed back to back."""
    from synth.inputs import act_bf16, seed_x
    arr = rabit.layer_array(cfg, layers)
    x0 = act_bf16(batch, cfg.hidden, seed_x(3, batch)).cuda()
    bufs = [x0.clone(), torch.empty_like(x0)]
    ws = rabit.decode_workspace(cfg, batch)

    def step(i):
        rabit.decode_step(cfg, arr, bufs[i % 2], out=bufs[(i + 1) % 2], workspace=ws)

    step(0)
    step(1)
    torch.cuda.synchronize()
    ms = _events_ms(torch, step, steps)
    del ws
    return ms


def bench_llama3_8b(args, rabit, torch):
    """Llama-3-8B-shaped decode step (32 layers of the layer set) at batch 1..16."""
    H, F, kv, L = 4096, 14336, 1024, 32
    layers, planes, _ = _decoder_layers(rabit, torch, 3, H, F, kv, L)
    cfg = rabit.DecoderCfg(hidden=H, ffn=F, n_heads=32, n_kv_heads=8, head_dim=128, n_layers=L)
    sweep = {}
    for b in (1, 2, 4, 8, 16):
        ms = _time_decode(rabit, torch, cfg, layers, b, 10)
        sweep[b] = {"ms_per_step": round(ms, 4), "plane_gbs": round(planes / (ms * 1e-3) / 1e9, 1),
                    "tokens_per_s": round(b * 1e3 / ms, 1)}
        log(f"llama3-8b batch {b}: {ms:.3f} ms/step, {sweep[b]['plane_gbs']} GB/s")
    cpu = None if args.no_cpu_baseline else cpu_baseline_layers(
        rabit, layer_shapes(H, F, kv), 3, batches=(1,))
    return _line("Llama-3-8B decode step, packed-weight GB/s at batch 1 (sweep 1..16)",
                 sweep[1]["plane_gbs"], "GB/s",
                 {"workload": "llama3-8b-decode-32-layers", "batch": [1, 2, 4, 8, 16],
                  "plane_bytes_per_step": planes}, dtype="fp4xfp6", sweep=sweep,
                 cpu_baseline=cpu, cpu_baseline_note="the oracle over one layer's seven matrices (the step "
                 "repeats them 32 times)")


def bench_gemm(args, rabit, torch):
    """Prefill GEMM with the Llama-3-8B MLP shapes at M = 512, 2048, 8192."""
    from synth.inputs import act_bf16, seed_w, seed_x
    wsh, res, res3 = [None], {}, {}
    for (N, K) in ((14336, 4096), (4096, 14336)):
        pl, _ = _pack_layer(rabit, torch, N, K, seed_w(4, 0, "gate" if N > K else "down"), wsh)
        for M in (512, 2048, 8192):
            X = act_bf16(M, K, seed_x(4, M)).cuda()
            ws = rabit.gemm_workspace(pl, M)
            Y = torch.empty(M, N, device="cuda")
            rabit.gemm(pl, X, y=Y, workspace=ws)
            ms = _events_ms(torch, lambda i: rabit.gemm(pl, X, y=Y, workspace=ws), 10)
            tf = 4.0 * M * N * K / (ms * 1e-3) / 1e12
            res[f"{N}x{K}_M{M}"] = {"ms": round(ms, 4), "tflops": round(tf, 1),
                                    "mfma_frac_fp16": round(tf / 2500.0, 4)}
            log(f"gemm {N}x{K} M={M}: {ms:.3f} ms {tf:.1f} TFLOP/s")
            del X, ws, Y
        # the 3-bit variant (three planes): 6 M N K flops
        from synth.inputs import weight_f32
        l3 = rabit.PackedLayer.empty(N, K, n_paths=3)
        w = weight_f32(N, K, seed_w(4, 1, "gate" if N > K else "down"), device="cuda")
        rabit.pack(w, l3, workspace=wsh[0])
        del w
        for M in (2048, 8192):
            X = act_bf16(M, K, seed_x(4, M)).cuda()
            ws = rabit.gemm_workspace(l3, M)
            Y = torch.empty(M, N, device="cuda")
            rabit.gemm(l3, X, y=Y, workspace=ws)
            ms = _events_ms(torch, lambda i: rabit.gemm(l3, X, y=Y, workspace=ws), 10)
            tf = 6.0 * M * N * K / (ms * 1e-3) / 1e12
            res3[f"{N}x{K}_M{M}"] = {"ms": round(ms, 4), "tflops": round(tf, 1),
                                     "mfma_frac_fp16": round(tf / 2500.0, 4)}
            log(f"gemm 3-bit {N}x{K} M={M}: {ms:.3f} ms {tf:.1f} TFLOP/s")
            del X, ws, Y
    # the effective-weight variant (fp16 W_hat per tile): dense-equivalent 2 M N K
    resw = {}
    for (N, K) in ((14336, 4096), (4096, 14336)):
        for P in (2, 3):
            pl = rabit.PackedLayer.empty(N, K, n_paths=P)
            w = weight_f32(N, K, seed_w(4, P, "gate" if N > K else "down"), device="cuda")
            rabit.pack(w, pl, workspace=wsh[0])
            del w
            for M in (2048, 8192):
                X = act_bf16(M, K, seed_x(4, M)).cuda()
                ws = rabit.gemm_workspace(pl, M)
                Y = torch.empty(M, N, device="cuda")
                rabit.gemm(pl, X, y=Y, workspace=ws, weff=True)
                ms = _events_ms(torch, lambda i: rabit.gemm(pl, X, y=Y, workspace=ws, weff=True), 10)
                tf = 2.0 * M * N * K / (ms * 1e-3) / 1e12
                resw[f"{N}x{K}_P{P}_M{M}"] = {"ms": round(ms, 4), "tflops_dense_equiv": round(tf, 1)}
                log(f"gemm weff P={P} {N}x{K} M={M}: {ms:.3f} ms {tf:.1f} dense-equivalent TFLOP/s")
                del X, ws, Y
    best = max(v["tflops"] for v in res.values())
    cpu = None if args.no_cpu_baseline else cpu_baseline_gemm(rabit, ((14336, 4096), (4096, 14336)))
    return _line("Residual-binary prefill GEMM TFLOP/s (4 M N K, fp16 MFMA)", best, "TFLOP/s",
                 {"workload": "llama3-8b-mlp-gemm", "M": [512, 2048, 8192]}, dtype="fp16",
                 runs=res, runs_3bit=res3, runs_weff=resw, cpu_baseline=cpu,
                 roofline={"bound": "mfma", "peak": 2500.0, "unit": "TFLOP/s",
                                     "achieved": best, "frac": round(best / 2500.0, 4)})


def bench_train(args, rabit, torch):
    """Training step of one layer (the coupled forward: derive with the current
    scales + GEMM; the backward: dX, and dW with dg, dh) on the Llama-2-7B
    layer shapes at M = 2048 and 8192 tokens, next to a dense bf16 layer's
    three matrix products (torch.mm: forward, dX, dW in bf16)."""
    import numpy as np
    from synth.inputs import act_bf16, grad_bf16, random_f16_scales, seed_w, seed_x, seed_dy, weight_f32
    res = {}
    best_gw = 0.0
    gw_launch = None
    for (N, K, name) in ((4096, 4096, "q"), (11008, 4096, "gate"), (4096, 11008, "down")):
        w = weight_f32(N, K, seed_w(6, 0, name), device="cuda")
        pl = rabit.PackedLayer.empty(N, K)
        g = torch.from_numpy(np.stack([random_f16_scales(N, 61), random_f16_scales(N, 62, 0.002, 0.01)]))
        h = torch.from_numpy(np.stack([random_f16_scales(K, 63), random_f16_scales(K, 64, 0.002, 0.01)]))
        pl.g.copy_(g.view(torch.int16))
        pl.h.copy_(h.view(torch.int16))
        wd = w.to(torch.bfloat16)
        for M in (2048, 8192):
            X = act_bf16(M, K, seed_x(6, M)).cuda()
            dY = grad_bf16(M, N, seed_dy(6, M)).cuda()
            Y = torch.empty(M, N, device="cuda", dtype=torch.bfloat16)
            dX = torch.empty(M, K, device="cuda", dtype=torch.bfloat16)
            dW = torch.empty(N, K, device="cuda")
            dg = torch.empty(2, N, device="cuda")
            dh = torch.empty(2, K, device="cuda")
            wsf = rabit.gemm_workspace(pl, M)
            wsx = rabit.grad_input_workspace(pl, M)
            wsw = rabit.grad_weight_workspace(pl)
            derive = lambda i: rabit.pack(w, pl, rabit.RABIT_SCALES_GIVEN)
            fwd = lambda i: rabit.gemm(pl, X, rabit.RABIT_OUT_BF16, y=Y, workspace=wsf)
            gx = lambda i: rabit.grad_input(pl, dY, rabit.RABIT_OUT_BF16, dx=dX, workspace=wsx)
            gw = lambda i: rabit.grad_weight(pl, X, dY, dw=dW, dg=dg, dh=dh, workspace=wsw)
            fwdw = lambda i: rabit.gemm(pl, X, rabit.RABIT_OUT_BF16, y=Y, workspace=wsf, weff=True)
            gxw = lambda i: rabit.grad_input(pl, dY, rabit.RABIT_OUT_BF16, dx=dX, workspace=wsx,
                                             weff=True)
            for f in (derive, fwd, gx, gw, fwdw, gxw):
                f(0)
            t = {k: _events_ms(torch, f, 5) for k, f in
                 (("derive", derive), ("forward", fwd), ("grad_input", gx), ("grad_weight", gw))}
            tw = {k: _events_ms(torch, f, 5) for k, f in (("forward", fwdw), ("grad_input", gxw))}
            dense = {
                "forward": _events_ms(torch, lambda i: torch.mm(X, wd.t()), 5),
                "grad_input": _events_ms(torch, lambda i: torch.mm(dY, wd), 5),
                "grad_weight": _events_ms(torch, lambda i: torch.mm(dY.t(), X), 5),
            }
            flop = 2.0 * M * N * K
            ours = sum(t.values())
            ours_w = t["derive"] + tw["forward"] + tw["grad_input"] + t["grad_weight"]
            dn = sum(dense.values())
            tf_gw = flop / (t["grad_weight"] * 1e-3) / 1e12
            if tf_gw > best_gw and M == 8192:
                best_gw = tf_gw
            if name == "gate" and M == 8192:
                gw_launch = t["grad_weight"]
            res[f"{N}x{K}_M{M}"] = {
                "ms": {k: round(v, 4) for k, v in t.items()}, "ms_step": round(ours, 4),
                "dense_bf16_ms": {k: round(v, 4) for k, v in dense.items()},
                "dense_bf16_ms_step": round(dn, 4),
                "grad_weight_tflops": round(tf_gw, 1),
                "step_tflops_dense_equiv": round(3 * flop / (ours * 1e-3) / 1e12, 1),
                "speedup_vs_dense": round(dn / ours, 3),
                "weff_ms": {k: round(v, 4) for k, v in tw.items()}, "weff_ms_step": round(ours_w, 4),
                "weff_speedup_vs_dense": round(dn / ours_w, 3)}
            log(f"train {N}x{K} M={M}: derive {t['derive']:.3f} fwd {t['forward']:.3f} "
                f"dX {t['grad_input']:.3f} dW {t['grad_weight']:.3f} ms (dW {tf_gw:.0f} TFLOP/s); "
                f"step {ours:.3f} ms vs dense bf16 {dn:.3f} ms; fp16 W_hat tiles: fwd {tw['forward']:.3f} "
                f"dX {tw['grad_input']:.3f} step {ours_w:.3f} ms")
            del X, dY, Y, dX, dW, wsf, wsx, wsw
        del w, wd, pl
    gate = res["11008x4096_M8192"]
    return _line("Coupled training step of one layer, dense-equivalent TFLOP/s (6 M N K), "
                 "Llama-2-7B gate shape at M = 8192", gate["step_tflops_dense_equiv"], "TFLOP/s",
                 {"workload": "llama2-7b-layer-train-step", "M": [2048, 8192]}, dtype="bf16",
                 runs=res, roofline={"bound": "mfma", "kernel": "k_grad_w<2>", "peak": 2500.0,
                                     "unit": "TFLOP/s", "achieved": round(best_gw, 1),
                                     "frac": round(best_gw / 2500.0, 4),
                                     "launch_ms_gate_M8192": round(gw_launch, 4)})


def bench_init(args, rabit, torch):
    """Initialisation of the scales: iterative residual SVID (20 sweeps, 5
    power passes per re-fit, two paths) on the Llama-2-7B layer shapes."""
    from synth.inputs import seed_w, weight_f32
    res = {}
    P, T, K = 2, 20, 5
    best = None
    for (N, K_in, name) in ((4096, 4096, "q"), (11008, 4096, "gate"), (4096, 11008, "down")):
        w = weight_f32(N, K_in, seed_w(7, 0, name), device="cuda")
        g = torch.zeros(P, N, device="cuda")
        h = torch.zeros(P, K_in, device="cuda")
        pl = torch.zeros(rabit.planes_bytes(N, K_in, P), dtype=torch.uint8, device="cuda")
        ws = rabit.svid_workspace(N, K_in)
        run = lambda i: rabit.svid_init(w, P, T, K, g=g, h=h, planes=pl, workspace=ws)
        run(0)
        ms = _events_ms(torch, run, 1, reps=2)
        passes = T * P * K
        # per pass: W (4 B) and the other path's bits (1/8 B) per weight
        alg = passes * N * K_in * (4 + (P - 1) / 8)
        gbs = alg / (ms * 1e-3) / 1e9
        res[f"{N}x{K_in}"] = {"ms": round(ms, 3), "passes": passes, "alg_gbs": round(gbs, 1),
                              "us_per_pass": round(1e3 * ms / passes, 2)}
        log(f"svid init {N}x{K_in}: {ms:.2f} ms for {passes} passes ({1e3 * ms / passes:.1f} us/pass), "
            f"{gbs:.0f} GB/s algorithmic")
        if name == "gate":
            best = gbs
        del w, g, h, pl, ws
    return _line("Iterative residual SVID initialisation, algorithmic GB/s (W read per power pass), "
                 "Llama-2-7B gate shape", round(best, 1), "GB/s",
                 {"workload": "llama2-7b-svid-init", "sweeps": T, "power_passes": K, "paths": P},
                 dtype="f32", runs=res,
                 roofline={"bound": "hbm", "kernel": "k_svid_pass", "peak": 8000.0, "unit": "GB/s",
                           "achieved": round(best, 1), "frac": round(best / 8000.0, 4)})


def _timed_decode(rabit, torch, cfg, arr, batch, steps, warmup, use_graph, xseed, dist=0):
    """ms per decode step at `batch`: `warmup` untimed steps, then exactly
    `steps` steps between two HIP events on the launch stream, bracketed by
    device synchronisations. Steps ping-pong between two activation buffers
    and are replayed from HIP graphs (checked bit-identical to eager steps)."""
    from synth.inputs import act_bf16
    x0 = act_bf16(batch, cfg.hidden, xseed).cuda()
    bufs = [x0.clone(), torch.empty_like(x0)]
    ws = rabit.decode_workspace(cfg, batch)

    def step(i):
        rabit.decode_step(cfg, arr, bufs[i % 2], out=bufs[(i + 1) % 2], workspace=ws)

    step(0)
    step(1)
    torch.cuda.synchronize()
    eager = bufs[0].clone()
    graphs = None
    if use_graph:
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            step(0)  # warm the capture path
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        graphs = []
        for par in (0, 1):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                step(par)
            graphs.append(g)
        torch.cuda.synchronize()
        bufs[0].copy_(x0)
        graphs[0].replay()
        graphs[1].replay()
        torch.cuda.synchronize()
        assert torch.equal(bufs[0], eager), "graph replay differs from the eager steps"

    def run(n, start=0):
        for k in range(start, start + n):
            if graphs is not None:
                graphs[k % 2].replay()
            else:
                step(k)
        return start + n

    bufs[0].copy_(x0)
    nxt = run(warmup)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    run(steps, nxt)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    if dist:
        # after the timed region: `dist` more steps, one event after each,
        # for the per-step distribution
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(dist + 1)]
        ev[0].record()
        k = nxt + steps
        for i in range(dist):
            k = run(1, k)
            ev[i + 1].record()
        torch.cuda.synchronize()
        per_step = [ev[i].elapsed_time(ev[i + 1]) for i in range(dist)]
        del graphs, ws
        return ms, per_step
    del graphs, ws
    return ms


def _stack_kinds(rabit, layers, H, F, batch):
    """The step's four GEMV launch shapes as callables on one layer: [q,k,v]
    and [gate,up] in one launch each (rabit_gemv_partial_multi), o and down
    (rabit_gemv_partial), with resident bf16 inputs."""
    from synth.inputs import act_bf16
    xh = act_bf16(batch, H, 11).cuda()
    xf = act_bf16(batch, F, 12).cuda()
    L0 = layers[0]
    ws_qkv = rabit.gemv_multi_workspace([L0["q"], L0["k"], L0["v"]], batch)
    ws_o = rabit.gemv_workspace(L0["o"], batch)
    ws_gu = rabit.gemv_multi_workspace([L0["gate"], L0["up"]], batch)
    ws_d = rabit.gemv_workspace(L0["down"], batch)
    return {
        "qkv": lambda L: rabit.gemv_partial_multi([L["q"], L["k"], L["v"]], xh, ws_qkv),
        "o": lambda L: rabit.gemv_partial(L["o"], xh, ws_o),
        "gate+up": lambda L: rabit.gemv_partial_multi([L["gate"], L["up"]], xh, ws_gu),
        "down": lambda L: rabit.gemv_partial(L["down"], xf, ws_d),
    }


def _linear_only(rabit, torch, layers, H, F, KV, batch, reps=3):
    """Time of the step's GEMV launches without the glue kernels: each launch
    shape over all layers (us per launch), and the whole sequence in step
    order (ms per step), graph-replayed back to back between HIP events."""
    kinds = _stack_kinds(rabit, layers, H, F, batch)
    per = {}
    for k, f in kinds.items():
        per[k] = graph_ms(torch, lambda: [f(L) for L in layers], reps) / len(layers)

    def seq():
        for L in layers:
            for f in kinds.values():
                f(L)
    step_ms = graph_ms(torch, seq, reps)
    alg = {"qkv": launch_alg_bytes([H, KV, KV], H, batch), "o": gemv_alg_bytes(H, H, batch),
           "gate+up": launch_alg_bytes([F, F], H, batch), "down": gemv_alg_bytes(H, F, batch)}
    return per, step_ms, alg


def cpu_baseline_70b(rabit, budget_s, frac=8):
    """The oracle (float64 numpy) on the host over a bounded sample of the
    Llama-2-70B step: for layers {0, 39, 79}, blocks of out/frac output rows
    of each of the seven matrices (given fp16 scales of the mean-|.|
    magnitude; the derivation is set-up and not timed), the oracle's GEMV
    (W_eff reconstruction in float64, then the product with x) at batch 1.
    Row blocks are added, all 21 matrices at a time, until the timed GEMVs
    reach budget_s seconds (or every row is done). Extrapolated to the whole
    step: x (rows / sampled rows) per matrix and x 80/3 over the layers."""
    import numpy as np
    import oracle
    from synth.inputs import act_bf16, bf16_values, random_f16_scales, weight_f32
    try:
        from threadpoolctl import threadpool_info
        blas = [(t.get("internal_api"), t.get("num_threads")) for t in threadpool_info()]
    except Exception:  # pragma: no cover
        blas = []
    c = L70
    H, F, KV = c["H"], c["F"], c["KV"]
    shapes = layer_shapes(H, F, KV)
    t_sample, w_sample, blocks = 0.0, 0, 0
    done = {}    # (layer, matrix) -> [seconds, rows]
    for blk in range(frac):
        for li in (0, 39, 79):
            for k, (name, (o, i)) in enumerate(shapes.items()):
                R = max(64, o // frac)
                rows = min(R, o - blk * R)
                if rows <= 0:
                    continue
                w = weight_f32(rows, i, 5000 + 10 * li + k + 1000 * blk).numpy()
                g1, g2 = random_f16_scales(rows, 1, 0.010, 0.022), random_f16_scales(rows, 2, 0.008, 0.018)
                h1, h2 = random_f16_scales(i, 3, 0.010, 0.022), random_f16_scales(i, 4, 0.008, 0.018)
                d = oracle.derive(w, mode="given", g1=g1, h1=h1, g2=g2, h2=h2)
                d.r = None
                del w
                x = bf16_values(act_bf16(1, i, 7 + k))
                t0 = time.perf_counter()
                oracle.gemv(d, x)
                dt = time.perf_counter() - t0
                t_sample += dt
                w_sample += rows * i
                s = done.setdefault((li, name), [0.0, 0])
                s[0] += dt
                s[1] += rows
                del d
        blocks += 1
        if t_sample >= budget_s:
            break
    t_step = sum(s[0] * shapes[name][0] / s[1] for (li, name), s in done.items()) * c["L"] / 3.0
    plane_bytes = sum(rabit.planes_bytes(o, i) for o, i in shapes.values()) * c["L"]
    return {
        "value": round(plane_bytes / t_step / 1e9, 5),
        "unit": "GB/s",
        "cores": len(os.sched_getaffinity(0)),
        "kind": "oracle",
        "sample": (f"layers 0, 39, 79 of the Llama-2-70B stack, first {blocks}/{frac} of the output rows of each of "
                   f"q, k, v, o, gate, up, down ({w_sample / 1e6:.0f} M weights, {t_sample:.1f} s): oracle "
                   "float64 W_eff reconstruction + product with x at batch 1; extrapolated x rows/sample "
                   "per matrix and x 80/3 over the layers; GB/s of packed-plane bytes per step"),
        "tokens_per_s": round(1.0 / t_step, 6),
        "s_per_step_extrapolated": round(t_step, 1),
        "blas_threads": blas,
    }


def bench_llama70b(args, rabit, torch):
    """Llama-2-70B-shaped stack: derive+pack all layers, then decode at batch
    1 (timed steps, the headline) and 32."""
    from synth.inputs import seed_x
    c = L70
    H, F, KV = c["H"], c["F"], c["KV"]
    L = args.layers or c["L"]
    t0 = time.time()
    log(f"packing {L} Llama-2-70B layers ...")
    layers, planes, pack = _decoder_layers(rabit, torch, 5, H, F, KV, L)
    torch.cuda.synchronize()
    log(f"packed {L} layers ({planes / 1e9:.2f} GB of planes) in {time.time() - t0:.1f} s")
    weights = sum(w for w, _ in pack)
    pack_ms = sum(ms for _, ms in pack)
    # the same work timed on the GPU alone: each matrix shape's pack
    # graph-replayed, times its count in the stack
    from synth.inputs import seed_w
    counts = {(H, H): 2, (KV, H): 2, (F, H): 2, (H, F): 1}
    names = {(H, H): "q", (KV, H): "k", (F, H): "gate", (H, F): "down"}
    pack_gpu = {sh: pack_graph_ms(rabit, torch, sh[0], sh[1], seed_w(5, 0, names[sh])) for sh in counts}
    pack_gpu_ms = L * sum(pack_gpu[sh] * n for sh, n in counts.items())
    log(f"derive/pack: {pack_ms:.1f} ms event-timed per call, {pack_gpu_ms:.1f} ms graph-replayed")
    cfg = rabit.DecoderCfg(hidden=H, ffn=F, n_heads=c["n_heads"], n_kv_heads=c["n_kv_heads"],
                           head_dim=c["head_dim"], n_layers=L)
    arr = rabit.layer_array(cfg, layers)
    use_graph = not args.no_graph

    ms1, steps1 = _timed_decode(rabit, torch, cfg, arr, 1, args.steps, args.warmup, use_graph, seed_x(5, 1),
                                dist=20)
    step_dist = {k: (round(v, 4) if k != "n" else v) for k, v in dist_summary(steps1).items()}
    gbs1 = planes / (ms1 * 1e-3) / 1e9
    log(f"batch 1: {args.steps} steps, {ms1:.3f} ms/step, {1e3 / ms1:.1f} tokens/s, {gbs1:.1f} GB/s of planes")
    steps32 = max(2, args.steps // 5)
    ms32 = _timed_decode(rabit, torch, cfg, arr, 32, steps32, 1, use_graph, seed_x(5, 32))
    log(f"batch 32: {steps32} steps, {ms32:.3f} ms/step, {32e3 / ms32:.1f} tokens/s")

    lin = {}
    for b in (1, 32):
        per, step_ms, alg = _linear_only(rabit, torch, layers, H, F, KV, b, reps=3 if b == 1 else 1)
        lin[b] = (per, step_ms, alg)
        log(f"linear only, batch {b}: {step_ms:.3f} ms/step; per launch (us): "
            + ", ".join(f"{k} {v * 1e3:.2f}" for k, v in per.items()))
    kinds1 = _stack_kinds(rabit, layers, H, F, 1)
    launch_dist = {}
    for k, f in kinds1.items():
        d = dist_summary([t / L for t in graph_ms_dist(torch, lambda: [f(Lr) for Lr in layers], 20)])
        launch_dist[k] = {q: (round(v * 1e3, 3) if q != "n" else v) for q, v in d.items()}
    log(f"per-launch distribution over 20 replays (us): {launch_dist}")
    per1, lin_ms1, alg1 = lin[1]
    per32, lin_ms32, _ = lin[32]
    tot_alg = sum(alg1.values())
    tot_ms = sum(per1.values())
    achieved = tot_alg / (tot_ms * 1e-3) / 1e9
    traffic = committed_traffic()

    # practical ceilings: plain read-only streams of each launch shape's plane bytes
    pb = {"qkv": rabit.planes_bytes(H, H) + 2 * rabit.planes_bytes(KV, H), "o": rabit.planes_bytes(H, H),
          "gate+up": 2 * rabit.planes_bytes(F, H), "down": rabit.planes_bytes(H, F)}
    st = {k: stream_read_ms(rabit, torch, v) for k, v in pb.items()}
    stream = {
        "read_only_us": {k: round(v * 1e3, 2) for k, v in st.items()},
        "read_only_gbs": {k: round(pb[k] / (v * 1e-3) / 1e9, 1) for k, v in st.items()},
        "read_only_step_ms": round(L * sum(st.values()), 4),
        "gemv_launch_over_read_only": {k: round(per1[k] / st[k], 3) for k in st},
        "note": "rabit_stream_read (16-byte loads) over cold rotating buffers of the same plane bytes as "
                "each launch shape, graph-replayed back to back",
    }
    log(f"streaming ceiling: {stream}")

    cpu = None
    if not args.no_cpu_baseline:
        log("timing the CPU oracle baseline ...")
        cpu = cpu_baseline_70b(rabit, args.cpu_budget_s)
        log(f"cpu oracle: {cpu}")

    # plain device copy of a known size: the counter summaries use it to
    # calibrate FETCH_SIZE / WRITE_SIZE
    cal_a = torch.empty(256 << 20, dtype=torch.uint8, device="cuda").fill_(1)
    cal_b = torch.empty_like(cal_a)
    cal_b.copy_(cal_a)
    torch.cuda.synchronize()
    del cal_a, cal_b

    return {
        "metric": "W2 residual-binary GEMV packed-weight GB/s (% HBM peak) + decode tokens/s",
        "value": round(gbs1, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms1, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp4xfp6",
        "data": "synthetic",
        "config": {"workload": "llama2-70b-stack-decode-b1", "layers": L, "hidden": H, "ffn": F,
                   "n_heads": c["n_heads"], "n_kv_heads": c["n_kv_heads"], "head_dim": c["head_dim"],
                   "batch": 1, "graph_replay": use_graph, "plane_bytes_per_step": planes},
        "pct_hbm_peak": round(100.0 * gbs1 / HBM_PEAK_GBS, 2),
        "decode_tokens_per_s": round(1e3 / ms1, 2),
        "step_ms_dist": step_dist,
        "batch32": {"ms_per_step": round(ms32, 4), "tokens_per_s": round(32e3 / ms32, 1),
                    "plane_gbs": round(planes / (ms32 * 1e-3) / 1e9, 1), "steps": steps32},
        "linear_only": {
            "b1": {"ms_per_step": round(lin_ms1, 4), "tokens_per_s": round(1e3 / lin_ms1, 2),
                   "plane_gbs": round(planes / (lin_ms1 * 1e-3) / 1e9, 1),
                   "pct_hbm_peak": round(100.0 * planes / (lin_ms1 * 1e-3) / 1e9 / HBM_PEAK_GBS, 2),
                   "launch_us": {k: round(v * 1e3, 3) for k, v in per1.items()},
                   "launch_us_dist": launch_dist},
            "b32": {"ms_per_step": round(lin_ms32, 4), "tokens_per_s": round(32e3 / lin_ms32, 1),
                    "plane_gbs": round(planes / (lin_ms32 * 1e-3) / 1e9, 1),
                    "launch_us": {k: round(v * 1e3, 3) for k, v in per32.items()}},
            "note": "the step's GEMV launches alone ([q,k,v], o, [gate,up], down per layer; resident bf16 "
                    "inputs, no RMSNorm prologue), graph-replayed back to back; the range sums run in the "
                    "glue kernels and are not included",
        },
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": None if traffic is None else int(traffic),
                     "kernel": "k_gemv", "avg_launch_us": round(tot_ms * 1e3 / 4, 3),
                     "alg_bytes_per_launch": int(tot_alg / 4),
                     "launch_us": {k: round(v * 1e3, 3) for k, v in per1.items()},
                     "alg_bytes": alg1},
        "stream_ceiling": stream,
        "derive_pack": {"weights": weights, "ms": round(pack_gpu_ms, 2), "alg_bytes_per_weight": 8.25,
                        "gbs": round(8.25 * weights / (pack_gpu_ms * 1e-3) / 1e9, 1),
                        "frac_hbm": round(8.25 * weights / (pack_gpu_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                        "per_call_ms": {f"{o}x{i}": round(v, 4) for (o, i), v in pack_gpu.items()},
                        "event_timed_ms": round(pack_ms, 2),
                        "note": "rabit_pack MEANABS, GPU time: each matrix shape's call graph-replayed, times its "
                                "count in the stack; event_timed_ms: the packing of the stack itself, an event pair "
                                "around each Python call (includes the host-side call overhead)"},
        "cpu_baseline": cpu,
    }


if __name__ == "__main__":
    main()
