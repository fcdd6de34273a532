#!/usr/bin/env python3
"""Benchmark of the RaBiT 2-path residual-binary hot path on one MI355X.

Metric: W2 residual-binary GEMV packed-weight GB/s (% HBM peak) + decode
tokens/s. Default workload: a Llama-2-7B-shaped MLP block at batch 1 (gate
and up 11008x4096, down 4096x11008, SiLU gating), random-init weights
W ~ 0.02 N(0,1) packed by rabit_pack, activations bf16 N(0,1).

A step = one token through the MLP block (RMSNorm, gate/up GEMV, SiLU*up,
down GEMV, residual) via rabit_decode_step. Steps rotate over --copies
distinct packed copies of the block (32 = the depth of Llama-2-7B, 1.08 GB
of planes) so that every step streams its weights from HBM, not from the
256 MB last-level cache. The steps are replayed from HIP graphs.

Printed: one JSON line (stdout). Diagnostics go to stderr.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X published HBM3E bandwidth


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def mlp_shapes(hidden=4096, ffn=11008):
    return {"gate": (ffn, hidden), "up": (ffn, hidden), "down": (hidden, ffn)}


def gemv_alg_bytes(out, inp, b=1):
    """Algorithmic bytes of one GEMV: planes (0.25 B/weight), fp16 g and h of
    both paths, bf16 x, fp32 y."""
    return out * inp // 4 + 4 * (out + inp) + 2 * b * inp + 4 * b * out


def build_copies(rabit, torch, copies, shapes, cfg_id=2, time_pack=True):
    """Generate and pack `copies` distinct copies of the matrices in `shapes`."""
    from synth.inputs import weight_f32, seed_w
    layers = []
    pack_ms = []
    ws = None
    for c in range(copies):
        d = {}
        for name, (o, i) in shapes.items():
            w = weight_f32(o, i, seed_w(cfg_id, c, name), device="cuda")
            pl = rabit.PackedLayer.empty(o, i)
            if ws is None or ws.numel() < rabit.load().rabit_pack_workspace_bytes(o, i):
                ws = torch.empty(rabit.load().rabit_pack_workspace_bytes(o, i), dtype=torch.uint8,
                                 device="cuda")
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            rabit.pack(w, pl, workspace=ws)
            e1.record()
            e1.synchronize()
            if time_pack:
                pack_ms.append((name, o, i, e0.elapsed_time(e1)))
            del w
            d[name] = pl
        layers.append(d)
    return layers, pack_ms


def cpu_baseline_mlp(shapes, budget_s):
    """The oracle (float64 numpy) on the host: derive one copy of the block,
    then time its GEMV path (W_eff reconstruction + matmul) for the three
    matrices, repeated until about `budget_s` seconds of work."""
    import numpy as np
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
        "ms_per_step": round(1e3 * t_gemv / reps, 3),
        "derive_pack_s": round(t_derive, 3),
        "derive_pack_gbs_w_read": round(8 * weights / t_derive / 1e9, 4),
    }


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=640)
    ap.add_argument("--warmup", type=int, default=64)
    ap.add_argument("--copies", type=int, default=32)
    ap.add_argument("--cpu-budget-s", type=float, default=8.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-graph", action="store_true", help="launch eagerly instead of graph replay")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: this build measures one GPU only; the multi-GPU split is a design "
              "(DESIGN.md, 'Sharding'), run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch
    from bit_residual_binarized_amd import rabit
    from synth.inputs import act_bf16, seed_x

    rabit.load()
    torch.cuda.set_device(0)
    hidden, ffn = 4096, 11008
    shapes = mlp_shapes(hidden, ffn)
    cfg = rabit.DecoderCfg(hidden=hidden, ffn=ffn, n_layers=1, mlp_only=True)

    t0 = time.time()
    log(f"packing {args.copies} copies of the MLP block ...")
    layers, pack_ms = build_copies(rabit, torch, args.copies, shapes)
    torch.cuda.synchronize()
    log(f"packed in {time.time() - t0:.1f} s")
    plane_bytes_step = sum(rabit.planes_bytes(o, i) for o, i in shapes.values())

    arrays = [rabit.layer_array(cfg, [L]) for L in layers]
    x0 = act_bf16(1, hidden, seed_x(2, 1)).cuda()
    bufs = [x0.clone(), torch.empty_like(x0)]
    ws = rabit.decode_workspace(cfg, 1)

    def step(i):
        src, dst = bufs[i % 2], bufs[(i + 1) % 2]
        rabit.decode_step(cfg, arrays[i % args.copies], src, out=dst, workspace=ws)

    # eager reference of one pass over the copies, then graphs
    bufs[0].copy_(x0)
    for i in range(args.copies):
        step(i)
    torch.cuda.synchronize()
    eager_out = bufs[args.copies % 2].clone()

    graphs_one, graph_all = [], None
    if not args.no_graph:
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            for i in range(args.copies):  # warm the capture path
                step(i)
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        graph_all = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph_all):
            for i in range(args.copies):
                step(i)
        for i in range(args.copies):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                step(i)
            graphs_one.append(g)
        torch.cuda.synchronize()
        # graph replay must reproduce the eager pass
        bufs[0].copy_(x0)
        graph_all.replay()
        torch.cuda.synchronize()
        assert torch.equal(bufs[args.copies % 2], eager_out), "graph replay differs from eager run"

    def run_steps(n, start=0):
        i = start
        if graph_all is not None:
            while n > 0:
                if i % args.copies == 0 and n >= args.copies:
                    graph_all.replay()
                    i += args.copies
                    n -= args.copies
                else:
                    graphs_one[i % args.copies].replay()
                    i += 1
                    n -= 1
        else:
            for k in range(n):
                step(start + k)
        return i

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
    log(f"{args.steps} steps in {total_ms:.3f} ms: {ms_step * 1e3:.2f} us/step, {gbs:.1f} GB/s of planes")

    # dominant kernel: the plane-streaming GEMV kernel (rabit_gemv_partial is
    # exactly one launch of it); time each launch with events on the stream it
    # is launched on (eager, same rotation over the copies as the steps)
    gws = {n: rabit.gemv_workspace(layers[0][n], 1) for n in shapes}
    xin = {"gate": torch.empty(1, hidden, dtype=torch.bfloat16, device="cuda"),
           "down": torch.empty(1, ffn, dtype=torch.bfloat16, device="cuda")}
    xin["gate"].normal_()
    xin["down"].normal_()
    xin["up"] = xin["gate"]
    yout = {n: torch.empty(1, o, device="cuda") for n, (o, i) in shapes.items()}
    stream = torch.cuda.current_stream()
    durs = []
    reps = max(1, 96 // args.copies)
    for r in range(reps + 1):
        for c in range(args.copies):
            for n in ("gate", "up", "down"):
                a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                a.record(stream)
                rabit.gemv_partial(layers[c][n], xin[n], gws[n])
                b.record(stream)
                rabit.gemv_reduce(layers[c][n], 1, yout[n], gws[n])
                if r > 0:
                    durs.append((a, b))
    torch.cuda.synchronize()
    kms = [a.elapsed_time(b) for a, b in durs]
    kavg_ms = sum(kms) / len(kms)
    alg_bytes = sum(gemv_alg_bytes(o, i) for o, i in shapes.values()) / 3.0
    achieved = alg_bytes / (kavg_ms * 1e-3) / 1e9
    log(f"gemv kernel (k_gemv<1>): avg {kavg_ms * 1e3:.2f} us over {len(kms)} launches -> {achieved:.1f} GB/s")

    pk = [p for p in pack_ms[3:]] or pack_ms
    pk_ms = sum(p[3] for p in pk) / len(pk)
    pk_weights = sum(p[1] * p[2] for p in pk) / len(pk)
    derive = {
        "ms_per_matrix": round(pk_ms, 4),
        "alg_bytes_per_weight": 8.25,
        "gbs": round(8.25 * pk_weights / (pk_ms * 1e-3) / 1e9, 1),
        "frac_hbm": round(8.25 * pk_weights / (pk_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        "note": "rabit_pack MEANABS: 2 reads of W fp32 + planes, 4 kernels; event-timed",
    }

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
                   "batch": 1, "weight_copies": args.copies, "graph_replay": graph_all is not None,
                   "plane_bytes_per_step": plane_bytes_step},
        "pct_hbm_peak": round(100.0 * gbs / HBM_PEAK_GBS, 2),
        "decode_tokens_per_s": round(1e3 / ms_step, 1),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None,
                     "kernel": "k_gemv<1>", "avg_launch_us": round(kavg_ms * 1e3, 3),
                     "alg_bytes_per_launch": int(alg_bytes)},
        "derive_pack": derive,
        "cpu_baseline": cpu,
    }
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
