#!/usr/bin/env python3
"""Benchmark of the RaBiT 2-path residual-binary hot path on one MI355X.

Metric: W2 residual-binary GEMV packed-weight GB/s (% HBM peak) + decode
tokens/s, on the Llama-2-7B-shaped MLP block at batch 1 (gate and up
11008x4096, down 4096x11008, SiLU gating). Weights are random-init
W ~ 0.02 N(0,1) packed by rabit_pack (mean-|.| scales); activations are bf16
N(0,1).

A step is one decode call, rabit_decode_step, through --layers consecutive MLP
blocks with distinct weights (default 32, the depth of Llama-2-7B: 1.08 GB of
planes per step, far above the 256 MB last-level cache, so every block streams
its planes from HBM). Per block the library runs: the gate+up GEMV as one
launch on RMSNorm(x), SiLU(gate)*up, the down GEMV, and x + down with its x^2
statistics. Steps are replayed from a HIP graph.

value = plane bytes per step / step time. The roofline object describes the
dominant kernel, k_gemv<1> (the plane-streaming GEMV): the bench times its two
launch shapes of the step (gate+up, down) back to back with HIP events on the
launch stream, over all layers, and divides algorithmic bytes by the average
launch duration. traffic comes from the committed rocprofv3 counter summary
when it was taken on the current GEMV source, else null.

Printed: one JSON line (stdout). Diagnostics go to stderr.
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
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "k_gemv_llama2_7b_mlp_b1_traffic.txt")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def mlp_shapes(hidden=4096, ffn=11008):
    return {"gate": (ffn, hidden), "up": (ffn, hidden), "down": (hidden, ffn)}


def gemv_alg_bytes(out, inp, b=1):
    """Algorithmic bytes of one GEMV: planes (0.25 B/weight), fp16 g and h of
    both paths, bf16 x, fp32 y."""
    return out * inp // 4 + 4 * (out + inp) + 2 * b * inp + 4 * b * out


def gemv_source_sha():
    with open(GEMV_SRC, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def committed_traffic():
    """HBM bytes per k_gemv<1> launch from the committed counter summary, or
    None when it is missing or was taken on another GEMV source."""
    try:
        kv = {}
        with open(TRAFFIC_FILE) as f:
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


def time_gemv_launches(rabit, torch, layers, hidden, ffn, reps=5):
    """Average duration of the step's two k_gemv<1> launch shapes, each timed
    as `len(layers)` back-to-back launches (one per layer, cold planes) between
    two events on the launch stream; median over `reps`."""
    stream = torch.cuda.current_stream()
    x_h = torch.randn(1, hidden, device="cuda").to(torch.bfloat16)
    x_f = torch.randn(1, ffn, device="cuda").to(torch.bfloat16)
    ws_gu = rabit.gemv_multi_workspace([layers[0]["gate"], layers[0]["up"]], 1)
    ws_d = rabit.gemv_workspace(layers[0]["down"], 1)
    res = {"gate+up": [], "down": []}
    for r in range(reps + 1):
        for kind in ("gate+up", "down"):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            for L in layers:
                if kind == "gate+up":
                    rabit.gemv_partial_multi([L["gate"], L["up"]], x_h, ws_gu)
                else:
                    rabit.gemv_partial(L["down"], x_f, ws_d)
            b.record(stream)
            b.synchronize()
            if r > 0:  # the first pass warms up
                res[kind].append(a.elapsed_time(b) / len(layers))
    med = {k: sorted(v)[len(v) // 2] for k, v in res.items()}
    return med, res


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=40)
    ap.add_argument("--warmup", type=int, default=4)
    ap.add_argument("--layers", type=int, default=32)
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
    traffic = committed_traffic()

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
        "derive_pack": derive,
        "cpu_baseline": cpu,
    }
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
