"""Summaries of rocprofv3 output (CSV) for the decode GEMV's launch shapes.

usage:
  python -m bit_residual_binarized_amd.profsum stats TRACE_DIR
      per (kernel, grid size): dispatch count and the median, mean and
      minimum of rocprof's per-dispatch durations (us), from the kernel trace
      of `rocprofv3 --kernel-trace --output-format csv`.
  python -m bit_residual_binarized_amd.profsum traffic FETCH_DIR WRITE_DIR
      HBM bytes per k_gemv launch of the Llama-2-70B batch-1 step's four
      launch shapes, from one `--pmc FETCH_SIZE` and one `--pmc WRITE_SIZE`
      pass over `bench.py` (counter_collection CSV). Each counter (KiB per
      dispatch) is divided by the factor the same counter reads on the plain
      256 MiB device copy that bench.py runs in the same process (the
      runtime's copy kernel), so that the result is bytes.
  python -m bit_residual_binarized_amd.profsum counters PMC_DIR
      per launch shape of the 70B batch-1 step (the four plain-input launches
      and the two that form their inputs), instruction counts per wave
      (device sums / SQ_WAVES) and SQ_WAIT_ANY / SQ_WAVE_CYCLES, from one
      `--pmc SQ_WAVES SQ_WAVE_CYCLES SQ_BUSY_CYCLES SQ_INSTS_VALU
      SQ_INSTS_MFMA SQ_INSTS_SALU SQ_INSTS_LDS SQ_WAIT_ANY` pass.
  python -m bit_residual_binarized_amd.profsum derive FETCH_DIR WRITE_DIR
      HBM bytes per launch of the derive/pack kernels (k_derive_tile passes,
      k_finalize) per matrix shape, copy-calibrated as for the GEMV, against
      the passes' algorithmic bytes (W read once per pass, 4 B per weight;
      the sign pass also writes the planes, 0.25 B per weight).

The output starts with `key: value` lines (the traffic form is what bench.py
reads back from the committed summary).
"""
from __future__ import annotations

import csv
import glob
import hashlib
import os
import re
import statistics
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
GEMV_SRC = os.path.join(ROOT, "bit_residual_binarized_amd", "csrc", "gemv.hip")
COPY_BYTES = 256 << 20  # the calibration copy in bench.py
CAL_KERNEL = "__amd_rocclr_copyBuffer"

# Llama-2-70B batch-1 launch shapes of the linear-only timing: (kernel
# template arguments, grid threads) -> label. The plan gives [q,k,v] and o one
# row group per wave (no weight ring), [gate,up] seven and down four (ring).
SHAPES_70B_B1 = {
    ("k_gemv<1, false, false, 2, 0>", 640 * 256): "qkv",
    ("k_gemv<1, false, false, 2, 0>", 512 * 256): "o",
    ("k_gemv<1, true, false, 2, 0>", 512 * 256): "gate+up",
    ("k_gemv<1, true, false, 2, 0>", 448 * 256): "down",
}


# the launches of the decode step that form their inputs from the previous
# launch's partials (attention output for o, SiLU(gate) * up for down)
SHAPES_70B_B1_FORMED = {
    ("k_gemv<1, false, false, 2, 1>", 512 * 256): "o, attention input formed",
    ("k_gemv<1, true, false, 2, 2>", 448 * 256): "down, SiLU input formed",
}
LABELS = {"qkv": "[q,k,v] 10240x8192", "o": "o 8192x8192", "gate+up": "[gate,up] 57344x8192",
          "down": "down 8192x28672"}


def gemv_sha() -> str:
    with open(GEMV_SRC, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def _rows(d: str, suffix: str) -> list[dict]:
    files = sorted(glob.glob(os.path.join(d, "**", f"*{suffix}"), recursive=True))
    if not files:
        raise SystemExit(f"no *{suffix} under {d}")
    rows = []
    for fn in files:
        with open(fn, newline="") as f:
            rows.extend(csv.DictReader(f))
    return rows


def _short(name: str) -> str:
    # "void rabit::(anonymous namespace)::k_gemv<1, true, false, 2, 0>(rabit::...)" -> "k_gemv<1, true, false, 2, 0>"
    m = re.search(r"(\w+)(<[^()]*>)?\(", name)
    if not m:
        return name.strip()
    return m.group(1) + (m.group(2) or "")


def _grid(r: dict) -> int:
    for k in ("Grid_Size", "Grid_Size_X", "grid_size"):
        if k in r and r[k]:
            return int(float(r[k]))
    return 0


# weights per matrix of the Llama-2-70B layer -> the matrices of that size
MATS_70B = {1024 * 8192: "k, v (1024x8192)", 8192 * 8192: "q, o (8192x8192)",
            28672 * 8192: "gate, up, down (28672x8192, 8192x28672)"}


def stats(trace_dir: str) -> None:
    rows = _rows(trace_dir, "kernel_trace.csv")
    groups: dict[tuple[str, int], list] = {}
    for r in rows:
        key = (_short(r["Kernel_Name"]), _grid(r))
        dur = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
        g = groups.setdefault(key, [[], r.get("VGPR_Count", ""), r.get("Accum_VGPR_Count", ""),
                                    r.get("Group_Segment_Size", r.get("LDS_Block_Size", ""))])
        g[0].append(dur)
    print(f"gemv_source_sha256: {gemv_sha()}")
    print(f"{'calls':>6} {'grid_threads':>13} {'median_us':>10} {'mean_us':>9} {'min_us':>8} "
          f"{'vgpr':>5} {'agpr':>4} {'lds':>6}  kernel  (launch)")
    for (k, grid), (d, vg, ag, lds) in sorted(groups.items(), key=lambda kv: -sum(kv[1][0])):
        lab = SHAPES_70B_B1.get((k, grid), "")
        print(f"{len(d):6d} {grid:13d} {statistics.median(d):10.2f} {statistics.fmean(d):9.2f} "
              f"{min(d):8.2f} {vg:>5} {ag:>4} {lds:>6}  {k}" + (f"  [{lab}] b1" if lab else ""))
    per = {}
    for (k, grid), (d, *_rest) in groups.items():
        lab = SHAPES_70B_B1.get((k, grid))
        if lab:
            per[lab] = statistics.median(d)
    if len(per) == 4:
        print("k_gemv_b1_median_us: " + ", ".join(f"{lab} {per[lab]:.2f}" for lab in ("qkv", "o", "gate+up", "down")))
        print(f"k_gemv_b1_mean_of_shapes_us: {statistics.fmean(per.values()):.2f}")


def _counter(d: str, counter: str) -> tuple[dict, float]:
    rows = [r for r in _rows(d, "counter_collection.csv") if r["Counter_Name"] == counter]
    cal = [float(r["Counter_Value"]) for r in rows if CAL_KERNEL in r["Kernel_Name"]]
    if not cal:
        raise SystemExit(f"{counter}: no {CAL_KERNEL} dispatch in {d}")
    # the calibration copy is the largest copy dispatch of the run
    factor = max(cal) / (COPY_BYTES / 1024)
    per: dict[str, list] = {}
    for r in rows:
        lab = SHAPES_70B_B1.get((_short(r["Kernel_Name"]), _grid(r)))
        if lab:
            per.setdefault(lab, []).append(float(r["Counter_Value"]) / factor)
    return per, factor


def traffic(fetch_dir: str, write_dir: str) -> None:
    sys.path.insert(0, ROOT)
    import bench  # algorithmic bytes of each launch shape, as bench.py counts them

    c = bench.L70
    H, F, KV = c["H"], c["F"], c["KV"]
    alg = {"qkv": bench.launch_alg_bytes([H, KV, KV], H), "o": bench.gemv_alg_bytes(H, H),
           "gate+up": bench.launch_alg_bytes([F, F], H), "down": bench.gemv_alg_bytes(H, F)}
    fetch, ff = _counter(fetch_dir, "FETCH_SIZE")
    write, wf = _counter(write_dir, "WRITE_SIZE")
    print(f"gemv_source_sha256: {gemv_sha()}")
    print(f"calibration_kernel: {CAL_KERNEL}")
    print(f"fetch_factor: {ff:.4f}")
    print(f"write_factor: {wf:.4f}")
    tot_t = tot_a = 0.0
    for lab in ("qkv", "o", "gate+up", "down"):
        if lab not in fetch or lab not in write:
            raise SystemExit(f"launch shape {lab} missing from the counter runs")
        fk = statistics.fmean(fetch[lab])
        wk = statistics.fmean(write[lab])
        t = (fk + wk) * 1024
        tot_t += t
        tot_a += alg[lab]
        print(f"{lab}_launches: {len(fetch[lab])}")
        print(f"{lab}_fetch_kib: {fk:.1f}")
        print(f"{lab}_write_kib: {wk:.1f}")
        print(f"{lab}_traffic_bytes: {t:.0f}")
        print(f"{lab}_algorithmic_bytes: {alg[lab]}")
        print(f"{lab}_fetch_over_algorithmic: {fk * 1024 / alg[lab]:.4f}")
    print(f"traffic_bytes_per_launch: {tot_t / 4:.0f}")
    print(f"algorithmic_bytes_per_launch: {tot_a / 4:.0f}")
    print(f"traffic_over_algorithmic: {tot_t / tot_a:.4f}")


def _calibrated(d: str, counter: str) -> tuple[list, float]:
    rows = [r for r in _rows(d, "counter_collection.csv") if r["Counter_Name"] == counter]
    cal = [float(r["Counter_Value"]) for r in rows if CAL_KERNEL in r["Kernel_Name"]]
    if not cal:
        raise SystemExit(f"{counter}: no {CAL_KERNEL} dispatch in {d}")
    return rows, max(cal) / (COPY_BYTES / 1024)


def derive(fetch_dir: str, write_dir: str) -> None:
    # k_derive_tile: a 256-thread workgroup per 64-row x 256-column tile, so
    # that its grid (the total thread count rocprof records) is out in / 64
    # and gives the matrix's weights. k_finalize (one launch per path) follows
    # each pass and is attributed to the matrix of the pass before it in
    # dispatch order.
    per: dict[tuple, dict] = {}
    for counter, d in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        rows, factor = _calibrated(d, counter)
        print(f"{counter.lower()}_factor: {factor:.4f}")
        key_of_last = None
        for r in sorted(rows, key=lambda r: int(r.get("Dispatch_Id") or r.get("Correlation_Id") or 0)):
            k = _short(r["Kernel_Name"])
            if k.startswith("k_derive_tile"):
                key_of_last = 64 * _grid(r)
                key = (k, key_of_last)
            elif k == "k_finalize" and key_of_last:
                key = (k, key_of_last)
            else:
                continue
            per.setdefault(key, {}).setdefault(counter, []).append(float(r["Counter_Value"]) * 1024 / factor)
    print(f"{'kernel':>26} {'weights':>10} {'launches':>8} {'read_MB':>9} {'write_MB':>9} "
          f"{'alg_MB':>8} {'read/alg':>8}  matrices")
    for (k, w), v in sorted(per.items(), key=lambda kv: (kv[0][1], kv[0][0])):
        rd = statistics.fmean(v.get("FETCH_SIZE", [0.0]))
        wr = statistics.fmean(v.get("WRITE_SIZE", [0.0]))
        alg = 4 * w if k.startswith("k_derive_tile") else 0
        alg_w = w // 4 if k.startswith("k_derive_tile<1") or k.startswith("k_derive_tile<2") else 0
        ratio = f"{rd / alg:8.3f}" if alg else f"{'-':>8}"
        print(f"{k:>26} {w:10d} {len(v.get('FETCH_SIZE', [])):8d} {rd / 1e6:9.2f} "
              f"{wr / 1e6:9.2f} {(alg + alg_w) / 1e6:8.2f} {ratio}  {MATS_70B.get(w, '')}")


def counters(pmc_dir: str) -> None:
    rows = _rows(pmc_dir, "counter_collection.csv")
    shapes = {**{k: LABELS[v] for k, v in SHAPES_70B_B1.items()}, **SHAPES_70B_B1_FORMED}
    # per dispatch: counter -> value (a dispatch is one Dispatch_Id)
    disp: dict[tuple, dict] = {}
    for r in rows:
        key = (_short(r["Kernel_Name"]), _grid(r))
        if key not in shapes:
            continue
        d = disp.setdefault((key, r.get("Dispatch_Id", r.get("Correlation_Id"))), {})
        d[r["Counter_Name"]] = d.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    print(f"gemv_source_sha256: {gemv_sha()}")
    order = list(shapes)
    for key in order:
        ds = [v for (k, _), v in disp.items() if k == key]
        if not ds:
            continue
        tot = {c: sum(d.get(c, 0.0) for d in ds) for c in ds[0]}
        waves = tot["SQ_WAVES"] / len(ds)
        per = {c: tot[c] / tot["SQ_WAVES"] for c in tot}
        kern, grid = key
        ring, xm = kern.split(", ")[1], kern.split(", ")[4].rstrip(">")
        print(f"\n{shapes[key]} (ring {ring}, XM {xm}, grid {grid}), launches {len(ds)}")
        print(f"  waves {waves:.0f}; per wave: VALU {per['SQ_INSTS_VALU']:.0f} (matrix {per['SQ_INSTS_MFMA']:.0f}), "
              f"SALU {per['SQ_INSTS_SALU']:.0f}, LDS {per['SQ_INSTS_LDS']:.0f}")
        print(f"  wait_fraction = SQ_WAIT_ANY / SQ_WAVE_CYCLES: {tot['SQ_WAIT_ANY'] / tot['SQ_WAVE_CYCLES']:.3f}")


if __name__ == "__main__":
    if len(sys.argv) == 3 and sys.argv[1] == "stats":
        stats(sys.argv[2])
    elif len(sys.argv) == 3 and sys.argv[1] == "counters":
        counters(sys.argv[2])
    elif len(sys.argv) == 4 and sys.argv[1] == "derive":
        derive(sys.argv[2], sys.argv[3])
    elif len(sys.argv) == 4 and sys.argv[1] == "traffic":
        traffic(sys.argv[2], sys.argv[3])
    else:
        raise SystemExit(__doc__)
