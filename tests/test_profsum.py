"""Host logic of the rocprof summariser (bit_residual_binarized_amd.profsum) on
small hand-written CSV files in rocprofv3's column layout."""
import csv
import os

from bit_residual_binarized_amd import profsum

NAME = "void rabit::(anonymous namespace)::k_gemv<1, {ring}, false, 2, 0>(rabit::(anonymous namespace)::Args)"
COPY = "__amd_rocclr_copyBuffer"


def _write(path, rows):
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=list(rows[0]))
        w.writeheader()
        w.writerows(rows)


def _counter_rows(counter, per_shape_kib, copy_kib):
    rows = [{"Kernel_Name": COPY, "Grid_Size": 131072, "Counter_Name": counter, "Counter_Value": copy_kib}]
    shapes = {("false", 640 * 256): "qkv", ("false", 512 * 256): "o", ("true", 512 * 256): "gate+up",
              ("true", 448 * 256): "down"}
    for (ring, grid), lab in shapes.items():
        for v in per_shape_kib[lab]:
            rows.append({"Kernel_Name": NAME.format(ring=ring), "Grid_Size": grid, "Counter_Name": counter,
                         "Counter_Value": v})
    return rows


def test_short_names():
    assert profsum._short(NAME.format(ring="true")) == "k_gemv<1, true, false, 2, 0>"
    assert profsum._short("k_resid_stats(double const*, int)") == "k_resid_stats"


def test_traffic_divides_by_the_copy_factor(tmp_path, capsys):
    # FETCH reads half the true bytes on the copy: every k_gemv figure doubles
    fetch = {"qkv": [100.0, 300.0], "o": [50.0], "gate+up": [1000.0], "down": [400.0]}
    write = {"qkv": [10.0], "o": [5.0], "gate+up": [40.0], "down": [20.0]}
    _write(str(tmp_path / "f" / "host" / "1_fetch_counter_collection.csv"),
           _counter_rows("FETCH_SIZE", fetch, 0.5 * (256 << 20) / 1024))
    _write(str(tmp_path / "w" / "host" / "1_write_counter_collection.csv"),
           _counter_rows("WRITE_SIZE", write, 1.0 * (256 << 20) / 1024))
    profsum.traffic(str(tmp_path / "f"), str(tmp_path / "w"))
    kv = dict(l.split(": ", 1) for l in capsys.readouterr().out.splitlines())
    assert kv["fetch_factor"] == "0.5000" and kv["write_factor"] == "1.0000"
    assert kv["qkv_launches"] == "2"
    assert float(kv["qkv_fetch_kib"]) == 400.0  # mean of 200 and 600
    assert float(kv["qkv_traffic_bytes"]) == (400.0 + 10.0) * 1024
    per = [(400 + 10), (100 + 5), (2000 + 40), (800 + 20)]
    assert float(kv["traffic_bytes_per_launch"]) == round(sum(per) * 1024 / 4)
    assert kv["gemv_source_sha256"] == profsum.gemv_sha()
