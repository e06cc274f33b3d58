"""Host-side logic of bench.py (no GPU): the one-GPU guard, and the per-launch traffic summaries built
from rocprofv3 counter CSVs (dispatch order -> op names, calibration on the 1 GiB copy, source hashes)."""
import csv
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, cwd=ROOT, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def _write_csv(path, counter, rows):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for i, (name, value) in enumerate(rows):
            # a counter summed over two hardware instances, as rocprofv3 reports per-block values
            w.writerow({"Dispatch_Id": i + 1, "Kernel_Name": name, "Counter_Name": counter, "Counter_Value": value / 2})
            w.writerow({"Dispatch_Id": i + 1, "Kernel_Name": name, "Counter_Name": counter, "Counter_Value": value / 2})


def test_pmc_summary_maps_dispatches_and_calibrates(tmp_path, monkeypatch):
    gemm = "void mxmoe::(anonymous namespace)::mx_grouped_gemm_kernel<0, 0, true, false, false>(mxmoe::GemmArgs)"
    quant = "void mxmoe::mx_colwise_kernel<true, false, true, false>(...)"
    copy = "__amd_rocclr_copyBuffer"
    # the step's launch order (bench.STEP_ORDER): quantisers and GEMMs of both layers interleaved
    order = [quant if "quant" in n else gemm for n in bench.STEP_ORDER]
    assert len(order) == 11 and order.count(gemm) == 6
    fetch_kib = 2 * (1 << 20)            # the 1 GiB copy reads as 2 GiB: factor 1/2
    write_kib = 1 << 20
    fetch = [(copy, 8.0), (copy, fetch_kib)] + [(n, 1000.0 * (i + 1)) for i, n in enumerate(order)]
    write = [(copy, 4.0), (copy, write_kib)] + [(n, 10.0 * (i + 1)) for i, n in enumerate(order)]
    fcsv, wcsv = tmp_path / "f.csv", tmp_path / "w.csv"
    _write_csv(fcsv, "FETCH_SIZE", fetch)
    _write_csv(wcsv, "WRITE_SIZE", write)
    gfile, qfile = tmp_path / "gemm.txt", tmp_path / "quant.txt"
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(gfile))
    monkeypatch.setattr(bench, "QUANT_TRAFFIC_FILE", str(qfile))
    bench.pmc_summary(str(fcsv), str(wcsv), ["cmd a", "cmd b"])
    g = json.loads(gfile.read_text().splitlines()[-1])
    q = json.loads(qfile.read_text().splitlines()[-1])
    assert g["source_sha256"] == bench.gemm_source_hash() and q["source_sha256"] == bench.quant_source_hash()
    assert abs(g["calibration"]["FETCH_SIZE"] - 0.5) < 1e-12 and g["calibration"]["WRITE_SIZE"] == 1.0
    # dispatch k of `order` (1-based) read 1000 k KiB fetched and 10 k KiB written
    want = {}
    gi = qi = 0
    for k, n in enumerate(order, start=1):
        name = bench.GEMM_NAMES[gi] if n == gemm else bench.QUANT_NAMES[qi]
        if n == gemm:
            gi += 1
        else:
            qi += 1
        want[name] = (1000.0 * k * 1024 * 0.5, 10.0 * k * 1024)
    for name in bench.GEMM_NAMES:
        assert g["fetch"][name] == round(want[name][0]) and g["write"][name] == round(want[name][1])
        assert g["ops"][name] == round(want[name][0] + want[name][1])
    for name in bench.QUANT_NAMES:
        assert q["ops"][name] == round(want[name][0] + want[name][1])
    assert "cmd a" in gfile.read_text() and "cmd b" in qfile.read_text()
    # the summaries are read back while the kernel sources are unchanged, and ignored otherwise
    assert bench.read_traffic(str(gfile)) == g["ops"]
    assert bench.read_traffic(str(qfile), bench.quant_source_hash()) == q["ops"]
    assert bench.read_traffic(str(qfile), "0" * 16) is None


def test_layer_shapes_match_the_workloads():
    import numpy as np
    import workloads as W
    tiny = W.make_workload("tiny").layers[0]
    assert W.layer_shapes("tiny") == [(tiny.name, tiny.M, tiny.N, tiny.K)]
    # the routed-row counts of the large workloads, from their (cheap) group-size draws
    assert int(np.sum(W._sizes_zipf_shard(np.random.default_rng(103)))) == W.layer_shapes("dsv3_671b_shard")[0][1]
    assert int(np.sum(W._sizes_top6(np.random.default_rng(102)))) == W.layer_shapes("dsv3_16b")[0][1]
    assert int(np.sum(W._sizes_dirichlet(np.random.default_rng(104)))) == W.layer_shapes("llama4_scout")[0][1]


def test_mfma_summary_clock_and_utilisation(tmp_path, monkeypatch):
    gemm = "void mxmoe::(anonymous namespace)::mx_grouped_gemm_kernel<0, 0, true, false, false>(mxmoe::GemmArgs)"
    quant = "void mxmoe::mx_colwise_kernel<true, false, true, false>(...)"
    order = [quant if "quant" in n else gemm for n in bench.STEP_ORDER] * 2
    ns = {}
    with open(tmp_path / "p_counter_collection.csv", "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for i, n in enumerate(order, start=1):
            ns[i] = 1_000_000 * i                                 # launch i lasts i ms
            # 2 GHz on every XCD: 8 x 2e6 i cycles summed over the XCDs; MfmaUtil 50 + i %
            for c, v in (("GRBM_GUI_ACTIVE", 8 * 2.0 * ns[i]), ("SQ_VALU_MFMA_BUSY_CYCLES", 1e6 * i),
                         ("MfmaUtil", 50.0 + i)):
                w.writerow({"Dispatch_Id": i, "Kernel_Name": n, "Counter_Name": c, "Counter_Value": v})
    with open(tmp_path / "p_kernel_trace.csv", "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Dispatch_Id", "Start_Timestamp", "End_Timestamp"])
        w.writeheader()
        for i in ns:
            w.writerow({"Dispatch_Id": i, "Start_Timestamp": 10 * ns[i], "End_Timestamp": 11 * ns[i]})
    out = tmp_path / "mfma.txt"
    monkeypatch.setattr(bench, "MFMA_FILE", str(out))
    bench.mfma_summary(str(tmp_path), ["cmd"])
    rec = json.loads(out.read_text().splitlines()[-1])
    gemm_disp = [i for i, n in enumerate(order, start=1) if n == gemm]
    shapes = {f"{l}.{k}": 2.0 * M * N * K for l, M, N, K in bench_shapes()
              for k in ("fwd", "fwd_swiglu", "dgrad", "wgrad")}
    assert len(gemm_disp) == 2 * len(bench.GEMM_NAMES)
    for j, name in enumerate(bench.GEMM_NAMES):
        # two steps: each op's figures are the mean over its two launches
        i, i2 = gemm_disp[j], gemm_disp[j + len(bench.GEMM_NAMES)]
        o = rec["ops"][name]
        t = (ns[i] + ns[i2]) / 2
        assert abs(o["clock_ghz"] - 2.0) < 1e-9 and o["us"] == round(t / 1e3, 1)
        assert o["mfma_util"] == round((50.0 + (i + i2) / 2) / 100, 4)
        tf = shapes[name] / (t * 1e-9) / 1e12
        assert abs(o["tflops"] - round(tf, 1)) < 1e-9
        assert abs(o["frac_of_rate_at_clock"] - round(tf / (1024 * 1024 * 2.0e9 / 1e12), 4)) < 1e-9


def bench_shapes():
    from workloads import layer_shapes
    return layer_shapes("dsv3_671b_shard")


def test_stats_summary_groups_launches_by_grid(tmp_path, monkeypatch):
    name = "void mxmoe::(anonymous namespace)::mx_grouped_gemm_kernel<2, 0, true, false, false>(mxmoe::GemmArgs)"
    with open(tmp_path / "bench_kernel_stats.csv", "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Name", "Calls", "TotalDurationNs", "AverageNs", "Percentage", "MinNs", "MaxNs", "StdDev"])
        w.writerow([name, 3, 600, 200, 100.0, 100, 300, 81.6])
    fields = ["Kernel_Name", "Start_Timestamp", "End_Timestamp", "Grid_Size_X", "Grid_Size_Y", "Grid_Size_Z",
              "VGPR_Count", "Accum_VGPR_Count", "LDS_Block_Size", "Scratch_Size"]
    with open(tmp_path / "bench_kernel_trace.csv", "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=fields)
        w.writeheader()
        for start, end, grid in ((0, 1000, 512), (5000, 8000, 1024), (9000, 14000, 1024)):
            w.writerow({"Kernel_Name": name, "Start_Timestamp": start, "End_Timestamp": end, "Grid_Size_X": grid,
                        "Grid_Size_Y": 1, "Grid_Size_Z": 1, "VGPR_Count": 112, "Accum_VGPR_Count": 0,
                        "LDS_Block_Size": 139264, "Scratch_Size": 0})
    out = tmp_path / "stats.md"
    monkeypatch.setattr(bench, "STATS_FILE", str(out))
    bench.stats_summary(str(tmp_path))
    text = out.read_text()
    assert bench.STATS_CMD in text and "mxmoe::mx_grouped_gemm_kernel<2, 0, true, false, false>" in text
    rows = [l for l in text.splitlines() if l.startswith("| `")]
    # grid 512: one launch of 1 us; grid 1024: two launches of 3 and 5 us
    assert rows[0].endswith("| 512 | 112 | 0 | 139264 | 0 | 1 | 1.0 | 1.0 |")
    assert rows[1].endswith("| 1024 | 112 | 0 | 139264 | 0 | 2 | 4.0 | 3.0 |")
