"""Benchmark of the MXFP8 expert-layer hot path on one MI355X.

One step is the whole path, forward and backward, of both expert linear layers
(gate+up and down) of the DeepSeek-V3-671B one-GPU expert shard: 8 local
experts, 65536 routed rows with Zipf(1.2)-skewed group sizes (one expert with
17 rows), hidden 7168, gate+up N=4096, down N=7168.  In training order:

    gate+up: X, W -> both MX layouts (one launch each)
             grouped GEMM forward, SwiGLU and MX quantisation of H (both layouts) in its epilogue
    down:    W -> both layouts; grouped GEMM forward on H
             dY -> both layouts; grouped GEMM dgrad (dH bf16); grouped GEMM wgrad on H column-wise
    gate+up: dY -> both layouts; grouped GEMM dgrad (dX bf16); grouped GEMM wgrad (dW fp32)

`value` = algorithmic GEMM flops of the step (2*M*N*K per GEMM, real rows only)
divided by the wall time of the whole step, quantisers included, inputs
resident in HBM.  Every kernel launch is also timed with HIP events on the
stream it runs on; the JSON line carries per-op figures, the roofline of the
dominant kernel and the CPU oracle timed on a bounded sample.

    python bench.py [--steps K] [--warmup W] [--gpus 1]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import platform
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0           # MI355X HBM3E
MFMA_PEAK_TFLOPS = {"bf16": 2500.0, "mxfp8": 5000.0, "mxfp4": 10100.0}
QUANT_BYTES_PER_ELEM = 2.0 + 1.0 + 1.0 / 32.0   # bf16 in, E4M3 out, one E8M0 per 32
DUAL_BYTES_PER_ELEM = 2.0 + 2.0 * (1.0 + 1.0 / 32.0)   # bf16 in once, both MX layouts out
# the workload the step runs on (the DeepSeek-V3-671B one-GPU expert shard unless --workload says
# otherwise; the profile summaries are named for it)
WORKLOAD = "dsv3_671b_shard"
WORKLOAD_TITLE = {"dsv3_671b_shard": "DeepSeek-V3-671B expert shard", "dsv3_16b": "DeepSeek-V3-16B layers",
                  "llama4_scout": "Llama-4-Scout layers"}
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "gemm_traffic_dsv3_671b_shard.txt")
GEMM_SOURCES = [os.path.join(ROOT, "precision_moe_expert_mx_amd", "csrc", f) for f in ("gemm_mx.hip", "grouped_tile.h", "common.h")]


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def gemm_source_hash() -> str:
    h = hashlib.sha256()
    for p in GEMM_SOURCES:
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


# ------------------------------------------------------------------------------------------- ops
class Op:
    """One kernel launch of the step: `kind` is 'quant' (work = bytes) or 'gemm' (work = flops)."""

    def __init__(self, name, kind, fn, work, kernel):
        self.name, self.kind, self.fn, self.work, self.kernel = name, kind, fn, work, kernel
        self.ms = []


def build_layer_ops(m, torch, lay, dev_in, fast=False, fused=True, tiled=False):
    """Allocate the layer's device buffers and return its ops in step order.

    fused: X, W and dY each get both MX layouts from one dual-layout launch (3 quantiser launches
    per layer); otherwise six separate row-wise / column-wise launches.  tiled: the column-wise copies
    in the 128-byte tiled layout (dual launches and the backward GEMMs of that layout; fused only)."""
    assert fused or not tiled
    G, M, N, K = lay.G, lay.M, lay.N, lay.K
    x, w, dy, offs = dev_in
    d = x.device
    u8 = torch.uint8
    # recommended row pitches of the column-wise copies (the minimum, off pitches that write slowly)
    ld = m.mx_colwise_ld(M, G)
    ldw = m.mx_colwise_ld(G * N)
    b = dict(
        qx=torch.empty((M, K), dtype=u8, device=d),
        sx=torch.empty((K // 128, M, 4) if tiled else (M, K // 32), dtype=u8, device=d),
        qw=torch.empty((G * N, K), dtype=u8, device=d),
        sw=torch.empty((K // 128, G * N, 4) if tiled else (G * N, K // 32), dtype=u8, device=d),
        y=torch.empty((M, N), dtype=torch.bfloat16, device=d),
        qdy=torch.empty((M, N), dtype=u8, device=d),
        sdy=torch.empty((N // 128, M, 4) if tiled else (M, N // 32), dtype=u8, device=d),
        qwT=torch.empty((ldw // 128, K, 128) if tiled else (K, ldw), dtype=u8, device=d),
        swT=torch.empty((ldw // 128, K, 4) if tiled else (K, ldw // 32), dtype=u8, device=d),
        dx=torch.empty((M, K), dtype=torch.bfloat16, device=d),
        qdyT=torch.empty((ld // 128, N, 128) if tiled else (N, ld), dtype=u8, device=d),
        sdyT=torch.empty((ld // 128, N, 4) if tiled else (N, ld // 32), dtype=u8, device=d),
        qxT=torch.empty((ld // 128, K, 128) if tiled else (K, ld), dtype=u8, device=d),
        sxT=torch.empty((ld // 128, K, 4) if tiled else (K, ld // 32), dtype=u8, device=d),
        dw=torch.empty((G, N, K), dtype=torch.float32, device=d),
    )
    w2 = w.view(G * N, K)
    f = 2.0 * M * N * K
    n = lay.name
    mxb = 1.0 + 1.0 / 32.0          # E4M3 byte plus its share of an E8M0 scale
    gemm_bytes = {"fwd": (M * K + G * N * K) * mxb + M * N * 2, "dgrad": (M * N + G * N * K) * mxb + M * K * 2,
                  "wgrad": (M * N + M * K) * mxb + G * N * K * 4}
    fw = m.mx_grouped_gemm_fwd_tiled if tiled else m.mx_grouped_gemm_fwd
    fwd = Op(f"{n}.fwd", "gemm", lambda: fw(b["qx"], b["sx"], b["qw"], b["sw"], offs, N, "bf16", y=b["y"], fast=fast),
             f, "grouped_gemm fwd")
    dg = m.mx_grouped_gemm_dgrad_tiled if tiled else m.mx_grouped_gemm_dgrad
    wg = m.mx_grouped_gemm_wgrad_tiled if tiled else m.mx_grouped_gemm_wgrad
    dual = m.mx_quantize_dual_tiled if tiled else m.mx_quantize_dual
    dual_kernel = "mx_colwise_kernel<true, false, true, false, true>" if tiled else "mx_colwise_kernel<true, false>"
    dgrad = Op(f"{n}.dgrad", "gemm", lambda: dg(b["qdy"], b["sdy"], b["qwT"], b["swT"], offs, K, "bf16", dx=b["dx"],
                                                fast=fast), f, "grouped_gemm dgrad")
    wgrad = Op(f"{n}.wgrad", "gemm", lambda: wg(b["qdyT"], b["sdyT"], b["qxT"], b["sxT"], offs, M, "f32", dw=b["dw"],
                                                fast=fast), f, "grouped_gemm wgrad")
    if fused:
        ops = [
            Op(f"{n}.quant_x_dual", "quant",
               lambda: dual(x, offs, ld=ld, q=b["qx"], s=b["sx"], qT=b["qxT"], sT=b["sxT"]),
               M * K * DUAL_BYTES_PER_ELEM, dual_kernel),
            Op(f"{n}.quant_w_dual", "quant",
               lambda: dual(w2, None, ld=ldw, q=b["qw"], s=b["sw"], qT=b["qwT"], sT=b["swT"]),
               G * N * K * DUAL_BYTES_PER_ELEM, dual_kernel),
            fwd,
            Op(f"{n}.quant_dy_dual", "quant",
               lambda: dual(dy, offs, ld=ld, q=b["qdy"], s=b["sdy"], qT=b["qdyT"], sT=b["sdyT"]),
               M * N * DUAL_BYTES_PER_ELEM, dual_kernel),
            dgrad,
            wgrad,
        ]
    else:
        ops = [
            Op(f"{n}.quant_x_row", "quant", lambda: m.mx_quantize_rowwise(x, b["qx"], b["sx"]),
               M * K * QUANT_BYTES_PER_ELEM, "mx_rowwise_kernel"),
            Op(f"{n}.quant_w_row", "quant", lambda: m.mx_quantize_rowwise(w2, b["qw"], b["sw"]),
               G * N * K * QUANT_BYTES_PER_ELEM, "mx_rowwise_kernel"),
            fwd,
            Op(f"{n}.quant_dy_row", "quant", lambda: m.mx_quantize_rowwise(dy, b["qdy"], b["sdy"]),
               M * N * QUANT_BYTES_PER_ELEM, "mx_rowwise_kernel"),
            Op(f"{n}.quant_w_col", "quant",
               lambda: m.mx_quantize_colwise(w2, None, ld=ldw, qT=b["qwT"], sT=b["swT"]),
               G * N * K * QUANT_BYTES_PER_ELEM, "mx_colwise_kernel<false, false>"),
            dgrad,
            Op(f"{n}.quant_dy_col", "quant", lambda: m.mx_quantize_colwise(dy, offs, ld=ld, qT=b["qdyT"], sT=b["sdyT"]),
               M * N * QUANT_BYTES_PER_ELEM, "mx_colwise_kernel<false, false>"),
            Op(f"{n}.quant_x_col", "quant", lambda: m.mx_quantize_colwise(x, offs, ld=ld, qT=b["qxT"], sT=b["sxT"]),
               M * K * QUANT_BYTES_PER_ELEM, "mx_colwise_kernel<false, false>"),
            wgrad,
        ]
    for op in ops:
        if op.kind == "gemm":
            op.bytes = gemm_bytes[op.name.split(".")[1]]
            # the MFMA rate the feed runs at: bf16 for the precise feed, the MXFP8 rate for the fast one
            op.peak_tflops = MFMA_PEAK_TFLOPS["mxfp8" if fast else "bf16"]
    return ops, b


# the step's column-wise copies (X, dY, W of both layers; H from the gated forward) use the 128-byte
# tiled layout: its quantiser launches write whole tiles (measured 0.4-1% faster per step than row-major)
STEP_TILED = True


def build_step_ops(m, torch, layers, dev_ins, tiled=False):
    """The expert MLP's step in training order, with both fused sides: per layer, X, W and dY each get
    both MX layouts from one dual-layout launch; the gate+up forward applies SwiGLU in its epilogue and
    writes H row-wise and column-wise, which the down layer's forward and weight gradient consume (no
    quantiser launch for H, H never in HBM in a wider format).  The two layers share the routing.

    Order: gate+up X, W; gate+up forward (+ H); down W; down forward; down dY; down dgrad; down wgrad;
    gate+up dY; gate+up dgrad; gate+up wgrad.  The dY of each layer is the workload's synthetic
    gradient (the activation's backward is not part of this path)."""
    gu, dn = layers
    assert gu.name == "gate_up" and dn.name == "down" and dn.K == gu.N // 2 and np.array_equal(gu.offs, dn.offs)
    gu_ops, gb = build_layer_ops(m, torch, gu, dev_ins[0], tiled=tiled)
    dn_ops, db = build_layer_ops(m, torch, dn, dev_ins[1], tiled=tiled)
    by = {op.name: op for op in gu_ops + dn_ops}
    G, M, N, K = gu.G, gu.M, gu.N, gu.K
    offs = dev_ins[0][3]
    H = N // 2
    mxb = 1.0 + 1.0 / 32.0
    swiglu = m.mx_grouped_gemm_fwd_swiglu_tiled if tiled else m.mx_grouped_gemm_fwd_swiglu
    fused = Op("gate_up.fwd_swiglu", "gemm",
               lambda: swiglu(gb["qx"], gb["sx"], gb["qw"], gb["sw"], offs, N, y=gb["y"], qh=db["qx"], sh=db["sx"],
                              qhT=db["qxT"], shT=db["sxT"]),
               2.0 * M * N * K, "grouped_gemm fwd + SwiGLU + MX(H) both layouts")
    fused.bytes = (M * K + G * N * K) * mxb + M * N * 2 + 2 * M * H * mxb
    fused.peak_tflops = MFMA_PEAK_TFLOPS["bf16"]
    by[fused.name] = fused
    ops = [by[n] for n in STEP_ORDER]
    return ops, (gb, db)


def to_device(torch, a: np.ndarray):
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).cuda().view(torch.bfloat16)
    return torch.from_numpy(a).cuda()


def time_ops(torch, ops, steps, warmup, per_op=True):
    """Run `warmup` untimed steps, then `steps` timed ones; returns ms per step (whole-step events)."""
    for _ in range(warmup):
        for op in ops:
            op.fn()
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    evs = []
    t0.record()
    for _ in range(steps):
        for op in ops:
            if per_op:
                a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                a.record()
                op.fn()
                b.record()
                evs.append((op, a, b))
            else:
                op.fn()
    t1.record()
    torch.cuda.synchronize()
    for op, a, b in evs:
        op.ms.append(a.elapsed_time(b))
    return t0.elapsed_time(t1) / steps


def op_summary(op):
    ms = float(np.mean(op.ms))
    d = {"ms": round(ms, 4), "ms_min": round(float(np.min(op.ms)), 4)}
    if op.kind == "gemm":
        d["tflops"] = round(op.work / (ms * 1e-3) / 1e12, 1)
        if getattr(op, "bytes", None) and getattr(op, "peak_tflops", None):
            # fraction of the op's own roofline: the larger of its time at the MFMA peak and its time at
            # the HBM peak (algorithmic bytes), over the measured time
            t_roof = max(op.work / (op.peak_tflops * 1e12), op.bytes / (HBM_PEAK_GBS * 1e9))
            d["frac_of_op_roofline"] = round(t_roof / (ms * 1e-3), 4)
    else:
        d["gbps"] = round(op.work / (ms * 1e-3) / 1e9, 1)
        d["frac_hbm"] = round(d["gbps"] / HBM_PEAK_GBS, 3)
    return d


# ------------------------------------------------------------------------------------------- traffic
# Per-launch HBM bytes of the step's launches come from two rocprofv3 counter runs of this script
# (FETCH_SIZE, then WRITE_SIZE); each summary carries a hash of the sources of the kernels it
# covers and is ignored once they change.
QUANT_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "quant_traffic_dsv3_671b_shard.txt")
QUANT_SOURCES = [os.path.join(ROOT, "precision_moe_expert_mx_amd", "csrc", f) for f in ("quant_mx.hip", "common.h")]
# the step's launches in order (build_step_ops): the profile summaries map kernel dispatches to these
STEP_ORDER = ["gate_up.quant_x_dual", "gate_up.quant_w_dual", "gate_up.fwd_swiglu", "down.quant_w_dual", "down.fwd",
              "down.quant_dy_dual", "down.dgrad", "down.wgrad", "gate_up.quant_dy_dual", "gate_up.dgrad",
              "gate_up.wgrad"]
GEMM_NAMES = [n for n in STEP_ORDER if "quant" not in n]
QUANT_NAMES = [n for n in STEP_ORDER if "quant" in n]


def quant_source_hash() -> str:
    h = hashlib.sha256()
    for p in QUANT_SOURCES:
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def read_traffic(path=TRAFFIC_FILE, src_hash=None):
    """Per-launch HBM bytes of the step's ops from a committed counter summary (None if stale)."""
    if not os.path.exists(path):
        return None
    rec = None
    with open(path) as f:
        for line in f:
            line = line.strip()
            if line.startswith("{"):
                rec = json.loads(line)
    if not rec or rec.get("source_sha256") != (src_hash or gemm_source_hash()):
        return None
    return rec.get("ops", {})


def pmc_summary(fetch_csv: str, write_csv: str, cmds) -> None:
    """Per-launch HBM bytes of the GEMM launches and the dual-layout quantiser launches of a step
    (STEP_ORDER) from two rocprofv3 counter runs of this script (FETCH_SIZE, then WRITE_SIZE, KiB per
    dispatch), each scaled by what the same counter reads for the 1 GiB device copy the script
    performs before timing."""
    import csv
    res = {}
    factors = {}
    for counter, path in (("FETCH_SIZE", fetch_csv), ("WRITE_SIZE", write_csv)):
        per_disp = {}
        for r in csv.DictReader(open(path)):
            if r["Counter_Name"] != counter:
                continue
            d = per_disp.setdefault(int(r["Dispatch_Id"]), {"name": r["Kernel_Name"], "v": 0.0})
            d["v"] += float(r["Counter_Value"])
        disp = [per_disp[k] for k in sorted(per_disp)]
        copies = [d["v"] for d in disp if "copyBuffer" in d["name"]]
        cal_kib = max(copies)
        factors[counter] = (1 << 30) / (cal_kib * 1024.0)
        for key, names in (("mx_grouped_gemm", GEMM_NAMES), ("mx_colwise_kernel", QUANT_NAMES)):
            launches = [d["v"] for d in disp if key in d["name"]]
            for i, v in enumerate(launches):
                res.setdefault(names[i % len(names)], {}).setdefault(counter, []).append(v * 1024.0 * factors[counter])
    for path, names, src, what in ((TRAFFIC_FILE, GEMM_NAMES, gemm_source_hash(), "grouped-GEMM"),
                                   (QUANT_TRAFFIC_FILE, QUANT_NAMES, quant_source_hash(), "dual-layout MX quantiser")):
        sel = {n: res[n] for n in names if n in res}
        rec = {"source_sha256": src, "calibration": factors,
               "ops": {n: round(float(np.mean(c["FETCH_SIZE"])) + float(np.mean(c["WRITE_SIZE"]))) for n, c in sel.items()},
               "fetch": {n: round(float(np.mean(c["FETCH_SIZE"]))) for n, c in sel.items()},
               "write": {n: round(float(np.mean(c["WRITE_SIZE"]))) for n, c in sel.items()}}
        with open(path, "w") as f:
            f.write(f"# HBM traffic per launch of the {len(names)} {what} launches of one step "
                    f"({WORKLOAD_TITLE[WORKLOAD]})\n")
            f.write("# bytes = counter KiB * 1024 * (2^30 / counter KiB of the 1 GiB device copy); commands (repository root):\n")
            for c in cmds:
                f.write(f"#   {c}\n")
            f.write(json.dumps(rec) + "\n")
        print(json.dumps(rec))


MFMA_FILE = os.path.join(ROOT, "profiles", "gemm_mfma_dsv3_671b_shard.txt")
MFMA_COUNTERS = ("GRBM_GUI_ACTIVE", "SQ_VALU_MFMA_BUSY_CYCLES", "MfmaUtil")
N_XCD = 8                                    # GRBM_GUI_ACTIVE is summed over the MI355X's 8 XCDs


def mfma_summary(pmc_dir: str, cmds) -> None:
    """Clock and MFMA use of the six GEMM launches of one step, from one rocprofv3 run of this script
    with --kernel-trace and --pmc of MFMA_COUNTERS: the shader clock is GRBM_GUI_ACTIVE (summed over the
    8 XCDs) / 8 over the launch's duration; the achieved rate is set against the bf16 MFMA rate at that
    clock (1024 flop per clock per SIMD, 1024 SIMDs); MfmaUtil is rocprofv3's own metric,
    sum(SQ_VALU_MFMA_BUSY_CYCLES) / (max over XCDs of GRBM_GUI_ACTIVE x SIMD count), the busy count being
    per SIMD."""
    import csv
    from workloads import layer_shapes
    flops = {}
    for name, M, N, K in layer_shapes(WORKLOAD):
        for k in ("fwd", "fwd_swiglu", "dgrad", "wgrad"):
            flops[f"{name}.{k}"] = 2.0 * M * N * K
    per_disp = {}
    for r in csv.DictReader(open(os.path.join(pmc_dir, "p_counter_collection.csv"))):
        d = per_disp.setdefault(int(r["Dispatch_Id"]), {"name": r["Kernel_Name"]})
        d[r["Counter_Name"]] = d.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    dur = {}
    for r in csv.DictReader(open(os.path.join(pmc_dir, "p_kernel_trace.csv"))):
        dur[int(r["Dispatch_Id"])] = int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
    gemm = [k for k in sorted(per_disp) if "mx_grouped_gemm" in per_disp[k]["name"]]
    acc = {}
    for i, k in enumerate(gemm):
        acc.setdefault(GEMM_NAMES[i % len(GEMM_NAMES)], []).append((per_disp[k], dur[k]))
    ops = {}
    for n in GEMM_NAMES:
        if n not in acc:
            continue
        c = {m_: float(np.mean([d[m_] for d, _ in acc[n]])) for m_ in MFMA_COUNTERS}
        ns = float(np.mean([t for _, t in acc[n]]))
        ghz = c["GRBM_GUI_ACTIVE"] / N_XCD / ns
        tf = flops[n] / (ns * 1e-9) / 1e12
        rate_at_clock = 1024 * 1024 * ghz * 1e9 / 1e12
        ops[n] = {"us": round(ns / 1e3, 1), "clock_ghz": round(ghz, 3), "tflops": round(tf, 1),
                  "bf16_rate_at_clock_tflops": round(rate_at_clock, 1),
                  "frac_of_rate_at_clock": round(tf / rate_at_clock, 4),
                  "frac_of_bf16_peak": round(tf / MFMA_PEAK_TFLOPS["bf16"], 4),
                  "mfma_util": round(c["MfmaUtil"] / 100.0, 4),
                  "counters": {m_: round(v) for m_, v in c.items()}}
    rec = {"source_sha256": gemm_source_hash(), "ops": ops}
    with open(MFMA_FILE, "w") as f:
        f.write(f"# Clock and MFMA use of the six grouped-GEMM launches of one step ({WORKLOAD_TITLE[WORKLOAD]},\n")
        f.write("# precise feed, bf16 MFMA).  clock = GRBM_GUI_ACTIVE / 8 XCDs / duration; frac_of_rate_at_clock =\n")
        f.write("# achieved TFLOP/s / (1024 flop/clk/SIMD x 1024 SIMDs x clock); mfma_util = rocprofv3 MfmaUtil\n")
        f.write("# (sum SQ_VALU_MFMA_BUSY_CYCLES / (max-XCD GRBM_GUI_ACTIVE x SIMDs)); commands (repository root):\n")
        for c_ in cmds:
            f.write(f"#   {c_}\n")
        f.write(json.dumps(rec) + "\n")
    print(json.dumps(rec))


STATS_FILE = os.path.join(ROOT, "profiles", "kernel_stats_dsv3_671b_shard.md")
STATS_CMD = ("rocprofv3 --kernel-trace --stats --output-format csv -d gpurun_out/prof5 -o bench -- "
             "python3 bench.py --steps 5 --warmup 2 --no-cpu-baseline --no-extra-legs")


def set_workload(wname: str) -> None:
    """Run on `wname`: the profile summaries and their commands are named for it."""
    global WORKLOAD, TRAFFIC_FILE, QUANT_TRAFFIC_FILE, MFMA_FILE, STATS_FILE, STATS_CMD
    if wname == WORKLOAD:
        return
    WORKLOAD = wname
    prof = os.path.join(ROOT, "profiles")
    TRAFFIC_FILE = os.path.join(prof, f"gemm_traffic_{wname}.txt")
    QUANT_TRAFFIC_FILE = os.path.join(prof, f"quant_traffic_{wname}.txt")
    MFMA_FILE = os.path.join(prof, f"gemm_mfma_{wname}.txt")
    STATS_FILE = os.path.join(prof, f"kernel_stats_{wname}.md")
    STATS_CMD = STATS_CMD.replace("gpurun_out/prof5 ", f"gpurun_out/prof5_{wname} ") + f" --workload {wname}"


def stats_summary(prof_dir: str) -> None:
    """Markdown summary of a rocprofv3 --kernel-trace --stats run of this script (STATS_CMD): the
    statistics table and, from the kernel trace, each kernel's launches grouped by grid size with their
    register and LDS use and mean and minimum durations."""
    import csv
    import re
    from collections import defaultdict

    def short(n):
        n = re.sub(r"^void ", "", n)
        n = re.sub(r"\(anonymous namespace\)::", "", n)
        return re.sub(r"\(.*\)$", "", n)

    out = [f"# Kernel statistics: {WORKLOAD_TITLE[WORKLOAD]}, fwd+bwd step (precise feed)", "",
           "Commands (from the repository root, one MI355X):", "", "```", STATS_CMD,
           f"python3 bench.py --stats-summary {prof_dir}"
           + ("" if WORKLOAD == "dsv3_671b_shard" else f" --workload {WORKLOAD}"), "```", "",
           "## rocprofv3 kernel statistics (all launches)", "",
           "| Name | Calls | TotalDurationNs | AverageNs | Percentage | MinNs | MaxNs | StdDev |",
           "|---|---|---|---|---|---|---|---|"]
    for r in csv.DictReader(open(os.path.join(prof_dir, "bench_kernel_stats.csv"))):
        out.append("| " + " | ".join([short(r["Name"])] + [r[k] for k in ("Calls", "TotalDurationNs", "AverageNs",
                                                                           "Percentage", "MinNs", "MaxNs", "StdDev")]) + " |")
    out += ["", "## Per kernel and grid size (from the kernel trace)", "",
            "| kernel | grid (work-items) | VGPR | AGPR | LDS B | scratch B | calls | avg µs | min µs |",
            "|---|---|---|---|---|---|---|---|---|"]
    groups, meta = defaultdict(list), {}
    for r in csv.DictReader(open(os.path.join(prof_dir, "bench_kernel_trace.csv"))):
        k = (short(r["Kernel_Name"]), int(r["Grid_Size_X"]) * int(r["Grid_Size_Y"]) * int(r["Grid_Size_Z"]))
        groups[k].append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
        meta[k] = (r["VGPR_Count"], r["Accum_VGPR_Count"], r["LDS_Block_Size"], r["Scratch_Size"])
    for k in sorted(groups):
        v = groups[k]
        out.append(f"| `{k[0]}` | {k[1]} | " + " | ".join(meta[k]) + f" | {len(v)} | {sum(v) / len(v):.1f} | {min(v):.1f} |")
    with open(STATS_FILE, "w") as f:
        f.write("\n".join(out) + "\n")
    print("\n".join(out))


# ------------------------------------------------------------------------------------------- CPU oracle
def gpu_sample(lay, bufs, rows_per_expert=2048):
    """Host copies of what the timed step left in the buffers the CPU oracle's sample covers: the
    largest expert's first routed rows of X's row-wise codes and scales and of the forward output."""
    g = int(np.argmax(lay.sizes))
    r0 = int(lay.offs[g])
    rows = int(min(rows_per_expert, lay.sizes[g]))
    sl = slice(r0, r0 + rows)
    y = bufs["y"][sl].view(__import__("torch").int16).cpu().numpy().view(np.uint16)
    sx = bufs["sx"]
    if sx.dim() == 3:
        # tiled scales [K / 128, M, 4] -> the rows' row-major [rows, K / 32]
        sx = sx[:, sl, :].permute(1, 0, 2).reshape(rows, -1)
    else:
        sx = sx[sl]
    return {"qx": bufs["qx"][sl].cpu().numpy(), "sx": sx.cpu().numpy(), "y_bf16": y}


def cpu_baseline(lay, rows_per_expert=2048, gpu=None):
    """The oracle, as it stands, on a bounded sample: the largest expert's weights and its first
    `rows_per_expert` routed rows, quantised and contracted (forward GEMM) on the host.  With `gpu`
    (gpu_sample of the timed buffers), the oracle's result also gives the parity verdict of those
    buffers: row-wise codes and scales bit-exact, the forward output within 1e-5 * sum|ab| (bf16)."""
    import oracle
    # threads the oracle ran on: its float64 products use the BLAS thread pool, the quantisers one thread
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # noqa: BLE001
        blas_threads = 1
    host_cores = len(os.sched_getaffinity(0))
    g = int(np.argmax(lay.sizes))
    r0 = int(lay.offs[g])
    rows = int(min(rows_per_expert, lay.sizes[g]))
    t = time.perf_counter()
    qw, sw = oracle.mx_quantize_rowwise(lay.w.reshape(lay.G, lay.N, lay.K)[g])
    qx, sx = oracle.mx_quantize_rowwise(lay.x[r0:r0 + rows])
    ref, bound = oracle.mx_gemm_fwd(qx, sx, qw, sw, np.array([0, rows]), lay.N)
    dt = time.perf_counter() - t
    parity = None
    if gpu is not None:
        got = (gpu["y_bf16"].astype(np.uint32) << 16).view(np.float32).astype(np.float64)
        ok, worst, _ = oracle.check_gemm(got, ref, bound, "bf16")
        parity = {"rows": f"{lay.name} rows {r0}..{r0 + rows - 1} (expert {g})",
                  "quantiser_bit_exact": bool(np.array_equal(gpu["qx"], qx) and np.array_equal(gpu["sx"], sx)),
                  "fwd_within_tolerance": bool(ok), "fwd_worst_err_over_tol": round(float(worst), 4)}
    flops = 2.0 * rows * lay.N * lay.K
    cpu = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    cpu = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"value": round(flops / dt / 1e12, 5), "unit": "TFLOP/s", "cores": int(min(blas_threads, host_cores)),
            "host_cores": host_cores, "blas_threads": int(blas_threads), "kind": "oracle",
            "sample": f"{lay.name} layer, expert {g}: its weights [{lay.N}x{lay.K}] and {rows} routed rows "
                      f"MX-quantised by the oracle, then the fp64 grouped forward GEMM "
                      f"({flops / 1e9:.1f} GFLOP) with its error-bound pass; {dt:.1f} s",
            "seconds": round(dt, 2), "cpu": cpu, "parity_of_timed_buffers": parity}


# ------------------------------------------------------------------------------------------- blockwise
def mxfp4_leg(m, torch, wl, keep, steps=5, sample_rows=64):
    """MXFP4 (E2M1 elements, E8M0 per 32, block-scaled FP4 MFMA) on the same expert-shard step: per
    layer the six quantisers (row-wise X, W, dY; column-wise W, dY, X) and the three grouped GEMMs,
    with the step's device inputs.  Accuracy: relative Frobenius error of Y and dX against an fp64
    product of the original bf16 tensors on sampled rows."""
    ops = []
    bufs = []
    fp4_bytes = 2.0 + 0.5 + 1.0 / 32.0            # bf16 in, half a byte out, one scale per 32
    for lay, (dev_in, _) in zip(wl.layers, keep):
        G, M, N, K = lay.G, lay.M, lay.N, lay.K
        x, w, dy, offs = dev_in
        w2 = w.view(G * N, K)
        ld = m.mxfp4_colwise_ld(M, G)
        q = {}
        bufs.append(q)
        f = 2.0 * M * N * K
        n = lay.name

        def add(name, kind, fn, work):
            ops.append(Op(f"{n}.{name}", kind, fn, work, ""))
        add("quant_x", "quant", lambda q=q, x=x: q.update(x=m.mxfp4_quantize_rowwise(x)), M * K * fp4_bytes)
        add("quant_w", "quant", lambda q=q, w2=w2: q.update(w=m.mxfp4_quantize_rowwise(w2)), G * N * K * fp4_bytes)
        add("fwd", "gemm", lambda q=q, offs=offs, N=N: q.update(y=m.mxfp4_grouped_gemm_fwd(*q["x"], *q["w"], offs, N,
                                                                                         "bf16")), f)
        add("quant_dy", "quant", lambda q=q, dy=dy: q.update(dy=m.mxfp4_quantize_rowwise(dy)), M * N * fp4_bytes)
        add("quant_w_col", "quant", lambda q=q, w2=w2, G=G, N=N: q.update(wc=m.mxfp4_quantize_colwise(w2, None,
                                                                                                     ld=G * N)),
            G * N * K * fp4_bytes)
        add("dgrad", "gemm", lambda q=q, offs=offs, K=K: q.update(dx=m.mxfp4_grouped_gemm_dgrad(*q["dy"], *q["wc"], offs,
                                                                                              K, "bf16")), f)
        add("quant_dy_col", "quant", lambda q=q, dy=dy, offs=offs, ld=ld: q.update(dyc=m.mxfp4_quantize_colwise(
            dy, offs, ld=ld)), M * N * fp4_bytes)
        add("quant_x_col", "quant", lambda q=q, x=x, offs=offs, ld=ld: q.update(xc=m.mxfp4_quantize_colwise(
            x, offs, ld=ld)), M * K * fp4_bytes)
        add("wgrad", "gemm", lambda q=q, offs=offs, M=M: q.update(dw=m.mxfp4_grouped_gemm_wgrad(*q["dyc"], *q["xc"],
                                                                                               offs, M, "f32")), f)
    ms = time_ops(torch, ops, steps, 1)
    flops = sum(o.work for o in ops if o.kind == "gemm")
    gm = sum(float(np.mean(o.ms)) for o in ops if o.kind == "gemm")
    out = {"ms_per_step": round(ms, 4), "tflops": round(flops / (ms * 1e-3) / 1e12, 1),
           "gemm_tflops": round(flops / (gm * 1e-3) / 1e12, 1),
           "gemm_frac_of_fp4_peak": round(flops / (gm * 1e-3) / 1e12 / MFMA_PEAK_TFLOPS["mxfp4"], 4),
           "ops": {o.name: op_summary(o) for o in ops}}
    # accuracy of the gate+up layer on sampled rows
    lay, q = wl.layers[0], bufs[0]
    rng = np.random.default_rng(8)
    rows = np.sort(rng.choice(lay.M, sample_rows, replace=False))
    grp = np.searchsorted(lay.offs.astype(np.int64), rows, side="right") - 1
    xb, dyb = bf16_to_f64(lay.x[rows]), bf16_to_f64(lay.dy[rows])
    wf = lay.w.reshape(lay.G, lay.N, lay.K)
    y_ref = np.stack([xb[i] @ bf16_to_f64(wf[g]).T for i, g in enumerate(grp)])
    dx_ref = np.stack([dyb[i] @ bf16_to_f64(wf[g]) for i, g in enumerate(grp)])
    ridx = torch.from_numpy(rows).cuda()
    yg = q["y"][ridx].double().cpu().numpy()
    dxg = q["dx"][ridx].double().cpu().numpy()
    out["rel_fro_err_y"] = float(np.linalg.norm(yg - y_ref) / np.linalg.norm(y_ref))
    out["rel_fro_err_dx"] = float(np.linalg.norm(dxg - dx_ref) / np.linalg.norm(dx_ref))
    del ops, bufs
    torch.cuda.empty_cache()
    return out


def swiglu_leg(m, torch, lay, dev_in, steps=10):
    """The gate+up forward with SwiGLU and the MX quantisation of H in the GEMM epilogue, against the
    same outputs produced unfused: the forward GEMM writing bf16 Y, the activation by torch
    elementwise ops (a comparison path only), and the row-wise MX quantiser on bf16 H."""
    G, M, N, K = lay.G, lay.M, lay.N, lay.K
    H = N // 2
    x, w, _, offs = dev_in
    w2 = w.view(G * N, K)
    qx, sx = m.mx_quantize_rowwise(x)
    qw, sw = m.mx_quantize_rowwise(w2)
    y = torch.empty((M, N), dtype=torch.bfloat16, device=x.device)
    qh = torch.empty((M, H), dtype=torch.uint8, device=x.device)
    sh = torch.empty((M, H // 32), dtype=torch.uint8, device=x.device)
    f = 2.0 * M * N * K
    fused = [Op("fused", "gemm", lambda: m.mx_grouped_gemm_fwd_swiglu(qx, sx, qw, sw, offs, N, y=y, qh=qh, sh=sh), f,
                "")]
    hb = {}
    unfused = [
        Op("fwd", "gemm", lambda: m.mx_grouped_gemm_fwd(qx, sx, qw, sw, offs, N, "bf16", y=y), f, ""),
        Op("act", "quant", lambda: hb.update(h=(torch.nn.functional.silu(y[:, :H].float()) * y[:, H:].float())
                                             .to(torch.bfloat16)), M * N * 2 + M * H * 2, ""),
        Op("quant_h", "quant", lambda: m.mx_quantize_rowwise(hb["h"], qh, sh), M * H * QUANT_BYTES_PER_ELEM, ""),
    ]
    ms_f = time_ops(torch, fused, steps, 2)
    ms_u = time_ops(torch, unfused, steps, 2)
    out = {"layer": lay.name, "fused_ms": round(ms_f, 4), "unfused_ms": round(ms_u, 4),
           "fused_tflops": round(f / (ms_f * 1e-3) / 1e12, 1),
           "unfused_ops": {o.name: op_summary(o) for o in unfused}}
    del y, qh, sh, hb
    torch.cuda.empty_cache()
    return out


def other_configs_leg(m, torch, steps=5, warmup=2):
    """The same MXFP8 fwd+bwd step (dual-layout quantisers, grouped GEMMs fwd/dgrad/wgrad, precise feed)
    on the other two full-size workloads: DeepSeek-V3-16B-shaped layers (64 experts, 49152 routed rows)
    and Llama-4-Scout-shaped layers (16 experts, 32768 rows, top-1).  Reported beside the headline."""
    from workloads import make_workload
    res = {}
    for wname in ("dsv3_16b", "llama4_scout"):
        wl = make_workload(wname)
        dev_ins = [(to_device(torch, lay.x), to_device(torch, lay.w), to_device(torch, lay.dy),
                    to_device(torch, lay.offs)) for lay in wl.layers]
        ops, keep = build_step_ops(m, torch, wl.layers, dev_ins, tiled=STEP_TILED)
        ms = time_ops(torch, ops, steps, warmup)
        gflop = sum(op.work for op in ops if op.kind == "gemm")
        gemm_ms = sum(float(np.mean(op.ms)) for op in ops if op.kind == "gemm")
        q_ms = sum(float(np.mean(op.ms)) for op in ops if op.kind == "quant")
        q_bytes = sum(op.work for op in ops if op.kind == "quant")
        gt = gflop / (gemm_ms * 1e-3) / 1e12
        res[wname] = {
            "layers": {l.name: {"G": l.G, "M": l.M, "N": l.N, "K": l.K} for l in wl.layers},
            "ms_per_step": round(ms, 4), "tflops": round(gflop / (ms * 1e-3) / 1e12, 1),
            "gemm_tflops": round(gt, 1), "gemm_frac_of_bf16_peak": round(gt / MFMA_PEAK_TFLOPS["bf16"], 4),
            "gemm_frac_of_mxfp8_peak": round(gt / MFMA_PEAK_TFLOPS["mxfp8"], 4),
            "quant_gbps": round(q_bytes / (q_ms * 1e-3) / 1e9, 1),
            "ops": {op.name: op_summary(op) for op in ops},
        }
        log(f"{wname}: {ms:.3f} ms/step, GEMMs {gt:.0f} TFLOP/s")
        del ops, keep, wl, dev_ins
        torch.cuda.empty_cache()
    return res


def blockwise_leg(m, torch, steps=5, sample_rows=256):
    """DeepSeek-style blockwise FP8 (1x128 activation tiles, 128x128 weight blocks, 128-token blocks
    for the weight gradient, fp32 scales, promotion every 128), also in its power-of-two scale mode
    (its GEMMs on the MX kernel, the scales folded into the operands), against MXFP8 on the same
    DeepSeek-V3-16B expert-layer tensors: forward, dgrad and wgrad, each recipe with its own
    quantisers.  Accuracy: relative Frobenius error of each recipe's fp32 Y, dX (sampled rows) and dW
    (two experts, sampled n and k) against fp64 products of the original bf16 tensors."""
    from workloads import make_workload
    wl = make_workload("dsv3_16b_blockwise")
    out = {"workload": "dsv3_16b (64 experts, 49152 routed rows)", "layers": {}}
    rng = np.random.default_rng(7)
    for lay in wl.layers:
        G, M, N, K = lay.G, lay.M, lay.N, lay.K
        x, w, dy = to_device(torch, lay.x), to_device(torch, lay.w).view(G * N, K), to_device(torch, lay.dy)
        offs = to_device(torch, lay.offs)
        f = 2.0 * M * N * K
        rec = {}
        # blockwise, with fp32 scales amax / 448 and in the power-of-two scale mode
        ldb = m.fp8bw_colwise_ld_min(M, G)

        def bw_ops(bq, p2):
            return [
                Op("quant_x", "quant", lambda: bq.update(x=m.fp8bw_quantize_act_1x128(x, pow2=p2)),
                   M * K * QUANT_BYTES_PER_ELEM, ""),
                Op("quant_w", "quant", lambda: bq.update(w=m.fp8bw_quantize_weight_128x128(w, transposed=True, pow2=p2)),
                   G * N * K * (QUANT_BYTES_PER_ELEM + 1), ""),
                # power-of-two scales: the GEMMs on the MX kernel (the _pow2 entry points)
                Op("fwd", "gemm", lambda: bq.update(y=(m.fp8bw_grouped_gemm_fwd_pow2 if p2 else m.fp8bw_grouped_gemm_fwd)(
                    *bq["x"], *bq["w"][:2], offs, N, "f32")), f, ""),
                Op("quant_dy", "quant", lambda: bq.update(dy=m.fp8bw_quantize_act_1x128(dy, pow2=p2)),
                   M * N * QUANT_BYTES_PER_ELEM, ""),
                Op("dgrad", "gemm", lambda: bq.update(dx=(m.fp8bw_grouped_gemm_dgrad_pow2 if p2 else m.fp8bw_grouped_gemm_dgrad)(
                    *bq["dy"], bq["w"][2], bq["w"][1], offs, K, "f32")), f, ""),
                Op("quant_dy_col", "quant", lambda: bq.update(dyc=m.fp8bw_quantize_colwise_128(dy, offs, ld=ldb, pow2=p2)),
                   M * N * QUANT_BYTES_PER_ELEM, ""),
                Op("quant_x_col", "quant", lambda: bq.update(xc=m.fp8bw_quantize_colwise_128(x, offs, ld=ldb, pow2=p2)),
                   M * K * QUANT_BYTES_PER_ELEM, ""),
                Op("wgrad", "gemm", lambda: bq.update(dw=(m.fp8bw_grouped_gemm_wgrad_pow2 if p2 else m.fp8bw_grouped_gemm_wgrad)(
                    *bq["dyc"], *bq["xc"], offs, M, "f32")), f, ""),
            ]
        bq, bq2 = {}, {}
        ops_bw, ops_bw2 = bw_ops(bq, False), bw_ops(bq2, True)
        mq = {}
        ld = m.mx_colwise_ld(G * N)
        ldm = m.mx_colwise_ld(M, G)
        ops_mx = [
            Op("quant_x", "quant", lambda: mq.update(x=m.mx_quantize_rowwise(x)), M * K * QUANT_BYTES_PER_ELEM, ""),
            Op("quant_w", "quant", lambda: mq.update(w=m.mx_quantize_rowwise(w)), G * N * K * QUANT_BYTES_PER_ELEM, ""),
            Op("fwd", "gemm", lambda: mq.update(y=m.mx_grouped_gemm_fwd(*mq["x"], *mq["w"], offs, N, "f32")), f, ""),
            Op("quant_dy", "quant", lambda: mq.update(dy=m.mx_quantize_rowwise(dy)), M * N * QUANT_BYTES_PER_ELEM, ""),
            Op("quant_w_col", "quant", lambda: mq.update(wc=m.mx_quantize_colwise(w, None, ld=ld)), G * N * K * QUANT_BYTES_PER_ELEM, ""),
            Op("dgrad", "gemm", lambda: mq.update(dx=m.mx_grouped_gemm_dgrad(*mq["dy"], *mq["wc"], offs, K, "f32")), f, ""),
            Op("quant_dy_col", "quant", lambda: mq.update(dyc=m.mx_quantize_colwise(dy, offs, ld=ldm)),
               M * N * QUANT_BYTES_PER_ELEM, ""),
            Op("quant_x_col", "quant", lambda: mq.update(xc=m.mx_quantize_colwise(x, offs, ld=ldm)),
               M * K * QUANT_BYTES_PER_ELEM, ""),
            Op("wgrad", "gemm", lambda: mq.update(dw=m.mx_grouped_gemm_wgrad(*mq["dyc"], *mq["xc"], offs, M, "f32")),
               f, ""),
        ]
        for name, ops_ in (("blockwise", ops_bw), ("blockwise_pow2", ops_bw2), ("mxfp8", ops_mx)):
            ms = time_ops(torch, ops_, steps, 1)
            gm = sum(float(np.mean(o.ms)) for o in ops_ if o.kind == "gemm")
            rec[name] = {"ms_fwd_bwd_with_quant": round(ms, 4),
                         "gemm_tflops": round(3 * f / (gm * 1e-3) / 1e12, 1),
                         "ops": {o.name: op_summary(o) for o in ops_}}
        # accuracy on sampled rows against fp64 products of the bf16 inputs
        rows = np.sort(rng.choice(M, sample_rows, replace=False))
        grp = np.searchsorted(lay.offs.astype(np.int64), rows, side="right") - 1
        xb = bf16_to_f64(lay.x[rows]); dyb = bf16_to_f64(lay.dy[rows])
        wf = lay.w.reshape(G, N, K)
        y_ref = np.stack([xb[i] @ bf16_to_f64(wf[g]).T for i, g in enumerate(grp)])
        dx_ref = np.stack([dyb[i] @ bf16_to_f64(wf[g]) for i, g in enumerate(grp)])
        for name, q in (("blockwise", bq), ("blockwise_pow2", bq2), ("mxfp8", mq)):
            yg = q["y"][torch.from_numpy(rows).cuda()].double().cpu().numpy()
            dxg = q["dx"][torch.from_numpy(rows).cuda()].double().cpu().numpy()
            rec[name]["rel_fro_err_y"] = float(np.linalg.norm(yg - y_ref) / np.linalg.norm(y_ref))
            rec[name]["rel_fro_err_dx"] = float(np.linalg.norm(dxg - dx_ref) / np.linalg.norm(dx_ref))
        # weight gradient of two sampled experts on sampled (n, k)
        sizes = np.diff(lay.offs.astype(np.int64))
        gs = [int(np.argmax(sizes)), int(rng.choice(np.flatnonzero(sizes > 0)))]
        n_idx = np.sort(rng.choice(N, 64, replace=False))
        k_idx = np.sort(rng.choice(K, 64, replace=False))
        for name, q in (("blockwise", bq), ("blockwise_pow2", bq2), ("mxfp8", mq)):
            num = den = 0.0
            for g in gs:
                r0, r1 = int(lay.offs[g]), int(lay.offs[g + 1])
                ref = bf16_to_f64(lay.dy[r0:r1][:, n_idx]).T @ bf16_to_f64(lay.x[r0:r1][:, k_idx])
                got = q["dw"][g][torch.from_numpy(n_idx).cuda()][:, torch.from_numpy(k_idx).cuda()].double().cpu().numpy()
                num += float(np.sum((got - ref) ** 2))
                den += float(np.sum(ref ** 2))
            rec[name]["rel_fro_err_dw"] = float(np.sqrt(num / den))
        out["layers"][lay.name] = rec
        del x, w, dy, bq, bq2, mq, ops_bw, ops_bw2, ops_mx
        torch.cuda.empty_cache()
    return out


def bf16_to_f64(a: np.ndarray) -> np.ndarray:
    return (np.asarray(a, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


# ------------------------------------------------------------------------------------------- main
def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true", help="skip the CPU oracle timing")
    ap.add_argument("--no-extra-legs", action="store_true",
                    help="skip the FP8-feed and blockwise legs (reported beside the headline)")
    ap.add_argument("--stats-summary", metavar="PROF_DIR",
                    help="write the kernel-statistics summary from a rocprofv3 --kernel-trace --stats run of this script")
    ap.add_argument("--mfma-summary", metavar="PMC_DIR",
                    help="write the GEMM clock / MFMA-use summary from a rocprofv3 --kernel-trace --pmc run of this script")
    ap.add_argument("--pmc-summary", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="write the GEMM and quantiser traffic summaries from two rocprofv3 counter runs of this script")
    ap.add_argument("--workload", default=WORKLOAD, choices=sorted(WORKLOAD_TITLE),
                    help="run the step on another workload (for its profiles; the headline is the default)")
    args = ap.parse_args()
    set_workload(args.workload)

    if args.stats_summary:
        stats_summary(args.stats_summary)
        return

    # (another workload: its own output folders and the --workload argument in every command)
    wl_arg, sfx = ("", "") if WORKLOAD == "dsv3_671b_shard" else (f" --workload {WORKLOAD}", f"_{WORKLOAD}")
    if args.mfma_summary:
        mfma_summary(args.mfma_summary, [
            "rocprofv3 --kernel-trace --pmc " + " ".join(MFMA_COUNTERS) + f" --output-format csv -d gpurun_out/pmc_mfma{sfx} "
            "-o p -- python3 bench.py --steps 1 --warmup 0 --no-cpu-baseline --no-extra-legs" + wl_arg,
            f"python3 bench.py --mfma-summary gpurun_out/pmc_mfma{sfx}{wl_arg}"])
        return

    if args.pmc_summary:
        cmds = [f"rocprofv3 --pmc {c} --output-format csv -d gpurun_out/pmc_{c.lower()}{sfx} -o p -- "
                "python3 bench.py --steps 1 --warmup 0 --no-cpu-baseline --no-extra-legs" + wl_arg
                for c in ("FETCH_SIZE", "WRITE_SIZE")]
        cmds.append(f"python3 bench.py --pmc-summary gpurun_out/pmc_fetch_size{sfx}/p_counter_collection.csv "
                    f"gpurun_out/pmc_write_size{sfx}/p_counter_collection.csv{wl_arg}")
        pmc_summary(args.pmc_summary[0], args.pmc_summary[1], cmds)
        return

    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); "
              "the expert-parallel split across GPUs is a design, not an implementation", file=sys.stderr)
        sys.exit(2)

    import torch
    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)
    import precision_moe_expert_mx_amd as m
    m.lib()                                    # raises if the HIP library is not built

    from workloads import make_workload
    wname = WORKLOAD
    t = time.perf_counter()
    wl = make_workload(wname)
    log(f"workload {wname} generated in {time.perf_counter() - t:.1f} s")

    # plain copy of known size: the calibration point for HBM byte counters
    cal = torch.empty(256 << 20, dtype=torch.float32, device="cuda")
    cal2 = torch.empty_like(cal)
    cal2.copy_(cal)
    torch.cuda.synchronize()
    # its rate (1 GiB read + 1 GiB written) is reported beside the quantisers' rate
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(5):
        cal2.copy_(cal)
    e1.record()
    torch.cuda.synchronize()
    copy_gbps = 2 * 5 * (1 << 30) / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del cal, cal2

    dev_ins = [(to_device(torch, lay.x), to_device(torch, lay.w), to_device(torch, lay.dy),
                to_device(torch, lay.offs)) for lay in wl.layers]
    ops, step_bufs = build_step_ops(m, torch, wl.layers, dev_ins, tiled=STEP_TILED)
    keep = list(zip(dev_ins, step_bufs))
    torch.cuda.synchronize()
    log(f"inputs resident; {torch.cuda.memory_allocated() / 2**30:.1f} GiB allocated")

    ms_step = time_ops(torch, ops, args.steps, args.warmup)
    log(f"timed {args.steps} steps: {ms_step:.3f} ms/step")

    gemm_flops = sum(op.work for op in ops if op.kind == "gemm")
    value = gemm_flops / (ms_step * 1e-3) / 1e12
    per_op = {op.name: op_summary(op) for op in ops}
    gemm_ms = sum(float(np.mean(op.ms)) for op in ops if op.kind == "gemm")
    quant_ms = sum(float(np.mean(op.ms)) for op in ops if op.kind == "quant")
    quant_bytes = sum(op.work for op in ops if op.kind == "quant")

    # dominant kernel: the GEMM op with the largest share of the step
    dom = max((op for op in ops if op.kind == "gemm"), key=lambda o: float(np.mean(o.ms)))
    dom_ms = float(np.mean(dom.ms))
    achieved = dom.work / (dom_ms * 1e-3) / 1e12
    traffic = read_traffic(TRAFFIC_FILE)
    # against the dense MXFP8 MFMA peak that the metric names; the precise feed runs on the bf16 MFMA,
    # whose peak (half of it) is its own ceiling, reported beside it
    roofline = {"bound": "mfma", "achieved": round(achieved, 1), "peak": MFMA_PEAK_TFLOPS["mxfp8"],
                "unit": "TFLOP/s", "frac": round(achieved / MFMA_PEAK_TFLOPS["mxfp8"], 4),
                "traffic": (traffic or {}).get(dom.name), "op": dom.name, "kernel": dom.kernel,
                "flop_per_launch": dom.work, "algorithmic_bytes_per_launch": round(dom.bytes),
                "avg_launch_ms": round(dom_ms, 4),
                "mfma_instruction": "v_mfma_f32_32x32x16_bf16 (E4M3 widened exactly, scale folded in)",
                "frac_of_bf16_peak": round(achieved / MFMA_PEAK_TFLOPS["bf16"], 4)}

    # the HBM-bound side: the longest dual-layout quantiser launch against the HBM peak
    qdom = max((op for op in ops if op.kind == "quant"), key=lambda o: float(np.mean(o.ms)))
    qdom_ms = float(np.mean(qdom.ms))
    qach = qdom.work / (qdom_ms * 1e-3) / 1e9
    qtraffic = read_traffic(QUANT_TRAFFIC_FILE, quant_source_hash())
    quant_roofline = {"bound": "hbm", "achieved": round(qach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                      "frac": round(qach / HBM_PEAK_GBS, 4), "traffic": (qtraffic or {}).get(qdom.name),
                      "op": qdom.name, "kernel": qdom.kernel, "algorithmic_bytes_per_launch": round(qdom.work),
                      "avg_launch_ms": round(qdom_ms, 4)}

    sample = None if args.no_cpu_baseline else gpu_sample(wl.layers[0], keep[0][1])
    extra = {"device_copy_gbps": round(copy_gbps, 1), "quant_frac_of_copy": round(quant_bytes / (quant_ms * 1e-3) / 1e9 / copy_gbps, 3)}
    if not args.no_extra_legs:
        # the same GEMMs on the full-rate block-scaled FP8 MFMA, whose sums are truncated per run of
        # 8 products: reported beside the headline, never as it
        fops = []
        for lay, (dev_in, _) in zip(wl.layers, keep):
            lops, bufs = build_layer_ops(m, torch, lay, dev_in, fast=True)
            fops.append((lops, bufs))
        flat = [op for lops, _ in fops for op in lops]
        for op in flat:                       # quantised operands for the GEMMs
            if op.kind == "quant":
                op.fn()
        g_ops = [op for op in flat if op.kind == "gemm"]
        time_ops(torch, g_ops, 5, 1)
        extra["fp8_feed_gemms"] = {op.name: op_summary(op) for op in g_ops}
        fms = sum(float(np.mean(op.ms)) for op in g_ops)
        extra["fp8_feed_gemm_tflops"] = round(gemm_flops / (fms * 1e-3) / 1e12, 1)
        del fops, flat, g_ops
        torch.cuda.empty_cache()
        # the six separate row-wise / column-wise launches per layer that the dual-layout launches
        # replace (same outputs)
        sops = []
        for lay, (dev_in, _) in zip(wl.layers, keep):
            lops, bufs = build_layer_ops(m, torch, lay, dev_in, fused=False)
            sops.append((lops, bufs))
        q_ops = [op for lops, _ in sops for op in lops if op.kind == "quant"]
        time_ops(torch, q_ops, 5, 1)
        sep_ms = sum(float(np.mean(op.ms)) for op in q_ops)
        extra["separate_quantisers"] = {"ms_per_step": round(sep_ms, 4), "dual_ms_per_step": round(quant_ms, 4),
                                        "ops": {op.name: op_summary(op) for op in q_ops}}
        del sops, q_ops
        torch.cuda.empty_cache()
        extra["mxfp4_step"] = mxfp4_leg(m, torch, wl, keep)
        extra["swiglu_fused_forward"] = swiglu_leg(m, torch, wl.layers[0], keep[0][0])
        del keep, ops
        torch.cuda.empty_cache()
        extra["blockwise_vs_mx"] = blockwise_leg(m, torch)
        extra["other_configs"] = other_configs_leg(m, torch)

    cpu = None
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on a bounded sample ...")
        cpu = cpu_baseline(wl.layers[0], gpu=sample)
        log(f"oracle: {cpu['value']} TFLOP/s in {cpu['seconds']} s")

    out = {
        "metric": "MXFP8 grouped-GEMM TFLOP/s fwd+bwd (% of MFMA peak); quantize GB/s",
        "value": round(value, 1),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "e4m3+e8m0 (bf16 MFMA, fp32 acc)",
        "data": "synthetic",
        "config": {"workload": wname, "experts": wl.layers[0].G, "routed_rows": wl.layers[0].M,
                   "group_sizes": [int(s) for s in wl.layers[0].sizes],
                   "layers": {l.name: {"N": l.N, "K": l.K} for l in wl.layers},
                   "step": "expert MLP fwd+bwd: per layer X, W, dY each quantised to both MX layouts in one launch; "
                           "gate+up forward with SwiGLU and H quantised to both layouts in its epilogue, consumed by "
                           "the down layer; grouped GEMM fwd/dgrad/wgrad of both layers"
                           + ("; column-wise copies in the 128-byte tiled layout" if STEP_TILED else "")},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "quant_roofline": quant_roofline,
        "gemm_only_tflops": round(gemm_flops / (gemm_ms * 1e-3) / 1e12, 1),
        "gemm_frac_of_mxfp8_peak": round(gemm_flops / (gemm_ms * 1e-3) / 1e12 / MFMA_PEAK_TFLOPS["mxfp8"], 4),
        "quant_gbps": round(quant_bytes / (quant_ms * 1e-3) / 1e9, 1),
        "quant_frac_hbm": round(quant_bytes / (quant_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 3),
        "step_gflop": round(gemm_flops / 1e9, 1),
        "ops": per_op,
        "gemm_source_sha256": gemm_source_hash(),
        "host": platform.node(),
    }
    out.update(extra)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
