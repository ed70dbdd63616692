"""HBM byte counters of the BitLinear kernels, scaled by a plain copy kernel.

Two parts:

``python -m ternary_weight_linear_quant_amd.counters run``
    The workload that ``rocprofv3 --pmc FETCH_SIZE`` and, in a second pass,
    ``rocprofv3 --pmc WRITE_SIZE`` profile: a copy of a known byte count (the
    calibration), then the kernels whose roofline the benchmark reports, each
    phase on the benchmark's shapes and weight rotation. Phases are separated
    by one-block marker copies so every dispatch can be attributed to its
    phase without knowing how many kernels a call launches.

``python -m ternary_weight_linear_quant_amd.counters trace PROF_DIR``
    Formats a ``rocprofv3 --kernel-trace --stats`` run (``*_kernel_stats.csv``
    and ``*_kernel_trace.csv`` under PROF_DIR) as a Markdown table: per kernel
    the call count and average duration, and per launch shape the median,
    p10 and p90.

``python -m ternary_weight_linear_quant_amd.counters busy PASS_DIR``
    Formats one SQ counter pass over the same workload (matrix-core busy
    cycles, VALU, MFMA and LDS instruction counts, LDS bank conflicts) per
    phase and kernel.

``python -m ternary_weight_linear_quant_amd.counters summarize FETCH_DIR WRITE_DIR``
    Reads the two passes' ``*counter_collection.csv``, scales each counter by
    (known bytes / counter reading) of the calibration copy, and prints a
    Markdown summary whose JSON block the benchmark reads: HBM bytes per
    launch per phase, next to the SHA-256 of the sources each phase's kernels
    are built from (a changed source voids the figure).
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "ternary_weight_linear_quant_amd", "csrc")

COPY_BYTES = 256 << 20          # calibration copy size
COPY_CALLS = 3
MARKER_BYTES = 16 * 256         # one block: a marker dispatch
LAYERS_2B4T = 40                # weight copies, as in the benchmark
COPIES_70B = 5                  # 5 x 2 x 58.7 MB > 2 x the 256 MB Infinity Cache
LAYERS_3B = 20                  # 20 x 31.1 MB of 3B-block weights
COPIES_2560 = 400               # 400 x 1.64 MB of 2560 x 2560 weights

# phase label -> (sources its kernels are built from, what the phase runs,
# roofline units in the phase, what one unit is). HBM bytes are reported per
# unit, the unit of the matching roofline in bench.py.
PHASES = {
    "ffn_2b4t_m1": (["ffn.hip", "common.hpp"],
                    "bl_ffn_relu2 at M=1 on 2560->6912->2560 weights, 40 rotated layers",
                    2 * LAYERS_2B4T,
                    "k_ffn_gemv launch (gate/up+gating, or act-quant+down)"),
    "gemv_70b_m1": (["gemv1.hip", "act_quant.hpp", "common.hpp"],
                    "bl_bitlinear at M=1 on 8192->28672 and 28672->8192, 5 rotated copies",
                    2 * COPIES_70B, "one-token GEMV launch (k_gemv1_rows / k_gemv1_stream)"),
    "quant_gemv_70b_m1": (["gemv1.hip", "act_quant.hpp", "common.hpp"],
                          "bl_quant_bitlinear at M=1 on 8192->28672 and 28672->8192 (the "
                          "bf16 token in, its codes and scale out), 5 rotated copies",
                          2 * COPIES_70B,
                          "one-token act quant + GEMV launch (quantising k_gemv1_rows / "
                          "k_gemv1_stream)"),
    "gemv_70b_m1_base3": (["gemv.hip", "common.hpp"],
                          "bl_bitlinear_base3 at M=1 on the 70B shapes, 5 rotated copies",
                          2 * COPIES_70B, "k_gemv launch (five ternary weights per byte)"),
    "gemv_70b_m1_binary": (["gemv.hip", "common.hpp"],
                           "bl_bitlinear_binary at M=1 on the 70B shapes, 5 rotated copies",
                           2 * COPIES_70B, "k_gemv launch (1 bit per +-1 weight)"),
    "decode_70b_m64": (["gemv_wide.hip", "gemm.hip", "common.hpp"],
                       "bl_bitlinear at M=64 on the 70B shapes, 5 rotated copies",
                       2 * COPIES_70B,
                       "bl_bitlinear call (up: k_gemm with two K groups and a 4-deep ring; "
                       "down: the same with split K between k_splitk_zero and "
                       "k_splitk_finalize)"),
    "gemv_2560_m1": (["gemv1.hip", "act_quant.hpp", "common.hpp"],
                     "bl_bitlinear at M=1 on 2560->2560, 400 rotated copies",
                     COPIES_2560, "one-token GEMV launch (k_gemv1_cached)"),
    "gemv_3b_m1": (["gemv1.hip", "act_quant.hpp", "gemv.hip", "common.hpp"],
                   "bl_bitlinear at M=1 on the 3B block (q, k, v, o 3200->3200; gate, up "
                   "3200->8640; down 8640->3200), 20 rotated layers",
                   7 * LAYERS_3B, "bl_bitlinear call (k_gemv1_cached; k_gemv on 8640->3200)"),
    "gemm_3b_m512": (["gemm.hip", "gemv_wide.hip", "common.hpp"],
                     "bl_bitlinear at M=512 on the 3B block's seven projections", 7,
                     "bl_bitlinear call"),
    "gemm_prefill_4096": (["gemm.hip", "common.hpp"],
                          "bl_bitlinear at M=4096 on 2560->6912 and 6912->2560", 2,
                          "bl_bitlinear call (k_gemm)"),
    "ste_dx_4096": (["ste.hip", "common.hpp"],
                    "bl_ste_backward_dx at M=4096 on 2560->6912 and 6912->2560 "
                    "(dy bf16 [4096][N] -> dx fp32 [4096][K])", 2,
                    "bl_ste_backward_dx call (k_ste_dx)"),
    "ste_dw_4096": (["ste_dw.hip", "common.hpp"],
                    "bl_ste_backward_dw at M=4096 on 2560->6912 and 6912->2560 "
                    "(dy bf16 [4096][N], x_q int8 [4096][K] -> dW fp32 [N][K])", 2,
                    "bl_ste_backward_dw call (k_dw_prep_a, k_dw_prep_b, k_ste_dw, k_dw_reduce)"),
    "gemm_prefill_70b": (["gemm.hip", "common.hpp"],
                         "bl_bitlinear at M=2048 on 8192->28672 and 28672->8192", 2,
                         "bl_bitlinear call (k_gemm)"),
}
PHASE_ORDER = ["copy_calibration"] + list(PHASES)


def source_hash(files):
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(f.encode() + b"\0" + fh.read())
    return h.hexdigest()


# ------------------------------------------------------------------ run ----

def run():
    import numpy as np
    import torch

    sys.path.insert(0, ROOT)
    import ternary_weight_linear_quant_amd as bl
    from ternary_weight_linear_quant_amd import workloads as wl

    dev = torch.device("cuda:0")
    bl.lib()

    def bf16(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(dev) \
            .view(torch.bfloat16)

    def weights(wid, idx, N, K, copies):
        W = torch.from_numpy(wl.weights(wid, idx, N, K)).to(dev)
        pk, g = bl.quantize_weights(W)
        del W
        return [(pk.clone(), g.clone()) for _ in range(copies)]

    print("setup", flush=True)
    msrc = torch.zeros(MARKER_BYTES // 4, dtype=torch.int32, device=dev)
    mdst = torch.zeros_like(msrc)
    csrc = torch.ones(COPY_BYTES // 4, dtype=torch.int32, device=dev)
    cdst = torch.zeros_like(csrc)

    _, p2, _ = wl.WORKLOADS[2]
    sh2 = {name: (K, N) for name, K, N in p2}
    w2 = {name: weights(2, i, N, K, LAYERS_2B4T) for i, (name, K, N) in enumerate(p2)}
    Kin, Nff = sh2["gate"]
    x2 = bf16(wl.activations(2, 9, 1, Kin))
    y2 = torch.empty((1, Kin), dtype=torch.float32, device=dev)
    ws2 = bl.ffn_relu2_workspace(1, Kin, Nff, dev)

    _, p5, _ = wl.WORKLOADS[5]
    w5 = {name: weights(5, i, N, K, COPIES_70B) for i, (name, K, N) in enumerate(p5)}
    q5 = {}
    for M in (1, 64, 2048):
        for i, (name, K, N) in enumerate(p5):
            xq, xs = bl.quantize_acts(bf16(wl.activations(5, i, M, K)))
            q5[(M, name)] = (xq, xs, torch.empty((M, N), dtype=torch.float32, device=dev))
    x5 = {}
    for i, (name, K, N) in enumerate(p5):
        x5[name] = (bf16(wl.activations(5, i, 1, K)),
                    torch.empty((1, N), dtype=torch.float32, device=dev),
                    torch.empty((1, K), dtype=torch.int8, device=dev),
                    torch.empty(1, dtype=torch.float32, device=dev))

    w5b3 = {name: [(bl.pack_base3(pk, K), g) for pk, g in w5[name]] for name, K, N in p5}
    w5bin = {}
    for i, (name, K, N) in enumerate(p5):
        W = torch.from_numpy(wl.weights(5, i, N, K)).to(dev)
        bits, gb = bl.quantize_weights_binary(W)
        del W
        w5bin[name] = [(bits.clone(), gb.clone()) for _ in range(COPIES_70B)]

    _, p1, _ = wl.WORKLOADS[1]
    _, K1, N1 = p1[0]
    w1 = weights(1, 0, N1, K1, COPIES_2560)
    xq1, xs1 = bl.quantize_acts(bf16(wl.activations(1, 0, 1, K1)))
    y1 = torch.empty((1, N1), dtype=torch.float32, device=dev)

    _, p4, _ = wl.WORKLOADS[4]
    w4 = {name: weights(4, i, N, K, LAYERS_3B) for i, (name, K, N) in enumerate(p4)}
    q4 = {}
    for M in (1, 512):
        for i, (name, K, N) in enumerate(p4):
            xq, xs = bl.quantize_acts(bf16(wl.activations(4, i, M, K)))
            q4[(M, name)] = (xq, xs, torch.empty((M, N), dtype=torch.float32, device=dev))

    _, p3, M3 = wl.WORKLOADS[3]
    s3 = []
    gen = torch.Generator(device=dev)
    gen.manual_seed(2024)
    for i, (name, K, N) in enumerate(p3):
        pk, g = weights(3, i, N, K, 1)[0]
        dy = (torch.randn((M3[0], N), generator=gen, device=dev) * 0.01).to(torch.bfloat16)
        s3.append((bl.pack_ste_t(pk, K), g, dy,
                   torch.empty((M3[0], K), dtype=torch.float32, device=dev), N))
        del pk
    d3 = []
    for i, (name, K, N) in enumerate(p3):
        xq, xs = bl.quantize_acts(bf16(wl.activations(3, i, M3[0], K)))
        d3.append((s3[i][2], xq, xs, bl.ste_dw_workspace(M3[0], N, K, dev),
                   torch.empty((N, K), dtype=torch.float32, device=dev)))
    q3 = []
    for i, (name, K, N) in enumerate(p3):
        pk, g = weights(3, i, N, K, 1)[0]
        xq, xs = bl.quantize_acts(bf16(wl.activations(3, i, M3[0], K)))
        q3.append((xq, xs, pk, g, torch.empty((M3[0], N), dtype=torch.float32, device=dev)))
    torch.cuda.synchronize()

    def marker():
        torch.cuda.synchronize()
        bl.calib_copy(mdst, msrc)
        torch.cuda.synchronize()

    def phase(name, fn):
        marker()
        fn()
        torch.cuda.synchronize()
        print("phase", name, flush=True)

    def copy_cal():
        for _ in range(COPY_CALLS):
            bl.calib_copy(cdst, csrc)

    def ffn():
        for lay in range(LAYERS_2B4T):
            bl.ffn_relu2(x2, *w2["gate"][lay], *w2["up"][lay], *w2["down"][lay],
                         workspace=ws2, out=y2)

    def rotate70(M):
        def fn():
            for c in range(COPIES_70B):
                for name, _, _ in p5:
                    xq, xs, y = q5[(M, name)]
                    bl.bitlinear(xq, xs, *w5[name][c], out=y)
        return fn

    def rotate70_quant():
        for c in range(COPIES_70B):
            for name, _, _ in p5:
                x, y, xq, xs = x5[name]
                bl.quant_bitlinear(x, *w5[name][c], out=(y, xq, xs))

    def rotate70_fmt(fn, wset):
        def run_fmt():
            for c in range(COPIES_70B):
                for name, _, _ in p5:
                    xq, xs, y = q5[(1, name)]
                    fn(xq, xs, *wset[name][c], out=y)
        return run_fmt

    def single2560():
        for c in range(COPIES_2560):
            bl.bitlinear(xq1, xs1, *w1[c], out=y1)

    def block3b(M):
        def fn():
            for c in range(LAYERS_3B if M == 1 else 1):
                for name, _, _ in p4:
                    xq, xs, y = q4[(M, name)]
                    bl.bitlinear(xq, xs, *w4[name][c], out=y)
        return fn

    def ste4096():
        for qT, g, dy, dx, N in s3:
            bl.ste_backward_dx(dy, qT, g, N, out=dx)

    def ste_dw4096():
        for dy, xq, xs, ws, dW in d3:
            bl.ste_backward_dw(dy, xq, xs, workspace=ws, out=dW)

    def prefill4096():
        for xq, xs, pk, g, y in q3:
            bl.bitlinear(xq, xs, pk, g, out=y)

    def prefill70():
        for name, _, _ in p5:
            xq, xs, y = q5[(2048, name)]
            bl.bitlinear(xq, xs, *w5[name][0], out=y)

    phase("copy_calibration", copy_cal)
    phase("ffn_2b4t_m1", ffn)
    phase("gemv_70b_m1", rotate70(1))
    phase("quant_gemv_70b_m1", rotate70_quant)
    phase("gemv_70b_m1_base3", rotate70_fmt(bl.bitlinear_base3, w5b3))
    phase("gemv_70b_m1_binary", rotate70_fmt(bl.bitlinear_binary, w5bin))
    phase("decode_70b_m64", rotate70(64))
    phase("gemv_2560_m1", single2560)
    phase("gemv_3b_m1", block3b(1))
    phase("gemm_3b_m512", block3b(512))
    phase("gemm_prefill_4096", prefill4096)
    phase("ste_dx_4096", ste4096)
    phase("ste_dw_4096", ste_dw4096)
    phase("gemm_prefill_70b", prefill70)
    marker()
    print("done", flush=True)


# ------------------------------------------------------------ summarize ----

def _read_pass(d, counter):
    """Library dispatches of one pass, in dispatch order: (name, grid, value)."""
    files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no counter_collection.csv under {d}")
    rows = {}
    for f in files:
        with open(f, newline="") as fh:
            for r in csv.DictReader(fh):
                name = r["Kernel_Name"]
                if name.startswith("void "):      # templates demangle with a return type
                    name = name[5:]
                if r["Counter_Name"] != counter or not name.startswith("bl::"):
                    continue
                key = (int(r["Process_Id"]), int(r["Dispatch_Id"]))
                rows[key] = (name, int(r["Grid_Size"]), float(r["Counter_Value"]))
    return [rows[k] for k in sorted(rows)]


def _phases(disp):
    """Split dispatches at the one-block marker copies."""
    out, cur = [], None
    for name, grid, val in disp:
        if name.startswith("bl::k_calib_copy") and grid <= 256:
            if cur is not None:
                out.append(cur)
            cur = []
        elif cur is not None:
            cur.append((name, grid, val))
    if len(out) != len(PHASE_ORDER):
        raise SystemExit(f"expected {len(PHASE_ORDER)} phases, found {len(out)}")
    return dict(zip(PHASE_ORDER, out))


def _short(name):
    return name.split("(")[0].replace("bl::", "")


def summarize(fetch_dir, write_dir, cmd_fetch, cmd_write):
    fetch = _phases(_read_pass(fetch_dir, "FETCH_SIZE"))
    write = _phases(_read_pass(write_dir, "WRITE_SIZE"))
    cal_f = [v for _, _, v in fetch["copy_calibration"]]
    cal_w = [v for _, _, v in write["copy_calibration"]]
    known_kib = COPY_BYTES / 1024
    f_fetch = known_kib / (sum(cal_f) / len(cal_f))
    f_write = known_kib / (sum(cal_w) / len(cal_w))
    result = {
        "calibration": {"kernel": "k_calib_copy", "bytes": COPY_BYTES, "calls": COPY_CALLS,
                        "fetch_kib_avg": round(sum(cal_f) / len(cal_f), 1),
                        "write_kib_avg": round(sum(cal_w) / len(cal_w), 1),
                        "fetch_factor": round(f_fetch, 5), "write_factor": round(f_write, 5)},
        "phases": {},
    }
    lines = [
        "# HBM traffic of the BitLinear kernels (rocprofv3 FETCH_SIZE / WRITE_SIZE)",
        "",
        "Commands (from the repository root, one pass each):",
        "",
        "```",
        cmd_fetch,
        cmd_write,
        f"python -m ternary_weight_linear_quant_amd.counters summarize {fetch_dir} {write_dir}",
        "```",
        "",
        f"Calibration: k_calib_copy of {COPY_BYTES} B read {result['calibration']['fetch_kib_avg']} "
        f"KiB (FETCH_SIZE) and wrote {result['calibration']['write_kib_avg']} KiB (WRITE_SIZE) per "
        f"dispatch against {known_kib:.0f} KiB moved each way, so the readings below are scaled by "
        f"{f_fetch:.4f} (fetch) and {f_write:.4f} (write).",
        "",
        "| phase | kernel | dispatches | FETCH KiB/disp | WRITE KiB/disp | scaled HBM bytes/disp |",
        "|---|---|---|---|---|---|",
    ]
    for label in PHASES:
        files, what, units, unit = PHASES[label]
        fd, wd = fetch[label], write[label]
        if len(fd) != len(wd):
            raise SystemExit(f"{label}: {len(fd)} fetch vs {len(wd)} write dispatches")
        per = {}
        for (n, _, fv), (_, _, wv) in zip(fd, wd):
            e = per.setdefault(_short(n), [0, 0.0, 0.0])
            e[0] += 1
            e[1] += fv
            e[2] += wv
        tot_f = sum(v for _, _, v in fd)
        tot_w = sum(v for _, _, v in wd)
        traffic = (tot_f * f_fetch + tot_w * f_write) * 1024 / units
        for k, (c, fv, wv) in per.items():
            lines.append(f"| {label} | {k} | {c} | {fv / c:.1f} | {wv / c:.1f} | "
                         f"{(fv * f_fetch + wv * f_write) * 1024 / c:.0f} |")
        result["phases"][label] = {
            "what": what, "dispatches": len(fd), "units": units, "unit": unit,
            "kernels": {k: {"dispatches": c, "fetch_kib": round(fv / c, 1),
                            "write_kib": round(wv / c, 1)} for k, (c, fv, wv) in per.items()},
            "traffic_bytes_per_unit": round(traffic),
            "sources": files, "source_sha256": source_hash(files),
        }
    lines += ["", "| phase | roofline unit | units | scaled HBM bytes per unit |", "|---|---|---|---|"]
    for label, ph in result["phases"].items():
        lines.append(f"| {label} | {ph['unit']} | {ph['units']} | {ph['traffic_bytes_per_unit']} |")
    lines += ["", "Machine-readable (read by bench.py; a figure is void once the hash of "
              "its sources differs):", "", "```json", json.dumps(result, indent=1), "```", ""]
    return "\n".join(lines)


BUSY_COUNTERS = ("SQ_VALU_MFMA_BUSY_CYCLES", "SQ_INSTS_MFMA", "SQ_INSTS_VALU",
                 "SQ_ACTIVE_INST_VALU", "SQ_INSTS_LDS", "SQ_LDS_BANK_CONFLICT",
                 "SQ_WAVE_CYCLES", "SQ_BUSY_CU_CYCLES", "GRBM_GUI_ACTIVE")
SIMDS, XCDS = 1024, 8


def _read_all(d):
    """Library dispatches of one pass with every counter it collected:
    (name, grid, {counter: value}) in dispatch order."""
    files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no counter_collection.csv under {d}")
    rows = {}
    for f in files:
        with open(f, newline="") as fh:
            for r in csv.DictReader(fh):
                name = r["Kernel_Name"]
                if name.startswith("void "):
                    name = name[5:]
                if not name.startswith("bl::"):
                    continue
                key = (int(r["Process_Id"]), int(r["Dispatch_Id"]))
                ent = rows.setdefault(key, (name, int(r["Grid_Size"]), {}))
                ent[2][r["Counter_Name"]] = float(r["Counter_Value"])
    return [rows[k] for k in sorted(rows)]


def busy(pass_dir, cmd):
    """Matrix-core and VALU evidence per phase and kernel from one SQ pass.

    SQ_VALU_MFMA_BUSY_CYCLES sums the matrix-core cycles of every MFMA issued
    (over all 1024 SIMDs); GRBM_GUI_ACTIVE sums the busy cycles of the 8 XCDs.
    MFMA busy = (MFMA cycles per SIMD) / (active cycles per XCD), at whatever
    clock the part ran."""
    phases = _phases(_read_all(pass_dir))
    lines = ["# Matrix-core and VALU counters of the BitLinear kernels (rocprofv3 SQ pass)", "",
             "Command (from the repository root, one pass):", "", "```", cmd,
             "python -m ternary_weight_linear_quant_amd.counters busy gpurun_out/pmc_busy",
             "```", "",
             "Per dispatch means. MFMA busy = (SQ_VALU_MFMA_BUSY_CYCLES / 1024 SIMDs) / "
             "(GRBM_GUI_ACTIVE / 8 XCDs): the share of the kernel's active cycles in which an "
             "average SIMD's matrix core works. VALU/MFMA = SQ_INSTS_VALU / SQ_INSTS_MFMA "
             "(wave instructions; gfx950 co-issues VALU work beside MFMAs of other waves).", "",
             "| phase | kernel | dispatches | MFMA busy | VALU/MFMA | VALU insts | MFMA insts "
             "| LDS insts | LDS bank conflicts | active cycles per XCD |",
             "|---|---|---|---|---|---|---|---|---|---|"]
    for ph in PHASE_ORDER:
        by = {}
        for name, _grid, vals in phases[ph]:
            by.setdefault(_short(name), []).append(vals)
        for kern, vs in by.items():
            mean = {c: sum(v.get(c, 0.0) for v in vs) / len(vs) for c in BUSY_COUNTERS}
            act = mean["GRBM_GUI_ACTIVE"] / XCDS
            mb = (mean["SQ_VALU_MFMA_BUSY_CYCLES"] / SIMDS) / act if act else 0.0
            vpm = (mean["SQ_INSTS_VALU"] / mean["SQ_INSTS_MFMA"]
                   if mean["SQ_INSTS_MFMA"] else float("nan"))
            lines.append(f"| {ph} | {kern} | {len(vs)} | {100 * mb:.1f}% | {vpm:.2f} | "
                         f"{mean['SQ_INSTS_VALU']:.0f} | {mean['SQ_INSTS_MFMA']:.0f} | "
                         f"{mean['SQ_INSTS_LDS']:.0f} | {mean['SQ_LDS_BANK_CONFLICT']:.0f} | "
                         f"{act:.0f} |")
    return "\n".join(lines) + "\n"


def trace(prof_dir, cmd, desc):
    def one(pattern):
        f = glob.glob(os.path.join(prof_dir, "**", pattern), recursive=True)
        if not f:
            raise SystemExit(f"no {pattern} under {prof_dir}")
        with open(f[0], newline="") as fh:
            return list(csv.DictReader(fh))
    stats, tr = one("*kernel_stats.csv"), one("*kernel_trace.csv")
    lines = [f"# rocprofv3 kernel statistics: {desc}", "",
             "Command (from the repository root, one MI355X):", "", "```", cmd,
             f"python -m ternary_weight_linear_quant_amd.counters trace {prof_dir}", "```", "",
             "Durations exclude launch gaps; the profiler serialises dispatches.", "",
             "| kernel | calls | avg us | min us | max us | % time |", "|---|---|---|---|---|---|"]
    for r in stats:
        lines.append(f"| `{r['Name'].split('(')[0]}` | {r['Calls']} | "
                     f"{float(r['AverageNs']) / 1e3:.2f} | {float(r['MinNs']) / 1e3:.2f} | "
                     f"{float(r['MaxNs']) / 1e3:.2f} | {float(r['Percentage']):.1f} |")
    per = {}
    for r in tr:
        n = r["Kernel_Name"].split("(")[0]
        if "bl::" not in n:
            continue
        wg = int(r["Grid_Size_X"]) // max(1, int(r["Workgroup_Size_X"]))
        per.setdefault((n, wg), []).append(
            (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    lines += ["", "Per launch shape (workgroups per launch):", "",
              "| kernel | workgroups | launches | median us | p10 us | p90 us |",
              "|---|---|---|---|---|---|"]
    for (n, wg), v in sorted(per.items()):
        v = sorted(v)
        lines.append(f"| `{n}` | {wg} | {len(v)} | {v[len(v) // 2]:.2f} | "
                     f"{v[len(v) // 10]:.2f} | {v[9 * len(v) // 10]:.2f} |")
    return "\n".join(lines) + "\n"


def load_traffic(path):
    """{phase: bytes per launch} for the phases whose sources are unchanged."""
    try:
        text = open(path).read()
    except OSError:
        return {}
    try:
        block = text.split("```json", 1)[1].split("```", 1)[0]
        data = json.loads(block)
    except (IndexError, ValueError):
        return {}
    out = {}
    for label, ph in data.get("phases", {}).items():
        try:
            if source_hash(ph["sources"]) == ph["source_sha256"]:
                out[label] = ph["traffic_bytes_per_unit"]
        except (OSError, KeyError):
            continue
    return out


def main():
    ap = argparse.ArgumentParser(description=__doc__,
                                 formatter_class=argparse.RawDescriptionHelpFormatter)
    sub = ap.add_subparsers(dest="cmd", required=True)
    sub.add_parser("run")
    t = sub.add_parser("trace")
    t.add_argument("prof_dir")
    t.add_argument("--cmd", dest="trace_cmd", default="rocprofv3 --kernel-trace --stats -d <PROF_DIR> -o bench "
                   "--output-format csv -- python3 bench.py --cpu-seconds 0")
    t.add_argument("--desc", default="bench.py, all legs")
    s = sub.add_parser("summarize")
    s.add_argument("fetch_dir")
    s.add_argument("write_dir")
    s.add_argument("--cmd-fetch", default="rocprofv3 --pmc FETCH_SIZE --output-format csv "
                   "-d <FETCH_DIR> -- python3 -m ternary_weight_linear_quant_amd.counters run")
    s.add_argument("--cmd-write", default="rocprofv3 --pmc WRITE_SIZE --output-format csv "
                   "-d <WRITE_DIR> -- python3 -m ternary_weight_linear_quant_amd.counters run")
    b = sub.add_parser("busy")
    b.add_argument("pass_dir")
    b.add_argument("--cmd", dest="busy_cmd", default="rocprofv3 --pmc " + " ".join(BUSY_COUNTERS)
                   + " --output-format csv -d <PASS_DIR> -- python3 -m "
                   "ternary_weight_linear_quant_amd.counters run")
    a = ap.parse_args()
    if a.cmd == "run":
        run()
    elif a.cmd == "busy":
        print(busy(a.pass_dir, a.busy_cmd), end="")
    elif a.cmd == "trace":
        print(trace(a.prof_dir, a.trace_cmd, a.desc), end="")
    else:
        print(summarize(a.fetch_dir, a.write_dir, a.cmd_fetch, a.cmd_write))


if __name__ == "__main__":
    main()
