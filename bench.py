#!/usr/bin/env python3
"""BitLinear forward benchmark on one MI355X.

Headline (`value`): decode packed-weight GB/s of a 2B4T-shaped FFN stack
(gate/up 2560 -> 6912, squared-ReLU gating, down 6912 -> 2560) at M = 1, 4
and 16 tokens. One step runs, for each M and each of L layers, one
bl_ffn_relu2 call: per-token act quant -> gate and up BitLinears ->
relu(gate)^2 * up -> act quant -> down BitLinear (two launches at 1 and 4
tokens, three at 16). The L layers hold distinct copies of the packed weights
(identical content, distinct addresses) whose total exceeds twice the 256 MB
Infinity Cache, so every BitLinear streams its weights from HBM. Weights are
quantised once before the timed region (offline in the method); that pass is
timed and reported separately. The step is captured in a HIP graph and
replayed.

Also reported, each with its roofline (achieved vs. the published peak,
HIP-event timing on the launching stream, HBM bytes per launch from the
committed rocprofv3 counter summary when the kernel sources are unchanged):
  - the decode weight-stream kernel of the headline step;
  - 70B-class decode (8192 -> 28672 and 28672 -> 8192) at M = 1 (GEMV) and
    M = 64 (GEMM), over rotated weight copies;
  - prefill GEMMs: M = 4096 on 2560 <-> 6912 and M = 2048 on the 70B shapes
    (int8 TOPS against the matrix-core peak);
  - one 2560 -> 2560 projection and a 3B-class block (q, k, v, o 3200 ->
    3200; gate, up 3200 -> 8640; down 8640 -> 3200) at M = 1 over rotated
    weight copies, and the 3B block's projections at M = 512;
  - measured ceilings of own-code calibration kernels (a read-only 16-byte
    HBM stream and an int8 matrix-core loop);
  - the CPU oracle timed on a bounded sample of the decode step.

    python bench.py [--steps K] [--warmup W] [--layers L]
"""
from __future__ import annotations

import argparse
import json
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "BitLinear decode packed-weight GB/s (% HBM peak); prefill int8 TOPS (% MFMA)"
HBM_PEAK_GBS = 8000.0       # MI355X HBM3E, published
I8_PEAK_TOPS = 5000.0       # MI355X dense int8 MFMA, published
BF16_PEAK_TFLOPS = 2500.0   # MI355X dense bf16 MFMA, published
DECODE_WORKLOAD = 2         # 2B4T-shaped FFN at decode
PREFILL_WORKLOAD = 3        # one 4096-token sequence
LARGE_WORKLOAD = 5          # 70B-class shapes
LARGE_COPIES = 5            # 5 x 2 x 58.7 MB of packed weights > 2 x 256 MB
SMALL_COPIES = 400          # 400 x 1.64 MB of 2560 x 2560 packed weights
BLOCK3B_COPIES = 20         # 20 x 31.1 MB of 3B-block packed weights
COUNTERS_FILE = os.path.join(ROOT, "profiles", "hbm_traffic_counters.md")


def parse_args():
    p = argparse.ArgumentParser(description=__doc__,
                                formatter_class=argparse.RawDescriptionHelpFormatter)
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--layers", type=int, default=40,
                   help="distinct weight copies per projection (default 40: 531 MB)")
    p.add_argument("--cpu-seconds", type=float, default=12.0,
                   help="CPU-oracle sample budget (0 disables the leg)")
    p.add_argument("--no-prefill", action="store_true")
    p.add_argument("--no-large", action="store_true", help="skip the 70B-class legs")
    p.add_argument("--no-small", action="store_true",
                   help="skip the single-2560 and 3B-block legs")
    p.add_argument("--no-graph", action="store_true", help="time eager launches instead")
    return p.parse_args()


def host_info():
    cpu = platform.processor()
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    cpu = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return cpu, os.cpu_count()


class Timer:
    """Per-launch HIP event pairs on the launching (current) stream."""

    def __init__(self, torch):
        self.torch = torch
        self.pairs = {}

    def run(self, key, fn):
        t = self.torch
        a = t.cuda.Event(enable_timing=True)
        b = t.cuda.Event(enable_timing=True)
        a.record()
        fn()
        b.record()
        self.pairs.setdefault(key, []).append((a, b))

    def total_ms(self, key):
        return sum(a.elapsed_time(b) for a, b in self.pairs.get(key, []))

    def count(self, key):
        return len(self.pairs.get(key, []))


def main():
    args = parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported "
              "(the BitLinear path here runs on a single MI355X)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import ternary_weight_linear_quant_amd as bl
    from ternary_weight_linear_quant_amd import workloads as wl

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    bl.lib()  # fail loudly if the HIP library is missing
    dev = torch.device("cuda:0")
    props = torch.cuda.get_device_properties(dev)

    def bf16_dev(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(dev) \
            .view(torch.bfloat16)

    # ------------------------------------------------ decode workload ----
    _, projs, Ms = wl.WORKLOADS[DECODE_WORKLOAD]
    shapes = {name: (K, N) for name, K, N in projs}
    Wdev = {name: torch.from_numpy(wl.weights(DECODE_WORKLOAD, i, N, K)).to(dev)
            for i, (name, K, N) in enumerate(projs)}

    # Weight preparation (offline): timed once per matrix after a warm call.
    base = {}
    wp_ms = 0.0
    wp_bytes = 0
    for name, W in Wdev.items():
        bl.quantize_weights(W)
        torch.cuda.synchronize()
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        base[name] = bl.quantize_weights(W)
        b.record()
        torch.cuda.synchronize()
        wp_ms += a.elapsed_time(b)
        wp_bytes += W.numel() * 4
    del Wdev

    L = args.layers
    layers = [{name: (pk.clone(), g.clone()) for name, (pk, g) in base.items()}
              for _ in range(L)]
    packed_per_layer = sum(pk.numel() * 4 for pk, _ in base.values())

    Kin, Nff = shapes["gate"]
    bufs = {}
    for M in Ms:
        bufs[M] = dict(
            x=bf16_dev(wl.activations(DECODE_WORKLOAD, 9, M, Kin)),
            y=torch.empty((M, Kin), dtype=torch.float32, device=dev),
            ws=bl.ffn_relu2_workspace(M, Kin, Nff, dev),
        )

    def decode_pass(M):
        """All L layers at one token count: act quant -> gate and up
        BitLinears -> relu(gate)^2 * up -> act quant -> down BitLinear, as one
        bl_ffn_relu2 call per layer (two launches at 1 and 4 tokens, three at
        16: the gate/up launch, an act quant of h, the down GEMV)."""
        B = bufs[M]
        for lay in layers:
            bl.ffn_relu2(B["x"], *lay["gate"], *lay["up"], *lay["down"], workspace=B["ws"],
                         out=B["y"])

    def decode_step():
        for M in Ms:
            decode_pass(M)

    def capture(fn):
        gr = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gr):
            fn()
        torch.cuda.synchronize()
        return gr

    def time_graph(gr, reps):
        gr.replay()
        torch.cuda.synchronize()
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(reps):
            gr.replay()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / reps

    decode_step()
    torch.cuda.synchronize()
    graph = None if args.no_graph else capture(decode_step)

    def replay():
        if graph is not None:
            graph.replay()
        else:
            decode_step()

    for _ in range(args.warmup):
        replay()
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record()
    for _ in range(args.steps):
        replay()
    t1.record()
    torch.cuda.synchronize()
    ms_per_step = t0.elapsed_time(t1) / args.steps
    packed_per_step = packed_per_layer * L * len(Ms)
    value = packed_per_step / (ms_per_step * 1e-3) / 1e9

    from ternary_weight_linear_quant_amd import counters
    traffic = counters.load_traffic(COUNTERS_FILE)

    def replay_stats(gr, reps, launches):
        """Per-launch time (us) of a graph of `launches` kernel launches: mean
        over `reps` replays timed as one, and p10 / median / p90 over replays
        timed one by one (HIP events on the replaying stream)."""
        mean_ms = time_graph(gr, reps)
        per = []
        for _ in range(reps):
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record()
            gr.replay()
            b.record()
            per.append((a, b))
        torch.cuda.synchronize()
        us = sorted(1e3 * a.elapsed_time(b) / launches for a, b in per)
        q = lambda f: us[min(len(us) - 1, int(round(f * (len(us) - 1))))]
        return {"mean_us": round(1e3 * mean_ms / launches, 3), "p10_us": round(q(0.1), 3),
                "median_us": round(q(0.5), 3), "p90_us": round(q(0.9), 3),
                "replays": reps, "launches_per_replay": launches,
                "note": "mean over replays timed as one; percentiles over replays timed one "
                        "by one (each includes its own event overhead)"}

    # Per token count, and the roofline of the weight-streaming kernel: the
    # M = 1 pass is nothing but k_ffn_gemv launches (gate/up + down per
    # layer), replayed from its own HIP graph and timed with HIP events on
    # the replaying stream.
    per_M = {}
    for M in Ms:
        gm = capture(lambda M=M: decode_pass(M))
        ms = time_graph(gm, 5)
        small = M * Kin <= 131072 and M * Nff <= 131072
        launches = (2 if M in (1, 2, 4, 8) else 3 if M == 16 else 4) if small else 4
        per_M[f"M{M}"] = {"ms": round(ms, 4), "launches_per_layer": launches,
                          "packed_GBps": round(packed_per_layer * L / (ms * 1e-3) / 1e9, 1)}
        if M == 1:
            stats1 = replay_stats(gm, 20, 2 * L)
        del gm
    Kd, Nd = shapes["down"]
    M = 1
    bytes_a = 2 * (Nff * Kin // 4 + 4) + 2 * M * Kin + 2 * M * Nff
    bytes_b = Nd * Kd // 4 + 4 + 2 * M * Kd + 4 * M * Nd
    alg_per_launch = (bytes_a + bytes_b) / 2
    achieved = alg_per_launch / (stats1["mean_us"] * 1e-6) / 1e9
    roofline = {
        "bound": "hbm",
        "kernel": "k_ffn_gemv (decode weight stream: gate/up+gating and act-quant+down "
                  "launches of the M=1 pass)",
        "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
        "frac": round(achieved / HBM_PEAK_GBS, 4),
        "traffic": traffic.get("ffn_2b4t_m1"),
        "traffic_unit": "HBM bytes per launch (rocprofv3 FETCH_SIZE + WRITE_SIZE, scaled "
                        "by a copy kernel)",
        "alg_bytes_per_launch": round(alg_per_launch),
        "launches": 2 * L, "avg_us": stats1["mean_us"], "per_launch": stats1,
        "timing": "HIP graph of the M=1 pass (k_ffn_gemv launches only), HIP events on "
                  "the replay stream",
    }
    # The same bytes through a plain 16-byte read stream in the same launch
    # pattern (one launch over the gate+up bytes, one over the down bytes,
    # per layer): the ceiling for launches of this size, where launch latency
    # and not HBM bandwidth dominates.
    sink = torch.zeros(4, dtype=torch.int32, device=dev)
    n_a = bytes_a // 16 * 16
    n_b = bytes_b // 16 * 16
    rbufs = [(torch.empty(n_a // 4, dtype=torch.int32, device=dev),
              torch.empty(n_b // 4, dtype=torch.int32, device=dev)) for _ in range(L)]

    def read_pass():
        for ra, rb in rbufs:
            bl.calib_read(ra, sink)
            bl.calib_read(rb, sink)

    read_pass()
    gr_read = capture(read_pass)
    st_read = replay_stats(gr_read, 20, 2 * L)
    del gr_read, rbufs
    read_gbps = (n_a + n_b) / 2 / (st_read["mean_us"] * 1e-6) / 1e9
    roofline["same_size_read_ceiling"] = {
        "kernel": "k_calib_read", "bytes_per_launch": round((n_a + n_b) / 2),
        "GBps": round(read_gbps, 1), "us_per_launch": st_read["mean_us"],
        "achieved_over_it": round(achieved / read_gbps, 4)}
    used_graph = graph is not None
    del layers, graph
    torch.cuda.empty_cache()
    print(f"decode: {value:.1f} GB/s per step, weight-stream kernel {achieved:.1f} GB/s "
          f"({roofline['avg_us']} us/launch), per M {per_M}", file=sys.stderr, flush=True)

    def prepare(wid, idx, N, K, copies=1):
        W = torch.from_numpy(wl.weights(wid, idx, N, K)).to(dev)
        pk, g = bl.quantize_weights(W)
        del W
        return [(pk, g)] + [(pk.clone(), g.clone()) for _ in range(copies - 1)]

    def gemm_leg(label, wid, M, legs_w, reps):
        """Prefill GEMMs at M tokens: act quant then BitLinear per projection;
        GEMM launches timed one by one with HIP events."""
        legs = []
        for i, (name, K, N) in enumerate(legs_w):
            pk, g = prepare(wid, i, N, K)[0]
            x = bf16_dev(wl.activations(wid, i, M, K))
            xq, xs = bl.quantize_acts(x)
            y = torch.empty((M, N), dtype=torch.float32, device=dev)
            legs.append((name, K, N, x, xq, xs, pk, g, y))

        def step(timer=None):
            for name, K, N, x, xq, xs, pk, g, y in legs:
                if timer is None:
                    bl.quantize_acts(x, out=(xq, xs))
                    bl.bitlinear(xq, xs, pk, g, out=y)
                else:
                    timer.run("act_quant", lambda: bl.quantize_acts(x, out=(xq, xs)))
                    timer.run(("gemm", name), lambda: bl.bitlinear(xq, xs, pk, g, out=y))

        for _ in range(1 + args.warmup):
            step()
        torch.cuda.synchronize()
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(reps):
            step()
        b.record()
        torch.cuda.synchronize()
        p_ms = a.elapsed_time(b) / reps
        ops = sum(2 * M * N * K for _, K, N, *_ in legs)
        tp = Timer(torch)
        for _ in range(reps):
            step(tp)
        torch.cuda.synchronize()
        per = {}
        gemm_ms = 0.0
        for name, K, N, *_ in legs:
            ms = tp.total_ms(("gemm", name))
            n = tp.count(("gemm", name))
            gemm_ms += ms
            per[name] = {"M": M, "K": K, "N": N, "avg_us": round(1e3 * ms / n, 2),
                         "TOPS": round(2 * M * N * K * n / (ms * 1e-3) / 1e12, 1)}
        tops = ops * reps / (gemm_ms * 1e-3) / 1e12
        # Context only: the vendor's plain int8 GEMM on the same shapes
        # (int8 x int8 -> int32, no ternary expansion, no fp32 epilogue).
        vendor_us = {}
        for name, K, N, x, xq, xs, pk, g, y in legs:
            b8 = torch.randint(-1, 2, (K, N), dtype=torch.int8, device=dev)
            torch._int_mm(xq, b8)
            torch.cuda.synchronize()
            ea = torch.cuda.Event(enable_timing=True)
            eb = torch.cuda.Event(enable_timing=True)
            ea.record()
            for _ in range(reps):
                torch._int_mm(xq, b8)
            eb.record()
            torch.cuda.synchronize()
            vendor_us[name] = 1e3 * ea.elapsed_time(eb) / reps
            per[name]["vendor_int8_gemm_us"] = round(vendor_us[name], 2)
            del b8
        vendor_tops = ops / (sum(vendor_us.values()) * 1e-6) / 1e12
        alg = sum(N * K // 4 + 4 + M * K + 4 * M + 4 * M * N for _, K, N, *_ in legs) / len(legs)
        out = {
            "ms_per_step": round(p_ms, 4),
            "step_TOPS": round(ops / (p_ms * 1e-3) / 1e12, 1),
            "roofline": {"bound": "mfma", "kernel": "k_gemm", "achieved": round(tops, 1),
                         "peak": I8_PEAK_TOPS, "unit": "TFLOP/s (int8 TOPS)",
                         "frac": round(tops / I8_PEAK_TOPS, 4),
                         "traffic": traffic.get(label),
                         "traffic_unit": "HBM bytes per bl_bitlinear call",
                         "alg_bytes_per_call": round(alg),
                         "per_projection": per},
            "act_quant_avg_us": round(1e3 * tp.total_ms("act_quant") / tp.count("act_quant"), 2),
            "vendor_int8_gemm": {
                "library": "hipBLASLt through torch._int_mm: int8 x int8 -> int32 on the same "
                           "shapes, without the ternary expansion or the fp32 epilogue "
                           "(context, not a target)",
                "TOPS": round(vendor_tops, 1)},
        }
        del legs
        torch.cuda.empty_cache()
        print(f"{label}: GEMM {tops:.1f} TOPS", file=sys.stderr, flush=True)
        return out

    def rotated_decode(wid, copies):
        """M = 1 BitLinears over `copies` rotated copies of every projection of
        a workload, replayed from one HIP graph: per-launch time and rates."""
        _, wprojs, _ = wl.WORKLOADS[wid]
        w = {name: prepare(wid, i, N, K, copies) for i, (name, K, N) in enumerate(wprojs)}
        io = {}
        for i, (name, K, N) in enumerate(wprojs):
            xq, xs = bl.quantize_acts(bf16_dev(wl.activations(wid, i, 1, K)))
            io[name] = (xq, xs, torch.empty((1, N), dtype=torch.float32, device=dev))

        def rotation():
            for c in range(copies):
                for name, K, N in wprojs:
                    xq, xs, y = io[name]
                    bl.bitlinear(xq, xs, *w[name][c], out=y)

        rotation()
        torch.cuda.synchronize()
        gr = capture(rotation)
        st = replay_stats(gr, 20, copies * len(wprojs))
        del gr, w, io
        torch.cuda.empty_cache()
        t = st["mean_us"] * 1e-6
        packed = sum(N * K // 4 for _, K, N in wprojs) / len(wprojs)
        alg = sum(N * K // 4 + 4 + K + 4 + 4 * N for _, K, N in wprojs) / len(wprojs)
        return {"kernel": "k_gemv", "copies": copies,
                "packed_GBps": round(packed / t / 1e9, 1),
                "roofline": {"bound": "hbm", "achieved": round(alg / t / 1e9, 1),
                             "peak": HBM_PEAK_GBS, "unit": "GB/s",
                             "frac": round(alg / t / 1e9 / HBM_PEAK_GBS, 4),
                             "traffic": traffic.get("gemv_2560_m1" if wid == 1
                                                    else "gemv_3b_m1"),
                             "traffic_unit": "HBM bytes per bl_bitlinear call",
                             "alg_bytes_per_call": round(alg)},
                "per_launch": st,
                "timing": "HIP graph of the rotation, HIP events on the replay stream"}

    # ----------------------- single 2560 projection and the 3B block ----
    small = None
    if not args.no_small:
        small = {"single_2560_decode_M1": rotated_decode(1, SMALL_COPIES)}
        small["single_2560_decode_M1"]["workload"] = "one 2560->2560 projection at M=1"
        small["block_3b_decode_M1"] = rotated_decode(4, BLOCK3B_COPIES)
        small["block_3b_decode_M1"]["workload"] = (
            "3B block at M=1: q, k, v, o 3200->3200; gate, up 3200->8640; down 8640->3200")
        print(f"2560 decode M=1: {small['single_2560_decode_M1']['packed_GBps']} GB/s packed; "
              f"3B block decode M=1: {small['block_3b_decode_M1']['packed_GBps']} GB/s packed",
              file=sys.stderr, flush=True)
        _, p4, _ = wl.WORKLOADS[4]
        small["block_3b_prefill_M512"] = gemm_leg("gemm_3b_m512", 4, 512, p4,
                                                  max(10, args.steps))
        small["block_3b_prefill_M512"]["workload"] = "3B block's seven projections at M=512"

    # ------------------------------------------------ prefill GEMM leg ----
    prefill = None
    if not args.no_prefill:
        _, pprojs, pMs = wl.WORKLOADS[PREFILL_WORKLOAD]
        prefill = {"workload": "prefill_4096 (M=4096; up 2560->6912, down 6912->2560)"}
        prefill.update(gemm_leg("gemm_prefill_4096", PREFILL_WORKLOAD, pMs[0], pprojs,
                                max(5, args.steps)))

    # ------------------------------- straight-through backward (dx) ----
    ste = None
    if not args.no_prefill:
        _, pprojs, pMs = wl.WORKLOADS[PREFILL_WORKLOAD]
        Mp = pMs[0]
        legs = []
        gen = torch.Generator(device=dev)
        gen.manual_seed(2024)
        for i, (name, K, N) in enumerate(pprojs):
            pk, g = prepare(PREFILL_WORKLOAD, i, N, K)[0]
            qT = bl.pack_ste_t(pk, K)
            dy = (torch.randn((Mp, N), generator=gen, device=dev) * 0.01).to(torch.bfloat16)
            dx = torch.empty((Mp, K), dtype=torch.float32, device=dev)
            legs.append((name, K, N, qT, g, dy, dx))
            del pk
        for _ in range(1 + args.warmup):
            for name, K, N, qT, g, dy, dx in legs:
                bl.ste_backward_dx(dy, qT, g, N, out=dx)
        torch.cuda.synchronize()
        tp = Timer(torch)
        reps = max(5, args.steps)
        for _ in range(reps):
            for name, K, N, qT, g, dy, dx in legs:
                tp.run(name, lambda: bl.ste_backward_dx(dy, qT, g, N, out=dx))
        torch.cuda.synchronize()
        per = {}
        tot_ms = 0.0
        flops = 0
        for name, K, N, *_ in legs:
            ms = tp.total_ms(name)
            tot_ms += ms
            flops += 2 * Mp * N * K * reps
            per[name] = {"M": Mp, "N_reduced": N, "K_out": K,
                         "avg_us": round(1e3 * ms / reps, 2),
                         "TFLOPs": round(2 * Mp * N * K * reps / (ms * 1e-3) / 1e12, 1)}
        tf = flops / (tot_ms * 1e-3) / 1e12
        # Context only: the vendor's dense bf16 GEMM dy . W on the same shapes
        # (W as a contiguous bf16 [N][K] matrix of {-1, 0, +1}, bf16 out).
        v_us = 0.0
        for name, K, N, qT, g, dy, dx in legs:
            wb = torch.randint(-1, 2, (N, K), device=dev).to(torch.bfloat16).contiguous()
            torch.matmul(dy, wb)
            torch.cuda.synchronize()
            ea = torch.cuda.Event(enable_timing=True)
            eb = torch.cuda.Event(enable_timing=True)
            ea.record()
            for _ in range(reps):
                torch.matmul(dy, wb)
            eb.record()
            torch.cuda.synchronize()
            us = 1e3 * ea.elapsed_time(eb) / reps
            per[name]["vendor_bf16_gemm_us"] = round(us, 2)
            v_us += us
            del wb
        vendor_tf = flops / reps / (v_us * 1e-6) / 1e12
        ste = {"workload": "dx of the 4096-token projections (dy bf16 [4096][N] -> dx fp32 "
                           "[4096][K]), straight-through estimator",
               "roofline": {"bound": "mfma", "kernel": "k_ste_dx (v_mfma_f32_32x32x16_bf16)",
                            "achieved": round(tf, 1), "peak": BF16_PEAK_TFLOPS,
                            "unit": "TFLOP/s", "frac": round(tf / BF16_PEAK_TFLOPS, 4),
                            "traffic": traffic.get("ste_dx_4096"),
                            "traffic_unit": "HBM bytes per bl_ste_backward_dx call",
                            "per_projection": per},
               "vendor_bf16_gemm": {
                   "library": "hipBLASLt through torch.matmul: dense bf16 x bf16 -> bf16 on "
                              "the same shapes, weights stored as bf16 (context, not a "
                              "target)",
                   "TFLOPs": round(vendor_tf, 1)}}
        del legs
        torch.cuda.empty_cache()
        print(f"ste dx: {tf:.1f} TFLOP/s", file=sys.stderr, flush=True)

    # ------------------------------------------- 70B-class shapes ----
    large = None
    ceilings = None
    if not args.no_large:
        _, lprojs, lMs = wl.WORKLOADS[LARGE_WORKLOAD]
        wts = {name: prepare(LARGE_WORKLOAD, i, N, K, LARGE_COPIES)
               for i, (name, K, N) in enumerate(lprojs)}
        large = {"workload": "70b_class (hidden 8192, FFN 28672; up 8192->28672, "
                             "down 28672->8192)", "weight_copies": LARGE_COPIES}
        for M in (1, 64):
            io = {}
            for i, (name, K, N) in enumerate(lprojs):
                xq, xs = bl.quantize_acts(bf16_dev(wl.activations(LARGE_WORKLOAD, i, M, K)))
                io[name] = (xq, xs, torch.empty((M, N), dtype=torch.float32, device=dev))

            def rotation(M=M, io=io):
                for c in range(LARGE_COPIES):
                    for name, K, N in lprojs:
                        xq, xs, y = io[name]
                        bl.bitlinear(xq, xs, *wts[name][c], out=y)

            rotation()
            torch.cuda.synchronize()
            gr = capture(rotation)
            launches = LARGE_COPIES * len(lprojs)
            st = replay_stats(gr, 20, launches)
            del gr
            packed = sum(N * K // 4 for _, K, N in lprojs) / len(lprojs)
            alg = sum(N * K // 4 + 4 + M * K + 4 * M + 4 * M * N for _, K, N in lprojs) \
                / len(lprojs)
            ops = sum(2 * M * N * K for _, K, N in lprojs) / len(lprojs)
            t = st["mean_us"] * 1e-6
            leg = {
                "kernel": "k_gemv" if M <= 16 else
                          "k_gemm (bl_bitlinear's choice at 64 tokens: four K groups per "
                          "workgroup; the down projection also splits K)",
                "packed_GBps": round(packed / t / 1e9, 1),
                "roofline": {"bound": "hbm", "achieved": round(alg / t / 1e9, 1),
                             "peak": HBM_PEAK_GBS, "unit": "GB/s",
                             "frac": round(alg / t / 1e9 / HBM_PEAK_GBS, 4),
                             "traffic": traffic.get("gemv_70b_m1" if M == 1
                                                    else "decode_70b_m64"),
                             "traffic_unit": "HBM bytes per bl_bitlinear call",
                             "alg_bytes_per_call": round(alg)},
                "per_launch": st,
                "timing": "HIP graph of the rotation (up and down over the weight copies), "
                          "HIP events on the replay stream",
            }
            if M > 16:
                leg["mfma"] = {"achieved_TOPS": round(ops / t / 1e12, 1),
                               "frac": round(ops / t / 1e12 / I8_PEAK_TOPS, 4)}
            large[f"decode_M{M}"] = leg
            print(f"70b decode M={M}: {leg['packed_GBps']} GB/s packed, "
                  f"{st['mean_us']} us/launch", file=sys.stderr, flush=True)

        # The same decode (M = 1) from the denser formats: five ternary weights
        # per byte repacked from the 2-bit copies, and 1-bit binary weights of
        # the same latent matrices.
        io1 = {}
        for i, (name, K, N) in enumerate(lprojs):
            xq, xs = bl.quantize_acts(bf16_dev(wl.activations(LARGE_WORKLOAD, i, 1, K)))
            io1[name] = (xq, xs, torch.empty((1, N), dtype=torch.float32, device=dev))
        fmt_w = {"base3": {name: [(bl.pack_base3(pk, K), g) for pk, g in wts[name]]
                           for name, K, N in lprojs}}
        binw = {}
        for i, (name, K, N) in enumerate(lprojs):
            W = torch.from_numpy(wl.weights(LARGE_WORKLOAD, i, N, K)).to(dev)
            bits, gb = bl.quantize_weights_binary(W)
            del W
            binw[name] = [(bits, gb)] + [(bits.clone(), gb.clone())
                                         for _ in range(LARGE_COPIES - 1)]
        fmt_w["binary"] = binw
        fmt_fn = {"base3": bl.bitlinear_base3, "binary": bl.bitlinear_binary}
        for fmt, wsets in fmt_w.items():
            def rotation_f(fmt=fmt, wsets=wsets):
                for c in range(LARGE_COPIES):
                    for name, K, N in lprojs:
                        xq, xs, y = io1[name]
                        fmt_fn[fmt](xq, xs, *wsets[name][c], out=y)

            rotation_f()
            torch.cuda.synchronize()
            gr = capture(rotation_f)
            st = replay_stats(gr, 20, LARGE_COPIES * len(lprojs))
            del gr
            t = st["mean_us"] * 1e-6
            wbytes = sum(wsets[name][0][0].numel() * wsets[name][0][0].element_size()
                         for name, _, _ in lprojs) / len(lprojs)
            alg = sum(wsets[name][0][0].numel() * wsets[name][0][0].element_size()
                      + 4 + K + 4 + 4 * N for name, K, N in lprojs) / len(lprojs)
            weights = sum(N * K for _, K, N in lprojs) / len(lprojs)
            large[f"decode_M1_{fmt}"] = {
                "kernel": f"k_gemv ({'five ternary weights per byte' if fmt == 'base3' else '1 bit per +-1 weight'})",
                "bits_per_weight": round(8 * wbytes / weights, 4),
                "packed_GBps": round(wbytes / t / 1e9, 1),
                "weights_per_s": round(weights / t / 1e12, 3),
                "weights_unit": "T weights/s",
                "roofline": {"bound": "hbm", "achieved": round(alg / t / 1e9, 1),
                             "peak": HBM_PEAK_GBS, "unit": "GB/s",
                             "frac": round(alg / t / 1e9 / HBM_PEAK_GBS, 4),
                             "traffic": traffic.get(f"gemv_70b_m1_{fmt}"),
                             "traffic_unit": "HBM bytes per launch",
                             "alg_bytes_per_launch": round(alg)},
                "per_launch": st,
            }
            print(f"70b decode M=1 {fmt}: {large[f'decode_M1_{fmt}']['packed_GBps']} GB/s packed, "
                  f"{large[f'decode_M1_{fmt}']['weights_per_s']} T weights/s", file=sys.stderr,
                  flush=True)
        large["decode_M1"]["weights_per_s"] = round(
            sum(N * K for _, K, N in lprojs) / len(lprojs) / (large["decode_M1"]["per_launch"]["mean_us"] * 1e-6) / 1e12, 3)
        del fmt_w, binw, io1

        # Measured ceilings: a read-only 16-byte stream over the same rotated
        # packed weights, and the int8 matrix-core loop.
        sink = torch.zeros(4, dtype=torch.int32, device=dev)
        bufs_r = [w[0] for name in wts for w in wts[name]]

        def read_all():
            for buf in bufs_r:
                bl.calib_read(buf, sink)

        read_all()
        gr = capture(read_all)
        st = replay_stats(gr, 10, len(bufs_r))
        del gr
        nbytes = bufs_r[0].numel() * 4
        msink = bl.calib_mfma_sink(dev)
        iters = 4000
        bl.calib_mfma_i8(iters, msink)
        torch.cuda.synchronize()
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(5):
            mops = bl.calib_mfma_i8(iters, msink)
        b.record()
        torch.cuda.synchronize()
        mfma_tops = mops * 5 / (a.elapsed_time(b) * 1e-3) / 1e12
        ceilings = {
            "hbm_read_stream": {"kernel": "k_calib_read", "bytes_per_launch": nbytes,
                                "GBps": round(nbytes / (st["mean_us"] * 1e-6) / 1e9, 1),
                                "frac_of_peak": round(nbytes / (st["mean_us"] * 1e-6) / 1e9
                                                      / HBM_PEAK_GBS, 4),
                                "per_launch": st},
            "i8_mfma_loop": {"kernel": "k_calib_mfma (v_mfma_i32_32x32x32_i8, 8 waves/CU)",
                             "TOPS": round(mfma_tops, 1),
                             "frac_of_peak": round(mfma_tops / I8_PEAK_TOPS, 4)},
        }
        print(f"ceilings: read {ceilings['hbm_read_stream']['GBps']} GB/s, "
              f"mfma {mfma_tops:.0f} TOPS", file=sys.stderr, flush=True)
        del wts, bufs_r
        torch.cuda.empty_cache()
        large["prefill_M2048"] = gemm_leg("gemm_prefill_70b", LARGE_WORKLOAD, 2048, lprojs,
                                          max(3, args.steps // 4))

    # ------------------------------------------------ CPU oracle leg ----
    cpu_baseline = None
    if args.cpu_seconds > 0:
        import oracle
        codes = {}
        for i, (name, K, N) in enumerate(projs):
            _, g_ref, q_ref = oracle.quantize_weights(wl.weights(DECODE_WORKLOAD, i, N, K))
            codes[name] = (q_ref, g_ref)
        xs_host = {M: wl.activations(DECODE_WORKLOAD, 9, M, Kin) for M in Ms}
        layers_done = 0
        t_start = time.perf_counter()
        while True:
            for M in Ms:
                xq, sc = oracle.act_quant(xs_host[M])
                yg = oracle.epilogue(oracle.int_matmul(xq, codes["gate"][0]), sc, codes["gate"][1])
                yu = oracle.epilogue(oracle.int_matmul(xq, codes["up"][0]), sc, codes["up"][1])
                h = oracle.relu2_glu(yg, yu)
                hq, hs = oracle.act_quant(h)
                oracle.epilogue(oracle.int_matmul(hq, codes["down"][0]), hs, codes["down"][1])
            layers_done += 1
            el = time.perf_counter() - t_start
            if el >= args.cpu_seconds:
                break
        cpu_value = packed_per_layer * len(Ms) * layers_done / el / 1e9
        cpu_baseline = {
            "value": round(cpu_value, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"{layers_done} layer(s) of the decode step (M=1,4,16; gate, up, glue, "
                      f"down; act quant, int matmul, epilogue) in {el:.1f} s, single-threaded "
                      f"C oracle, weights pre-quantised like the GPU step",
        }

    cpu_model, ncpu = host_info()
    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "i8",
        "data": "synthetic",
        "config": {
            "workload": "ffn_2b4t_decode: gate/up 2560->6912, relu^2 gating, down 6912->2560",
            "tokens_per_pass": list(Ms), "layers": L,
            "packed_weight_bytes_per_step": packed_per_step,
            "hip_graph": used_graph,
            "parallelism": "single GPU",
        },
        "frac_hbm_step": round(value / HBM_PEAK_GBS, 4),
        "per_M": per_M,
        "roofline": roofline,
        "cpu_baseline": cpu_baseline,
        "prefill": prefill,
        "ste_backward": ste,
        "large_70b": large,
        "small_configs": small,
        "ceilings": ceilings,
        "weight_prep": {"matrices": list(base), "ms_total": round(wp_ms, 3),
                        "fp32_read_GBps": round(wp_bytes / (wp_ms * 1e-3) / 1e9, 1)},
        "device": {"name": props.name, "cus": props.multi_processor_count,
                   "host_cpu": cpu_model, "host_nproc": ncpu},
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
