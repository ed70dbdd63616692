#!/usr/bin/env python3
"""BitLinear forward benchmark on one MI355X.

Headline (`value`): decode packed-weight GB/s on the 70B-class shapes (hidden
8192, FFN 28672: up 8192 -> 28672, down 28672 -> 8192), the largest workload
that fits one GPU, at one token. One step runs, for each of L weight copies
(identical content at distinct addresses, 5 x 2 x 58.7 MB: more than twice the
256 MB Infinity Cache, so every call streams its weights from HBM): the
per-token act quant of the up input with the up BitLinear, then the act quant
of the down input with the down BitLinear, each pair one bl_quant_bitlinear
call -- one launch per projection, which also writes the codes and the scale
(`two_call_step`: the same with bl_quantize_acts + bl_bitlinear). Weights are
quantised once before the timed region (offline in the method); that pass is
timed and reported as weight_prep. The step is captured in a HIP graph and
replayed.

Beside it, each with its roofline (achieved against the published peak,
HIP-event timing on the launching stream, HBM bytes per launch from the
committed rocprofv3 counter summary while the kernel sources are unchanged):
  - `roofline`: the step's launches (act quant + GEMV in one kernel), and
    under `gemv_alone` the one-token GEMV on the quantised token;
  - `prefill_M2048`: act quant + GEMM at 2048 tokens on the same matrices
    (int8 TOPS against the matrix-core peak);
  - decode at 64 tokens, and the 1-bit and base-3 weight formats at one token;
  - the 2B4T FFN decode step at 1, 4 and 16 tokens, the 4096-token prefill,
    one 2560 -> 2560 projection and the 3B block at 1 and 512 tokens, the
    straight-through backward;
  - measured ceilings of own-code calibration kernels (a read-only HBM
    stream, an int8 matrix-core loop);
  - `cpu_baseline`: the CPU oracle on the 70B-class shapes, on one core, on a
    bounded sample (per-step times, decode GB/s, prefill GOPS).

    python bench.py [--steps K] [--warmup W] [--copies L]
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
HEADLINE_WORKLOAD = 5       # 70B-class shapes
DECODE_WORKLOAD = 2         # 2B4T-shaped FFN at decode
PREFILL_WORKLOAD = 3        # one 4096-token sequence
LARGE_COPIES = 5            # 5 x 2 x 58.7 MB of packed weights > 2 x 256 MB
FFN_LAYERS = 40             # 40 x 13.3 MB of 2B4T FFN weights
SMALL_COPIES = 400          # 400 x 1.64 MB of 2560 x 2560 packed weights
BLOCK3B_COPIES = 20         # 20 x 31.1 MB of 3B-block packed weights
GRAPH_CALLS = 4             # back-to-back calls per graph in the prefill legs
COUNTERS_FILE = os.path.join(ROOT, "profiles", "hbm_traffic_counters.md")


def parse_args():
    p = argparse.ArgumentParser(description=__doc__,
                                formatter_class=argparse.RawDescriptionHelpFormatter)
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--copies", type=int, default=LARGE_COPIES,
                   help="weight copies per 70B-class projection in the headline step "
                        "(default 5: 587 MB)")
    p.add_argument("--cpu-seconds", type=float, default=3.0,
                   help="CPU-oracle decode sample budget (0 disables the CPU leg)")
    p.add_argument("--no-extra", action="store_true",
                   help="only the headline step, its roofline and the 2048-token prefill")
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


# Untimed work before each timed region. Between legs the host prepares
# inputs and the GPU idles; its clocks then need 15-30 ms of continuous work
# to come back (replays of the 70B step right after an idle ran 15-17.5 us per
# projection for about 12 ms, then 13.8-14.1), far more than a few warm-up
# steps of a sub-millisecond step cover.
SETTLE_MS = 50.0


def settle(torch, fn, min_ms=SETTLE_MS):
    """Runs fn, untimed, until the GPU has been kept busy for min_ms of wall
    time (checked after every fourth call)."""
    t0 = time.perf_counter()
    fn()
    torch.cuda.synchronize()
    while (time.perf_counter() - t0) * 1e3 < min_ms:
        for _ in range(4):
            fn()
        torch.cuda.synchronize()


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


def other_workloads(args, bl, wl, np, torch, dev, bf16_dev, capture, time_graph,
                    replay_stats, prepare, gemm_leg, traffic, sink):
    """The other workloads' legs (extra keys of the JSON line): the 2B4T FFN
    decode step, the 4096-token prefill, the straight-through backward, one
    2560 -> 2560 projection and the 3B block."""
    out = {}

    # ------------------------------- 2B4T FFN decode step (M = 1, 4, 16) ----
    _, projs, Ms = wl.WORKLOADS[DECODE_WORKLOAD]
    shapes = {name: (K, N) for name, K, N in projs}
    base = {name: prepare(DECODE_WORKLOAD, i, N, K)[0] for i, (name, K, N) in enumerate(projs)}
    layers = [{name: (pk.clone(), g.clone()) for name, (pk, g) in base.items()}
              for _ in range(FFN_LAYERS)]
    packed_per_layer = sum(pk.numel() * 4 for pk, _ in base.values())
    Kin, Nff = shapes["gate"]
    bufs = {M: dict(x=bf16_dev(wl.activations(DECODE_WORKLOAD, 9, M, Kin)),
                    y=torch.empty((M, Kin), dtype=torch.float32, device=dev),
                    ws=bl.ffn_relu2_workspace(M, Kin, Nff, dev)) for M in Ms}

    def decode_pass(M):
        B = bufs[M]
        for lay in layers:
            bl.ffn_relu2(B["x"], *lay["gate"], *lay["up"], *lay["down"], workspace=B["ws"],
                         out=B["y"])

    def ffn_step():
        for M in Ms:
            decode_pass(M)

    ffn_step()
    torch.cuda.synchronize()
    gs = capture(ffn_step)
    ms_step = time_graph(gs, max(5, args.steps))
    del gs
    per_M = {}
    for M in Ms:
        gm = capture(lambda M=M: decode_pass(M))
        ms = time_graph(gm, 5)
        small = M * Kin <= 131072 and M * Nff <= 131072
        launches = (2 if M in (1, 2, 4, 8) else 3 if M == 16 else 4) if small else 4
        per_M[f"M{M}"] = {"ms": round(ms, 4), "launches_per_layer": launches,
                          "packed_GBps": round(packed_per_layer * FFN_LAYERS / (ms * 1e-3) / 1e9, 1)}
        if M == 1:
            stats1 = replay_stats(gm, 20, 2 * FFN_LAYERS)
        del gm
    Kd, Nd = shapes["down"]
    bytes_a = 2 * (Nff * Kin // 4 + 4) + 2 * Kin + 2 * Nff
    bytes_b = Nd * Kd // 4 + 4 + 2 * Kd + 4 * Nd
    alg_per_launch = (bytes_a + bytes_b) / 2
    achieved = alg_per_launch / (stats1["mean_us"] * 1e-6) / 1e9
    out["ffn_2b4t_decode"] = {
        "workload": "2B4T FFN decode step: gate/up 2560->6912, relu^2 gating, down "
                    "6912->2560, one bl_ffn_relu2 call per layer at M = 1, 4, 16",
        "layers": FFN_LAYERS, "ms_per_step": round(ms_step, 4),
        "packed_GBps": round(packed_per_layer * FFN_LAYERS * len(Ms) / (ms_step * 1e-3) / 1e9, 1),
        "per_M": per_M,
        "roofline": {"bound": "hbm", "kernel": "k_ffn_gemv (gate/up+gating and "
                     "act-quant+down launches of the M=1 pass)",
                     "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic.get("ffn_2b4t_m1"),
                     "traffic_unit": "HBM bytes per launch",
                     "alg_bytes_per_launch": round(alg_per_launch), "per_launch": stats1},
    }
    del layers, base, bufs
    torch.cuda.empty_cache()
    print(f"2b4t ffn decode: {out['ffn_2b4t_decode']['packed_GBps']} GB/s per step",
          file=sys.stderr, flush=True)

    # ---------------------------------------------- 4096-token prefill ----
    _, pprojs, pMs = wl.WORKLOADS[PREFILL_WORKLOAD]
    out["prefill_4096"] = {"workload": "prefill_4096 (M=4096; up 2560->6912, down 6912->2560)"}
    out["prefill_4096"].update(gemm_leg("gemm_prefill_4096", PREFILL_WORKLOAD, pMs[0], pprojs,
                                        max(5, args.steps)))

    # ------------------------------- straight-through backward (dx) ----
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
    def dx_all():
        for name, K, N, qT, g, dy, dx in legs:
            bl.ste_backward_dx(dy, qT, g, N, out=dx)

    settle(torch, dx_all)
    for _ in range(1 + args.warmup):
        dx_all()
    torch.cuda.synchronize()
    tp = Timer(torch)
    reps = max(5, args.steps)
    for _ in range(reps):
        for name, K, N, qT, g, dy, dx in legs:
            tp.run(name, lambda: bl.ste_backward_dx(dy, qT, g, N, out=dx))
    torch.cuda.synchronize()
    per, tot_ms, flops = {}, 0.0, 0
    for name, K, N, *_ in legs:
        ms = tp.total_ms(name)
        tot_ms += ms
        flops += 2 * Mp * N * K * reps
        per[name] = {"M": Mp, "N_reduced": N, "K_out": K, "avg_us": round(1e3 * ms / reps, 2),
                     "TFLOPs": round(2 * Mp * N * K * reps / (ms * 1e-3) / 1e12, 1)}
    tf = flops / (tot_ms * 1e-3) / 1e12
    v_us = 0.0
    for name, K, N, qT, g, dy, dx in legs:
        wb = torch.randint(-1, 2, (N, K), device=dev).to(torch.bfloat16).contiguous()
        settle(torch, lambda: torch.matmul(dy, wb))
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
    # dW = dy^T . (x_q * x_scale) on the same shapes: two transposing prep
    # launches and the bf16 GEMM per call.
    dw_legs = []
    for i, (name, K, N) in enumerate(pprojs):
        dy = legs[i][5]
        xq, xs = bl.quantize_acts(bf16_dev(wl.activations(PREFILL_WORKLOAD, i, Mp, K)))
        dw_legs.append((name, K, N, dy, xq, xs, bl.ste_dw_workspace(Mp, N, K, dev),
                        torch.empty((N, K), dtype=torch.float32, device=dev)))
    def dw_all():
        for name, K, N, dy, xq, xs, ws, dW in dw_legs:
            bl.ste_backward_dw(dy, xq, xs, workspace=ws, out=dW)

    settle(torch, dw_all)
    for _ in range(1 + args.warmup):
        dw_all()
    torch.cuda.synchronize()
    tw = Timer(torch)
    for _ in range(reps):
        for name, K, N, dy, xq, xs, ws, dW in dw_legs:
            tw.run(name, lambda: bl.ste_backward_dw(dy, xq, xs, workspace=ws, out=dW))
    torch.cuda.synchronize()
    per_dw, dw_ms = {}, 0.0
    for name, K, N, *_ in dw_legs:
        ms = tw.total_ms(name)
        dw_ms += ms
        per_dw[name] = {"M_reduced": Mp, "N": N, "K": K, "avg_us": round(1e3 * ms / reps, 2),
                        "TFLOPs": round(2 * Mp * N * K * reps / (ms * 1e-3) / 1e12, 1)}
    tf_dw = flops / (dw_ms * 1e-3) / 1e12
    del dw_legs
    out["ste_backward_dw"] = {
        "workload": "dW of the 4096-token projections (dy bf16 [4096][N], x_q int8 [4096][K] "
                    "-> dW fp32 [N][K]), straight-through estimator",
        "roofline": {"bound": "mfma", "kernel": "k_ste_dw (v_mfma_f32_32x32x16_bf16) after "
                     "k_dw_prep_a / k_dw_prep_b",
                     "achieved": round(tf_dw, 1), "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(tf_dw / BF16_PEAK_TFLOPS, 4),
                     "matrix_core_TFLOPs": round(2 * tf_dw, 1),
                     "note": "achieved counts the 2*M*N*K flops of the product; the matrix "
                             "cores run twice that (the hi and lo bf16 parts of dy * x_scale)",
                     "traffic": traffic.get("ste_dw_4096"),
                     "traffic_unit": "HBM bytes per bl_ste_backward_dw call",
                     "per_projection": per_dw}}
    print(f"ste dW: {tf_dw:.1f} TFLOP/s", file=sys.stderr, flush=True)
    out["ste_backward"] = {
        "workload": "dx of the 4096-token projections (dy bf16 [4096][N] -> dx fp32 [4096][K]), "
                    "straight-through estimator",
        "roofline": {"bound": "mfma", "kernel": "k_ste_dx (v_mfma_f32_32x32x16_bf16)",
                     "achieved": round(tf, 1), "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(tf / BF16_PEAK_TFLOPS, 4),
                     "traffic": traffic.get("ste_dx_4096"),
                     "traffic_unit": "HBM bytes per bl_ste_backward_dx call",
                     "per_projection": per},
        "vendor_bf16_gemm": {
            "library": "hipBLASLt through torch.matmul: dense bf16 x bf16 -> bf16 on the same "
                       "shapes, weights stored as bf16 (context, not a target)",
            "TFLOPs": round(flops / reps / (v_us * 1e-6) / 1e12, 1)}}
    del legs
    torch.cuda.empty_cache()
    print(f"ste dx: {tf:.1f} TFLOP/s", file=sys.stderr, flush=True)

    # -------------------- one 2560 projection and the 3B block (M = 1) ----
    def rotated_decode(wid, copies, key):
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
        del gr
        # The same projections from the bf16 token: bl_quant_bitlinear against
        # bl_quantize_acts + bl_bitlinear.
        xb = {name: bf16_dev(wl.activations(wid, i, 1, K)) for i, (name, K, N) in enumerate(wprojs)}

        def rotation_q(one_call):
            for c in range(copies):
                for name, K, N in wprojs:
                    xq, xs, y = io[name]
                    if one_call:
                        bl.quant_bitlinear(xb[name], *w[name][c], out=(y, xq, xs))
                    else:
                        bl.quantize_acts(xb[name], out=(xq, xs))
                        bl.bitlinear(xq, xs, *w[name][c], out=y)

        with_q = {}
        for label, one_call in (("one_call", True), ("two_calls", False)):
            rotation_q(one_call)
            torch.cuda.synchronize()
            gq = capture(lambda: rotation_q(one_call))
            with_q[label] = replay_stats(gq, 20, copies * len(wprojs))["mean_us"]
            del gq
        del w, io, xb
        torch.cuda.empty_cache()
        t = st["mean_us"] * 1e-6
        packed = sum(N * K // 4 for _, K, N in wprojs) / len(wprojs)
        alg = sum(N * K // 4 + 4 + K + 4 + 4 * N for _, K, N in wprojs) / len(wprojs)
        return {"kernel": "bl_bitlinear at one token (k_gemv1_*)", "copies": copies,
                "packed_GBps": round(packed / t / 1e9, 1),
                "roofline": {"bound": "hbm", "achieved": round(alg / t / 1e9, 1),
                             "peak": HBM_PEAK_GBS, "unit": "GB/s",
                             "frac": round(alg / t / 1e9 / HBM_PEAK_GBS, 4),
                             "traffic": traffic.get(key),
                             "traffic_unit": "HBM bytes per bl_bitlinear call",
                             "alg_bytes_per_call": round(alg)},
                "per_launch": st,
                "with_act_quant": {
                    "us_per_projection": {k: round(v, 3) for k, v in with_q.items()},
                    "packed_GBps_one_call": round(packed / (with_q["one_call"] * 1e-6) / 1e9, 1),
                    "note": "from the bf16 token: bl_quant_bitlinear (one_call: a single launch "
                            "where K <= 4096 or K is whole 4096-weight pieces, else the two "
                            "calls) against bl_quantize_acts + bl_bitlinear (two_calls)"},
                "timing": "HIP graph of the rotation, HIP events on the replay stream"}

    small = {"single_2560_decode_M1": rotated_decode(1, SMALL_COPIES, "gemv_2560_m1")}
    small["single_2560_decode_M1"]["workload"] = "one 2560->2560 projection at M=1"
    small["block_3b_decode_M1"] = rotated_decode(4, BLOCK3B_COPIES, "gemv_3b_m1")
    small["block_3b_decode_M1"]["workload"] = (
        "3B block at M=1: q, k, v, o 3200->3200; gate, up 3200->8640; down 8640->3200")
    _, p4, _ = wl.WORKLOADS[4]
    small["block_3b_prefill_M512"] = gemm_leg("gemm_3b_m512", 4, 512, p4, max(10, args.steps))
    small["block_3b_prefill_M512"]["workload"] = "3B block's seven projections at M=512"
    out["small_configs"] = small
    print(f"2560 decode M=1: {small['single_2560_decode_M1']['packed_GBps']} GB/s packed; 3B "
          f"block decode M=1: {small['block_3b_decode_M1']['packed_GBps']} GB/s packed",
          file=sys.stderr, flush=True)
    return out


def cpu_oracle_leg(args, lprojs, wl, np):
    """The CPU oracle on the 70B-class shapes, pinned to one core: per-step
    times for one matrix's weight preparation (absmean gamma, ternary codes,
    2-bit pack), the decode pass at one token (act quant, integer product,
    epilogue; both projections, repeated for about args.cpu_seconds) and a
    16-token slice of the 2048-token prefill per projection."""
    import oracle
    allowed = os.sched_getaffinity(0)
    core = min(allowed)
    os.sched_setaffinity(0, {core})
    try:
        codes, steps = {}, {}
        for i, (name, K, N) in enumerate(lprojs):
            W = wl.weights(HEADLINE_WORKLOAD, i, N, K)
            t = time.perf_counter()
            g = oracle.absmean_gamma(W)
            t_g = time.perf_counter() - t
            t = time.perf_counter()
            q = oracle.ternarize(W, g)
            t_q = time.perf_counter() - t
            t = time.perf_counter()
            oracle.pack(q)
            t_p = time.perf_counter() - t
            del W
            codes[name] = (q, g)
            steps[f"{name}_gamma_s"] = round(t_g, 4)
            steps[f"{name}_ternarize_s"] = round(t_q, 4)
            steps[f"{name}_pack_s"] = round(t_p, 4)
        xs1 = {name: wl.activations(HEADLINE_WORKLOAD, i, 1, K)
               for i, (name, K, N) in enumerate(lprojs)}
        t_aq = t_mm = t_ep = 0.0
        passes = 0
        t_start = time.perf_counter()
        while True:
            for name, K, N in lprojs:
                q, g = codes[name]
                t = time.perf_counter()
                xq, sc = oracle.act_quant(xs1[name])
                t1 = time.perf_counter()
                acc = oracle.int_matmul(xq, q)
                t2 = time.perf_counter()
                oracle.epilogue(acc, sc, g)
                t3 = time.perf_counter()
                t_aq += t1 - t
                t_mm += t2 - t1
                t_ep += t3 - t2
            passes += 1
            if time.perf_counter() - t_start >= args.cpu_seconds:
                break
        decode_s = (t_aq + t_mm + t_ep) / passes
        packed = sum(N * K // 4 for _, K, N in lprojs)
        Mp = 16
        t_pf, ops = 0.0, 0
        for i, (name, K, N) in enumerate(lprojs):
            q, g = codes[name]
            x = wl.activations(HEADLINE_WORKLOAD, i, 2048, K)[:Mp]
            t = time.perf_counter()
            xq, sc = oracle.act_quant(x)
            acc = oracle.int_matmul(xq, q)
            oracle.epilogue(acc, sc, g)
            t_pf += time.perf_counter() - t
            ops += 2 * Mp * N * K
        steps.update({"decode_act_quant_s": round(t_aq / passes, 6),
                      "decode_int_matmul_s": round(t_mm / passes, 6),
                      "decode_epilogue_s": round(t_ep / passes, 6)})
        cpu_model, ncpu = host_info()
        return {
            "value": round(packed / decode_s / 1e9, 4), "unit": "GB/s", "cores": 1,
            "kind": "oracle",
            "sample": f"70B-class shapes (up 8192->28672, down 28672->8192): {passes} decode "
                      f"pass(es) at one token (act quant, integer product, epilogue, both "
                      f"projections) in {passes * decode_s:.2f} s; weight preparation of each "
                      f"matrix once; a {Mp}-token slice of the 2048-token prefill per "
                      f"projection; single-threaded C oracle (gcc -O3 -ffp-contract=off) "
                      f"pinned to core {core}",
            "prefill_GOPS": round(ops / t_pf / 1e9, 2),
            "prefill_sample_tokens": Mp,
            "steps": steps,
            "host_cpu": cpu_model, "host_nproc": ncpu,
        }
    finally:
        os.sched_setaffinity(0, allowed)


def main():
    args = parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported "
              "(the BitLinear path here runs on a single MI355X)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import ternary_weight_linear_quant_amd as bl
    from ternary_weight_linear_quant_amd import counters
    from ternary_weight_linear_quant_amd import workloads as wl

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    bl.lib()  # fail loudly if the HIP library is missing or stale
    dev = torch.device("cuda:0")
    props = torch.cuda.get_device_properties(dev)
    traffic = counters.load_traffic(COUNTERS_FILE)

    def bf16_dev(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(dev) \
            .view(torch.bfloat16)

    def capture(fn):
        gr = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gr):
            fn()
        torch.cuda.synchronize()
        return gr

    def time_graph(gr, reps):
        settle(torch, gr.replay)
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(reps):
            gr.replay()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / reps

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

    def prepare(wid, idx, N, K, copies=1):
        W = torch.from_numpy(wl.weights(wid, idx, N, K)).to(dev)
        pk, g = bl.quantize_weights(W)
        del W
        return [(pk, g)] + [(pk.clone(), g.clone()) for _ in range(copies - 1)]

    sink = torch.zeros(4, dtype=torch.int32, device=dev)

    # ------------------------------------- headline: 70B-class decode ----
    _, lprojs, lMs = wl.WORKLOADS[HEADLINE_WORKLOAD]
    L = args.copies
    # Weight preparation (offline in the method): absmean gamma, ternary
    # codes and the 2-bit pack, timed once per matrix after a warm call.
    wts, wp_ms, wp_bytes = {}, 0.0, 0
    for i, (name, K, N) in enumerate(lprojs):
        W = torch.from_numpy(wl.weights(HEADLINE_WORKLOAD, i, N, K)).to(dev)
        bl.quantize_weights(W)
        torch.cuda.synchronize()
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        pk, g = bl.quantize_weights(W)
        b.record()
        torch.cuda.synchronize()
        wp_ms += a.elapsed_time(b)
        wp_bytes += W.numel() * 4
        del W
        wts[name] = [(pk, g)] + [(pk.clone(), g.clone()) for _ in range(L - 1)]
    io = {}
    for i, (name, K, N) in enumerate(lprojs):
        x = bf16_dev(wl.activations(HEADLINE_WORKLOAD, i, 1, K))
        xq = torch.empty((1, K), dtype=torch.int8, device=dev)
        xs = torch.empty(1, dtype=torch.float32, device=dev)
        io[name] = (x, xq, xs, torch.empty((1, N), dtype=torch.float32, device=dev))

    def decode_step():
        # One call per projection: bl_quant_bitlinear quantises the token and
        # multiplies in one launch on these rows, writing codes and scale too.
        for c in range(L):
            for name, _, _ in lprojs:
                x, xq, xs, y = io[name]
                bl.quant_bitlinear(x, *wts[name][c], out=(y, xq, xs))

    def two_call_step():
        for c in range(L):
            for name, _, _ in lprojs:
                x, xq, xs, y = io[name]
                bl.quantize_acts(x, out=(xq, xs))
                bl.bitlinear(xq, xs, *wts[name][c], out=y)

    def gemv_only():
        for c in range(L):
            for name, _, _ in lprojs:
                _, xq, xs, y = io[name]
                bl.bitlinear(xq, xs, *wts[name][c], out=y)

    decode_step()
    torch.cuda.synchronize()
    graph = None if args.no_graph else capture(decode_step)

    def replay():
        if graph is not None:
            graph.replay()
        else:
            decode_step()

    settle(torch, replay)
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
    packed_per_copy = sum(N * K // 4 for _, K, N in lprojs)
    packed_per_step = packed_per_copy * L
    value = packed_per_step / (ms_per_step * 1e-3) / 1e9

    # The roofline kernel: the step's launches are the fused act quant + GEMV
    # kernel alone, so the step's own graph times it (HIP events on the
    # replaying stream), and one graph per projection splits it by matrix.
    st_step = replay_stats(graph, 20, 2 * L) if graph is not None else None
    if st_step is None:
        gs = capture(decode_step)
        st_step = replay_stats(gs, 20, 2 * L)
        del gs

    def per_projection(body, kernel_of):
        out = {}
        for name, K, N in lprojs:
            def one(name=name):
                for c in range(L):
                    body(name, c)
            gp = capture(one)
            stp = replay_stats(gp, 20, L)
            del gp
            out[name] = {"K": K, "N": N, "kernel": kernel_of(K), "mean_us": stp["mean_us"],
                         "median_us": stp["median_us"],
                         "packed_GBps": round(N * K / 4 / (stp["mean_us"] * 1e-6) / 1e9, 1)}
        return out

    def fused_one(name, c):
        x, xq, xs, y = io[name]
        bl.quant_bitlinear(x, *wts[name][c], out=(y, xq, xs))

    def gemv_one(name, c):
        _, xq, xs, y = io[name]
        bl.bitlinear(xq, xs, *wts[name][c], out=y)

    # Algorithmic bytes of the fused launch: packed weights, the bf16 token and
    # gamma in; y, the codes and the scale out.
    alg_fused = sum(N * K // 4 + 2 * K + 4 + 4 * N + K + 4 for _, K, N in lprojs) / len(lprojs)
    achieved = alg_fused / (st_step["mean_us"] * 1e-6) / 1e9
    roofline = {
        "bound": "hbm",
        "kernel": "one-token act quant + GEMV in one launch (quantising k_gemv1_rows on "
                  "8192->28672, k_gemv1_stream on 28672->8192) with its fused epilogue",
        "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
        "frac": round(achieved / HBM_PEAK_GBS, 4),
        "traffic": traffic.get("quant_gemv_70b_m1"),
        "traffic_unit": "HBM bytes per launch (rocprofv3 FETCH_SIZE + WRITE_SIZE, scaled "
                        "by a copy kernel)",
        "alg_bytes_per_launch": round(alg_fused),
        "launches": 2 * L, "avg_us": st_step["mean_us"], "per_launch": st_step,
        "per_projection": per_projection(
            fused_one, lambda K: "k_gemv1_rows (quantising)" if K == 8192
            else "k_gemv1_stream (quantising)"),
        "timing": "the step's own HIP graph (its launches are this kernel only), HIP events "
                  "on the replay stream",
    }
    # Context: the GEMV alone on the quantised token (bl_bitlinear), and the
    # step as two calls per projection (bl_quantize_acts + bl_bitlinear).
    gg = capture(gemv_only)
    st_gemv = replay_stats(gg, 20, 2 * L)
    del gg
    alg_gemv = sum(N * K // 4 + 4 + K + 4 + 4 * N for _, K, N in lprojs) / len(lprojs)
    gemv_gbps = alg_gemv / (st_gemv["mean_us"] * 1e-6) / 1e9
    roofline["gemv_alone"] = {
        "kernel": "one-token GEMV on the quantised token (k_gemv1_rows / k_gemv1_stream), "
                  "bl_bitlinear",
        "achieved": round(gemv_gbps, 1), "frac": round(gemv_gbps / HBM_PEAK_GBS, 4),
        "traffic": traffic.get("gemv_70b_m1"), "alg_bytes_per_launch": round(alg_gemv),
        "avg_us": st_gemv["mean_us"], "per_launch": st_gemv,
        "per_projection": per_projection(
            gemv_one, lambda K: "k_gemv1_rows" if K == 8192 else "k_gemv1_stream"),
    }
    g2 = capture(two_call_step)
    st_two = replay_stats(g2, 20, 1)
    del g2
    two_call = {
        "calls": "bl_quantize_acts + bl_bitlinear per projection",
        "ms_per_step": round(st_two["mean_us"] * 1e-3, 4),
        "value": round(packed_per_step / (st_two["mean_us"] * 1e-6) / 1e9, 2),
        "act_quant_us_per_launch": round(
            (st_two["mean_us"] - st_gemv["mean_us"] * 2 * L) / (2 * L), 3),
    }
    # The same bytes through the read-only calibration stream, launch for launch.
    rbufs = [wts[name][c][0] for c in range(L) for name, _, _ in lprojs]

    def read_pass():
        for buf in rbufs:
            bl.calib_read(buf, sink)

    read_pass()
    gr = capture(read_pass)
    st_read = replay_stats(gr, 20, len(rbufs))
    del gr
    read_gbps = (packed_per_copy / 2) / (st_read["mean_us"] * 1e-6) / 1e9
    roofline["same_size_read_ceiling"] = {
        "kernel": "k_calib_read", "bytes_per_launch": packed_per_copy // 2,
        "GBps": round(read_gbps, 1), "frac_of_peak": round(read_gbps / HBM_PEAK_GBS, 4),
        "us_per_launch": st_read["mean_us"],
        "achieved_over_it": round(achieved / read_gbps, 4),
        "gemv_alone_over_it": round(gemv_gbps / read_gbps, 4)}
    print(f"70b decode step: {value:.1f} GB/s ({ms_per_step * 1e3 / L:.2f} us per copy), fused "
          f"launch {achieved:.1f} GB/s ({st_step['mean_us']} us), GEMV alone {gemv_gbps:.1f} "
          f"GB/s ({st_gemv['mean_us']} us), two calls {two_call['value']} GB/s, read stream "
          f"{read_gbps:.1f} GB/s", file=sys.stderr, flush=True)

    def gemm_leg(label, wid, M, legs_w, reps):
        """Prefill GEMMs at M tokens: act quant then BitLinear per projection;
        the step and each projection's GEMM timed from HIP graphs."""
        legs = []
        for i, (name, K, N) in enumerate(legs_w):
            pk, g = wts[name][0] if wid == HEADLINE_WORKLOAD else prepare(wid, i, N, K)[0]
            x = bf16_dev(wl.activations(wid, i, M, K))
            xq, xs = bl.quantize_acts(x)
            y = torch.empty((M, N), dtype=torch.float32, device=dev)
            legs.append((name, K, N, x, xq, xs, pk, g, y))

        def step():
            for name, K, N, x, xq, xs, pk, g, y in legs:
                bl.quantize_acts(x, out=(xq, xs))
                bl.bitlinear(xq, xs, pk, g, out=y)

        # Timed from HIP graphs (HIP events on the replaying stream), so the
        # host's launch cost never leaves the GPU idle between short calls:
        # the whole step, then each projection's GEMM and act quant alone,
        # GRAPH_CALLS back-to-back calls per graph.
        for _ in range(1 + args.warmup):
            step()
        torch.cuda.synchronize()
        gs = capture(step)
        p_ms = time_graph(gs, reps)
        del gs
        ops = sum(2 * M * N * K for _, K, N, *_ in legs)
        per = {}
        gemm_ms = 0.0
        aq_ms = 0.0
        for name, K, N, x, xq, xs, pk, g, y in legs:
            def gemms(xq=xq, xs=xs, pk=pk, g=g, y=y):
                for _ in range(GRAPH_CALLS):
                    bl.bitlinear(xq, xs, pk, g, out=y)

            def quants(x=x, xq=xq, xs=xs):
                for _ in range(GRAPH_CALLS):
                    bl.quantize_acts(x, out=(xq, xs))

            gg = capture(gemms)
            ms = time_graph(gg, reps) / GRAPH_CALLS
            del gg
            gq = capture(quants)
            aq_ms += time_graph(gq, reps) / GRAPH_CALLS
            del gq
            gemm_ms += ms
            per[name] = {"M": M, "K": K, "N": N, "avg_us": round(1e3 * ms, 2),
                         "TOPS": round(2 * M * N * K / (ms * 1e-3) / 1e12, 1)}
        tops = ops / (gemm_ms * 1e-3) / 1e12
        # Context only: the vendor's plain int8 GEMM on the same shapes
        # (int8 x int8 -> int32, no ternary expansion, no fp32 epilogue).
        vendor_us = {}
        for name, K, N, x, xq, xs, pk, g, y in legs:
            b8 = torch.randint(-1, 2, (K, N), dtype=torch.int8, device=dev)
            settle(torch, lambda: torch._int_mm(xq, b8))
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
            "TOPS": round(tops, 1),
            "roofline": {"bound": "mfma", "kernel": "k_gemm", "achieved": round(tops, 1),
                         "peak": I8_PEAK_TOPS, "unit": "TFLOP/s (int8 TOPS)",
                         "frac": round(tops / I8_PEAK_TOPS, 4),
                         "traffic": traffic.get(label),
                         "traffic_unit": "HBM bytes per bl_bitlinear call",
                         "alg_bytes_per_call": round(alg),
                         "per_projection": per},
            "act_quant_avg_us": round(1e3 * aq_ms / len(legs), 2),
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

    # ------------------------------------- prefill at 2048 tokens ----
    prefill70 = {"workload": "70b_class prefill: 2048 tokens, up 8192->28672 and down "
                             "28672->8192"}
    prefill70.update(gemm_leg("gemm_prefill_70b", HEADLINE_WORKLOAD, 2048, lprojs,
                              max(3, args.steps // 4)))

    extra = {}
    if not args.no_extra:
        # ----------------------------- 70B-class decode at 64 tokens ----
        io64 = {}
        for i, (name, K, N) in enumerate(lprojs):
            xq, xs = bl.quantize_acts(bf16_dev(wl.activations(HEADLINE_WORKLOAD, i, 64, K)))
            io64[name] = (xq, xs, torch.empty((64, N), dtype=torch.float32, device=dev))

        def rotation64():
            for c in range(L):
                for name, K, N in lprojs:
                    xq, xs, y = io64[name]
                    bl.bitlinear(xq, xs, *wts[name][c], out=y)

        rotation64()
        torch.cuda.synchronize()
        gr = capture(rotation64)
        st = replay_stats(gr, 20, 2 * L)
        del gr, io64
        t = st["mean_us"] * 1e-6
        alg = sum(N * K // 4 + 4 + 64 * K + 4 * 64 + 4 * 64 * N for _, K, N in lprojs) / 2
        ops = sum(2 * 64 * N * K for _, K, N in lprojs) / 2
        extra["decode_M64_70b"] = {
            "kernel": "k_gemm (bl_bitlinear's choice at 64 tokens: two K groups per "
                      "workgroup with a 4-deep ring; the down projection also splits K)",
            "packed_GBps": round(packed_per_copy / 2 / t / 1e9, 1),
            "roofline": {"bound": "hbm", "achieved": round(alg / t / 1e9, 1),
                         "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": round(alg / t / 1e9 / HBM_PEAK_GBS, 4),
                         "traffic": traffic.get("decode_70b_m64"),
                         "traffic_unit": "HBM bytes per bl_bitlinear call",
                         "alg_bytes_per_call": round(alg)},
            "mfma": {"achieved_TOPS": round(ops / t / 1e12, 1),
                     "frac": round(ops / t / 1e12 / I8_PEAK_TOPS, 4)},
            "per_launch": st}
        print(f"70b decode M=64: {extra['decode_M64_70b']['packed_GBps']} GB/s packed",
              file=sys.stderr, flush=True)

        # --------------------- the denser formats at one token (70B) ----
        fmt_w = {"base3": {name: [(bl.pack_base3(pk, K), g) for pk, g in wts[name]]
                           for name, K, N in lprojs}}
        binw = {}
        for i, (name, K, N) in enumerate(lprojs):
            W = torch.from_numpy(wl.weights(HEADLINE_WORKLOAD, i, N, K)).to(dev)
            bits, gb = bl.quantize_weights_binary(W)
            del W
            binw[name] = [(bits, gb)] + [(bits.clone(), gb.clone()) for _ in range(L - 1)]
        fmt_w["binary"] = binw
        fmt_fn = {"base3": bl.bitlinear_base3, "binary": bl.bitlinear_binary}
        for fmt, wsets in fmt_w.items():
            def rotation_f(fmt=fmt, wsets=wsets):
                for c in range(L):
                    for name, K, N in lprojs:
                        _, xq, xs, y = io[name]
                        fmt_fn[fmt](xq, xs, *wsets[name][c], out=y)

            rotation_f()
            torch.cuda.synchronize()
            gr = capture(rotation_f)
            st = replay_stats(gr, 20, L * len(lprojs))
            del gr
            t = st["mean_us"] * 1e-6
            wbytes = sum(wsets[name][0][0].numel() * wsets[name][0][0].element_size()
                         for name, _, _ in lprojs) / len(lprojs)
            alg = sum(wsets[name][0][0].numel() * wsets[name][0][0].element_size()
                      + 4 + K + 4 + 4 * N for name, K, N in lprojs) / len(lprojs)
            nweights = sum(N * K for _, K, N in lprojs) / len(lprojs)
            extra[f"decode_M1_70b_{fmt}"] = {
                "kernel": "k_gemv (" + ("five ternary weights per byte" if fmt == "base3"
                                        else "1 bit per +-1 weight") + ")",
                "bits_per_weight": round(8 * wbytes / nweights, 4),
                "packed_GBps": round(wbytes / t / 1e9, 1),
                "weights_per_s": round(nweights / t / 1e12, 3),
                "weights_unit": "T weights/s",
                "roofline": {"bound": "hbm", "achieved": round(alg / t / 1e9, 1),
                             "peak": HBM_PEAK_GBS, "unit": "GB/s",
                             "frac": round(alg / t / 1e9 / HBM_PEAK_GBS, 4),
                             "traffic": traffic.get(f"gemv_70b_m1_{fmt}"),
                             "traffic_unit": "HBM bytes per launch",
                             "alg_bytes_per_launch": round(alg)},
                "per_launch": st,
            }
            print(f"70b decode M=1 {fmt}: {extra[f'decode_M1_70b_{fmt}']['weights_per_s']} "
                  f"T weights/s", file=sys.stderr, flush=True)
        roofline["weights_per_s"] = round(
            sum(N * K for _, K, N in lprojs) / 2 / (st_step["mean_us"] * 1e-6) / 1e12, 3)
        roofline["gemv_alone"]["weights_per_s"] = round(
            sum(N * K for _, K, N in lprojs) / 2 / (st_gemv["mean_us"] * 1e-6) / 1e12, 3)
        del fmt_w, binw

        # -------------------------------------- the int8 MFMA ceiling ----
        msink = bl.calib_mfma_sink(dev)
        iters = 4000
        settle(torch, lambda: bl.calib_mfma_i8(iters, msink))
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(5):
            mops = bl.calib_mfma_i8(iters, msink)
        b.record()
        torch.cuda.synchronize()
        mfma_tops = mops * 5 / (a.elapsed_time(b) * 1e-3) / 1e12
        extra["ceilings"] = {
            "hbm_read_stream": roofline["same_size_read_ceiling"],
            "i8_mfma_loop": {"kernel": "k_calib_mfma (v_mfma_i32_32x32x32_i8, 8 waves/CU)",
                             "TOPS": round(mfma_tops, 1),
                             "frac_of_peak": round(mfma_tops / I8_PEAK_TOPS, 4)}}
        print(f"ceilings: mfma {mfma_tops:.0f} TOPS", file=sys.stderr, flush=True)
    del wts, graph
    torch.cuda.empty_cache()

    if not args.no_extra:
        extra.update(other_workloads(args, bl, wl, np, torch, dev, bf16_dev, capture,
                                     time_graph, replay_stats, prepare, gemm_leg, traffic,
                                     sink))

    cpu_baseline = None
    if args.cpu_seconds > 0:
        cpu_baseline = cpu_oracle_leg(args, lprojs, wl, np)

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
            "workload": "70b_class_decode_M1: per weight copy, act quant + BitLinear up "
                        "(8192->28672) and act quant + BitLinear down (28672->8192) at one "
                        "token, one bl_quant_bitlinear call (one launch) per projection",
            "tokens": 1, "weight_copies": L,
            "packed_weight_bytes_per_step": packed_per_step,
            "hip_graph": not args.no_graph,
            "parallelism": "single GPU",
        },
        "frac_hbm_step": round(value / HBM_PEAK_GBS, 4),
        "two_call_step": two_call,
        "settle_ms_before_timing": SETTLE_MS,
        "roofline": roofline,
        "prefill_M2048": prefill70,
        "cpu_baseline": cpu_baseline,
        "weight_prep": {"matrices": [name for name, _, _ in lprojs],
                        "ms_total": round(wp_ms, 3),
                        "fp32_read_GBps": round(wp_bytes / (wp_ms * 1e-3) / 1e9, 1)},
        "device": {"name": props.name, "cus": props.multi_processor_count,
                   "host_cpu": cpu_model, "host_nproc": ncpu},
    }
    out.update(extra)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
