"""Seeded synthetic inputs and the workload shapes.

This module only draws random numbers and lays them out; it holds none of
the method's arithmetic. Both the GPU library's tests/benchmark and the CPU
oracle take their inputs from here.

Recipe (the pages measure on trained models and public suites, none of which
is available; these seeded tensors stand in for them):
  * latent weights W: fp32 [N][K] = 0.02 * N(0, 1), one matrix per projection;
  * activations x: N(0, 1) fp32 [M][K], then round(0.001*K) channels, drawn
    without replacement and shared by every token of that input, scaled by
    20 as outliers, then rounded to bf16 (nearest, ties to even);
  * RMSNorm gain g: bf16(1 + 0.1 * N(0, 1)) [K].
Each tensor has its own numpy PCG64 stream, seed = 1000*workload + 10*role +
index (role 0 weights, 1 activations, 2 gain, 3 outlier columns).
"""
from __future__ import annotations

import numpy as np

ROLE_W, ROLE_X, ROLE_GAIN, ROLE_OUTLIER = 0, 1, 2, 3

# Workloads: id -> (name, [(projection, K, N), ...], token counts M).
WORKLOADS = {
    1: ("single_2560", [("proj", 2560, 2560)], [1]),
    2: ("ffn_2b4t_decode",
        [("gate", 2560, 6912), ("up", 2560, 6912), ("down", 6912, 2560)],
        [1, 4, 16]),
    3: ("prefill_4096", [("up", 2560, 6912), ("down", 6912, 2560)], [4096]),
    4: ("block_3b",
        [("q", 3200, 3200), ("k", 3200, 3200), ("v", 3200, 3200),
         ("o", 3200, 3200), ("gate", 3200, 8640), ("up", 3200, 8640),
         ("down", 8640, 3200)],
        [1, 512]),
    5: ("ffn_70b", [("up", 8192, 28672), ("down", 28672, 8192)],
        [1, 64, 2048]),
}


def seed(workload: int, role: int, index: int) -> int:
    return 1000 * workload + 10 * role + index


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16 (nearest, ties to even) and return the raw bits."""
    u = np.ascontiguousarray(a, np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    return ((u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, np.uint16).astype(np.uint32)
            << np.uint32(16)).view(np.float32)


def weights(workload: int, index: int, N: int, K: int,
            sigma: float = 0.02) -> np.ndarray:
    rng = np.random.default_rng(seed(workload, ROLE_W, index))
    w = rng.standard_normal((N, K), dtype=np.float32)
    w *= np.float32(sigma)
    return w


def outlier_columns(workload: int, index: int, K: int) -> np.ndarray:
    rng = np.random.default_rng(seed(workload, ROLE_OUTLIER, index))
    n_out = int(round(0.001 * K))
    return np.sort(rng.choice(K, size=n_out, replace=False))


def activations(workload: int, index: int, M: int, K: int,
                outlier_scale: float = 20.0) -> np.ndarray:
    """bf16 bits [M][K]."""
    rng = np.random.default_rng(seed(workload, ROLE_X, index))
    x = rng.standard_normal((M, K), dtype=np.float32)
    cols = outlier_columns(workload, index, K)
    x[:, cols] *= np.float32(outlier_scale)
    return f32_to_bf16_bits(x)


def rms_gain(workload: int, index: int, K: int) -> np.ndarray:
    """bf16 bits [K]."""
    rng = np.random.default_rng(seed(workload, ROLE_GAIN, index))
    g = np.float32(1.0) + np.float32(0.1) * rng.standard_normal(K, dtype=np.float32)
    return f32_to_bf16_bits(g)


def ffn_hidden(workload: int, index: int, M: int, N: int) -> tuple:
    """Synthetic fp32 gate/up outputs [M][N] for glue-only tests."""
    rng = np.random.default_rng(seed(workload, ROLE_X, 100 + index))
    g = rng.standard_normal((M, N), dtype=np.float32)
    u = rng.standard_normal((M, N), dtype=np.float32)
    return g, u
