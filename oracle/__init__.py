"""CPU oracle for the BitNet b1.58 BitLinear forward pass (ctypes wrapper).

TEST INFRASTRUCTURE ONLY: the plain single-threaded C reference in
``oracle.c`` that the GPU library is checked against. Only the tests, the
smoke check and the benchmark's CPU-baseline leg may import this package;
the product package never does.

Every function takes and returns numpy arrays. What each computes, and the
passage of the pages it follows, is documented in ``oracle.h``.
"""
from __future__ import annotations

import ctypes
import hashlib
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
CFLAGS = ["-std=c11", "-O3", "-ffp-contract=off", "-fno-fast-math",
          "-fPIC", "-shared", "-Wall", "-Wextra"]
_HDR = os.path.join(_HERE, "oracle.h")

WEIGHT_EPS = 1e-5   # s = gamma + eps before rounding the weights
RMS_EPS = 1e-5      # epsilon inside the RMSNorm square root

_lib = None


def source_sha256() -> str:
    """SHA-256 over oracle.c, oracle.h and the compile flags; embedded in
    liboracle.so so that a stale build is detected by content, not mtime."""
    h = hashlib.sha256()
    for f in (_SRC, _HDR):
        with open(f, "rb") as fh:
            h.update(fh.read())
        h.update(b"\0")
    h.update(" ".join(CFLAGS).encode())
    return h.hexdigest()


def build(force: bool = True) -> str:
    """Compile oracle.c into liboracle.so with gcc; returns the path. Without
    force, only when the library is missing or was built from other sources."""
    if force or _built_sha256() != source_sha256():
        tmp = _LIB_PATH + ".tmp"
        subprocess.run(["gcc", *CFLAGS, f'-DORACLE_SOURCE_SHA256="{source_sha256()}"', _SRC,
                        "-o", tmp, "-lm"], check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _built_sha256():
    """Digest embedded in the library file on disk (None if absent), read by
    name from the file's bytes, so no stale copy is loaded to ask it."""
    if not os.path.exists(_LIB_PATH):
        return None
    with open(_LIB_PATH, "rb") as fh:
        data = fh.read()
    i = data.find(b"oracle-source-sha256:")
    if i < 0:
        return None
    return data[i + 21:i + 21 + 64].decode("ascii", "replace")


def _load():
    global _lib
    if _lib is not None:
        return _lib
    build(force=False)
    lib = ctypes.CDLL(_LIB_PATH)
    got = ctypes.c_char_p.in_dll(lib, "oracle_source_sha256").value.decode()
    if got != "oracle-source-sha256:" + source_sha256():
        raise RuntimeError(f"{_LIB_PATH} does not match oracle.c (digest {got[21:37]})")
    P = ctypes.c_void_p
    I = ctypes.c_int64
    F = ctypes.c_float
    sig = {
        "oracle_absmean_rowsums": ([P, I, I, P], None),
        "oracle_absmean_gamma": ([P, I, I], F),
        "oracle_ternarize": ([P, I, I, F, F, P], None),
        "oracle_pack": ([P, I, I, P], None),
        "oracle_unpack": ([P, I, I, P], None),
        "oracle_act_quant": ([P, I, I, P, F, P, P, P], None),
        "oracle_int_matmul": ([P, I, I, P, I, P], None),
        "oracle_addsub_matmul": ([P, I, I, P, I, P], None),
        "oracle_epilogue": ([P, I, I, P, F, P], None),
        "oracle_relu2_glu": ([P, P, I, P], None),
        "oracle_swiglu": ([P, P, I, P], None),
        "oracle_binarize": ([P, I, I, P], None),
        "oracle_pack_binary": ([P, I, I, I, P], None),
        "oracle_unpack_binary": ([P, I, I, I, P], None),
        "oracle_pack_base3": ([P, I, I, I, P], None),
        "oracle_unpack_base3": ([P, I, I, I, P], None),
        "oracle_pack_ste_t": ([P, I, I, I, P], None),
        "oracle_ste_dx": ([P, I, I, P, I, F, P], None),
        "oracle_ste_dw": ([P, I, I, P, P, I, P], None),
    }
    for name, (args, res) in sig.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = res
    _lib = lib
    return lib


def _c(a: np.ndarray, dtype) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=dtype)


def _p(a: np.ndarray | None):
    return None if a is None else a.ctypes.data


def absmean_rowsums(W: np.ndarray) -> np.ndarray:
    W = _c(W, np.float32)
    N, K = W.shape
    R = np.empty(N, np.float64)
    _load().oracle_absmean_rowsums(_p(W), N, K, _p(R))
    return R


def absmean_gamma(W: np.ndarray) -> np.float32:
    W = _c(W, np.float32)
    N, K = W.shape
    return np.float32(_load().oracle_absmean_gamma(_p(W), N, K))


def ternarize(W: np.ndarray, gamma, eps: float = WEIGHT_EPS) -> np.ndarray:
    W = _c(W, np.float32)
    N, K = W.shape
    q = np.empty((N, K), np.int8)
    _load().oracle_ternarize(_p(W), N, K, float(np.float32(gamma)),
                             float(np.float32(eps)), _p(q))
    return q


def pack(q: np.ndarray) -> np.ndarray:
    q = _c(q, np.int8)
    N, K = q.shape
    if K % 16:
        raise ValueError("K must be a multiple of 16")
    out = np.empty((N, K // 16), np.uint32)
    _load().oracle_pack(_p(q), N, K, _p(out))
    return out


def unpack(packed: np.ndarray, K: int) -> np.ndarray:
    packed = _c(packed, np.uint32)
    N = packed.shape[0]
    q = np.empty((N, K), np.int8)
    _load().oracle_unpack(_p(packed), N, K, _p(q))
    return q


def quantize_weights(W: np.ndarray):
    """(packed uint32 [N][K/16], gamma fp32, codes int8 [N][K])."""
    g = absmean_gamma(W)
    q = ternarize(W, g)
    return pack(q), g, q


def act_quant(x_bits: np.ndarray, gain_bits: np.ndarray | None = None,
              rms_eps: float = RMS_EPS, return_rms: bool = False):
    """x_bits: uint16 bf16 bits [M][K]. Returns (x_q int8 [M][K], scale fp32 [M])."""
    x_bits = _c(x_bits, np.uint16)
    M, K = x_bits.shape
    g = None if gain_bits is None else _c(gain_bits, np.uint16)
    if g is not None and g.shape != (K,):
        raise ValueError("gain must have shape (K,)")
    xq = np.empty((M, K), np.int8)
    sc = np.empty(M, np.float32)
    rms = np.full(M, np.nan, np.float64)
    _load().oracle_act_quant(_p(x_bits), M, K, _p(g), float(np.float32(rms_eps)),
                             _p(xq), _p(sc), _p(rms))
    return (xq, sc, rms) if return_rms else (xq, sc)


def int_matmul(x_q: np.ndarray, q: np.ndarray) -> np.ndarray:
    x_q = _c(x_q, np.int8)
    q = _c(q, np.int8)
    M, K = x_q.shape
    N, K2 = q.shape
    if K != K2:
        raise ValueError("inner dimensions differ")
    acc = np.empty((M, N), np.int32)
    _load().oracle_int_matmul(_p(x_q), M, K, _p(q), N, _p(acc))
    return acc


def addsub_matmul(x_q: np.ndarray, q: np.ndarray) -> np.ndarray:
    x_q = _c(x_q, np.int8)
    q = _c(q, np.int8)
    M, K = x_q.shape
    N, K2 = q.shape
    if K != K2:
        raise ValueError("inner dimensions differ")
    acc = np.empty((M, N), np.int32)
    _load().oracle_addsub_matmul(_p(x_q), M, K, _p(q), N, _p(acc))
    return acc


def epilogue(acc: np.ndarray, scale: np.ndarray, gamma) -> np.ndarray:
    acc = _c(acc, np.int32)
    scale = _c(scale, np.float32)
    M, N = acc.shape
    y = np.empty((M, N), np.float32)
    _load().oracle_epilogue(_p(acc), M, N, _p(scale), float(np.float32(gamma)),
                            _p(y))
    return y


def bitlinear(x_q: np.ndarray, scale: np.ndarray, q: np.ndarray, gamma):
    """(y fp32 [M][N], acc int32 [M][N]) from codes."""
    acc = int_matmul(x_q, q)
    return epilogue(acc, scale, gamma), acc


def relu2_glu(g: np.ndarray, u: np.ndarray) -> np.ndarray:
    g = _c(g, np.float32)
    u = _c(u, np.float32)
    if g.shape != u.shape:
        raise ValueError("shape mismatch")
    h = np.empty(g.shape, np.uint16)
    _load().oracle_relu2_glu(_p(g), _p(u), g.size, _p(h))
    return h


def swiglu(g: np.ndarray, u: np.ndarray) -> np.ndarray:
    """bf16 bits of fp32(silu(g)) * u, silu in fp64 (oracle_swiglu)."""
    g = _c(g, np.float32)
    u = _c(u, np.float32)
    if g.shape != u.shape:
        raise ValueError("shape mismatch")
    h = np.empty(g.shape, np.uint16)
    _load().oracle_swiglu(_p(g), _p(u), g.size, _p(h))
    return h


# ------------------------------------------------- other weight formats ----

def binary_row_words(K: int) -> int:
    """uint32 words per row of 1-bit weights: 16-byte rows, 128 weights each."""
    return 4 * ((K + 127) // 128)


def base3_row_bytes(K: int) -> int:
    """Bytes per row of base-3 weights: ceil(K/5) rounded up to 16."""
    return 16 * (((K + 4) // 5 + 15) // 16)


def binarize(W: np.ndarray) -> np.ndarray:
    W = _c(W, np.float32)
    N, K = W.shape
    q = np.empty((N, K), np.int8)
    _load().oracle_binarize(_p(W), N, K, _p(q))
    return q


def pack_binary(q: np.ndarray) -> np.ndarray:
    q = _c(q, np.int8)
    N, K = q.shape
    rw = binary_row_words(K)
    out = np.empty((N, rw), np.uint32)
    _load().oracle_pack_binary(_p(q), N, K, rw, _p(out))
    return out


def unpack_binary(packed: np.ndarray, K: int) -> np.ndarray:
    packed = _c(packed, np.uint32)
    N = packed.shape[0]
    q = np.empty((N, K), np.int8)
    _load().oracle_unpack_binary(_p(packed), N, K, packed.shape[1], _p(q))
    return q


def quantize_weights_binary(W: np.ndarray):
    """(1-bit packed uint32 [N][row words], gamma fp32, codes int8 [N][K])."""
    g = absmean_gamma(W)
    q = binarize(W)
    return pack_binary(q), g, q


def pack_base3(q: np.ndarray) -> np.ndarray:
    q = _c(q, np.int8)
    N, K = q.shape
    rb = base3_row_bytes(K)
    out = np.empty((N, rb), np.uint8)
    _load().oracle_pack_base3(_p(q), N, K, rb, _p(out))
    return out


def unpack_base3(packed: np.ndarray, K: int) -> np.ndarray:
    packed = _c(packed, np.uint8)
    N = packed.shape[0]
    q = np.empty((N, K), np.int8)
    _load().oracle_unpack_base3(_p(packed), N, K, packed.shape[1], _p(q))
    return q


# ------------------------------------------- straight-through backward ----

def ste_t_row_bytes(N: int) -> int:
    """Bytes per row of the transposed backward codes: ceil(N/4) rounded to 16."""
    return 16 * (((N + 3) // 4 + 15) // 16)


def pack_ste_t(q: np.ndarray) -> np.ndarray:
    """Codes q [N][K] -> transposed uint8 [K][ste_t_row_bytes(N)], four n per byte."""
    q = _c(q, np.int8)
    N, K = q.shape
    rb = ste_t_row_bytes(N)
    out = np.empty((K, rb), np.uint8)
    _load().oracle_pack_ste_t(_p(q), N, K, rb, _p(out))
    return out


def ste_dx(dy_bits: np.ndarray, q: np.ndarray, gamma) -> np.ndarray:
    """dx fp32 [M][K] = gamma * dy . q for bf16 dy [M][N] (raw bits)."""
    dy_bits = _c(dy_bits, np.uint16)
    q = _c(q, np.int8)
    M, N = dy_bits.shape
    K = q.shape[1]
    dx = np.empty((M, K), np.float32)
    _load().oracle_ste_dx(_p(dy_bits), M, N, _p(q), K, float(np.float32(gamma)), _p(dx))
    return dx


def ste_dw(dy_bits: np.ndarray, x_q: np.ndarray, x_scale: np.ndarray) -> np.ndarray:
    """dW fp32 [N][K] = sum_m dy[m][n] * x_q[m][k] * x_scale[m] for bf16 dy
    [M][N] (raw bits), int8 x_q [M][K] and fp32 x_scale [M]."""
    dy_bits = _c(dy_bits, np.uint16)
    x_q = _c(x_q, np.int8)
    x_scale = _c(x_scale, np.float32)
    M, N = dy_bits.shape
    K = x_q.shape[1]
    if x_q.shape[0] != M or x_scale.shape != (M,):
        raise ValueError("shape mismatch")
    dW = np.empty((N, K), np.float32)
    _load().oracle_ste_dw(_p(dy_bits), M, N, _p(x_q), _p(x_scale), K, _p(dW))
    return dW
