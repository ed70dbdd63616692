"""Thin Python binding of the gfx950 BitLinear library (libbitlinear.so).

Argument marshalling only: every step of the BitLinear forward runs in the
HIP kernels behind the C ABI declared in include/bitlinear.h. PyTorch supplies
device memory and the current stream. There is no fallback: if the library is
not built, or no GPU is present, every call raises.

    W_packed, gamma = quantize_weights(W)          # fp32 [N][K] on the GPU
    x_q, x_scale = quantize_acts(x, rms_gain=g)    # bf16 [M][K]
    y = bitlinear(x_q, x_scale, W_packed, gamma)   # fp32 [M][N]
"""
from __future__ import annotations

import ctypes
import os

__all__ = ["lib", "library_path", "quantize_weights", "quantize_acts", "bitlinear",
           "bitlinear_pair", "relu2_glu", "relu2_glu_quant", "ffn_relu2", "ffn_relu2_workspace",
           "BitLinearError", "packed_bytes"]

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libbitlinear.so")
_lib = None

BL_OK, BL_ERR_INVALID_ARG, BL_ERR_HIP, BL_ERR_NO_DEVICE = 0, 1, 2, 3
BL_GLU_RELU2, BL_GLU_SWIGLU = 0, 1
_GLU_KINDS = {"relu2": BL_GLU_RELU2, "swiglu": BL_GLU_SWIGLU}

# name -> (argtypes, restype); the same names and order as include/bitlinear.h
_P, _I, _F, _S = ctypes.c_void_p, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t
_SIGNATURES = {
    "bl_status_string": ([ctypes.c_int], ctypes.c_char_p),
    "bl_last_hip_error": ([], ctypes.c_int),
    "bl_version": ([], ctypes.c_char_p),
    "bl_source_sha256": ([], ctypes.c_char_p),
    "bl_packed_bytes": ([_I, _I], _S),
    "bl_quantize_weights_workspace_bytes": ([_I, _I], _S),
    "bl_quantize_weights": ([_P, _I, _I, _P, _P, _P, _S, _P], ctypes.c_int),
    "bl_quantize_acts": ([_P, _I, _I, _P, _F, _P, _P, _P], ctypes.c_int),
    "bl_bitlinear_choice": ([_I, _I, _I, ctypes.c_int], ctypes.c_int),
    "bl_quant_bitlinear": ([_P, _I, _I, _P, _F, _P, _P, _I, _P, _P, _P, _P], ctypes.c_int),
    "bl_bitlinear": ([_P, _P, _I, _I, _P, _P, _I, _P, _P, _P], ctypes.c_int),
    "bl_bitlinear_path": ([_P, _P, _I, _I, _P, _P, _I, _P, _P, ctypes.c_int, _P],
                          ctypes.c_int),
    "bl_relu2_glu": ([_P, _P, _I, _P, _P], ctypes.c_int),
    "bl_glu": ([_P, _P, _I, ctypes.c_int, _P, _P], ctypes.c_int),
    "bl_bitlinear_pair": ([_P, _P, _I, _I, _P, _P, _I, _P, _P, _P, _I, _P, _P], ctypes.c_int),
    "bl_relu2_glu_quant": ([_P, _P, _I, _I, _P, _P, _P], ctypes.c_int),
    "bl_relu2_glu_subln_quant": ([_P, _P, _I, _I, _P, _F, _P, _P, _P], ctypes.c_int),
    "bl_glu_quant": ([_P, _P, _I, _I, ctypes.c_int, _P, _F, _P, _P, _P], ctypes.c_int),
    "bl_ffn_relu2_workspace_bytes": ([_I, _I, _I], _S),
    "bl_ffn_relu2": ([_P, _I, _I, _P, _P, _P, _P, _I, _P, _P, _P, _P, _S, _P], ctypes.c_int),
    "bl_ffn_relu2_subln": ([_P, _I, _I, _P, _P, _P, _P, _I, _P, _P, _P, _F, _P, _P, _S, _P],
                           ctypes.c_int),
    "bl_ffn_step": ([_P, _I, _I, _P, _P, _P, _P, _I, _P, _P, ctypes.c_int, _P, _F, _P, _P, _S,
                     _P], ctypes.c_int),
    "bl_ffn_step_noalloc": ([_P, _I, _I, _P, _P, _P, _P, _I, _P, _P, ctypes.c_int, _P, _F, _P,
                             _P], ctypes.c_int),
    "bl_packed_bytes_binary": ([_I, _I], _S),
    "bl_packed_bytes_base3": ([_I, _I], _S),
    "bl_quantize_weights_binary": ([_P, _I, _I, _P, _P, _P, _S, _P], ctypes.c_int),
    "bl_pack_base3": ([_P, _I, _I, _P, _P], ctypes.c_int),
    "bl_bitlinear_binary": ([_P, _P, _I, _I, _P, _P, _I, _P, _P, _P], ctypes.c_int),
    "bl_bitlinear_base3": ([_P, _P, _I, _I, _P, _P, _I, _P, _P, _P], ctypes.c_int),
    "bl_ste_t_bytes": ([_I, _I], _S),
    "bl_pack_ste_t": ([_P, _I, _I, _P, _P], ctypes.c_int),
    "bl_ste_backward_dx": ([_P, _I, _I, _P, _P, _I, _P, _P], ctypes.c_int),
    "bl_ste_dw_workspace_bytes": ([_I, _I, _I], _S),
    "bl_ste_backward_dw": ([_P, _I, _I, _P, _P, _I, _P, _P, _S, _P], ctypes.c_int),
    "bl_calib_read": ([_P, _S, _P, _P], ctypes.c_int),
    "bl_calib_copy": ([_P, _P, _S, _P], ctypes.c_int),
    "bl_calib_mfma_i8_ops": ([_I], _I),
    "bl_calib_mfma_i8_sink_elems": ([], _S),
    "bl_calib_mfma_i8": ([_I, _P, _P], ctypes.c_int),
}


class BitLinearError(RuntimeError):
    pass


def library_path() -> str:
    return _LIB_PATH


def lib():
    """Load libbitlinear.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise BitLinearError(
                f"{_LIB_PATH} is missing: build it with "
                "`python -c 'import __graft_entry__ as g; g.build()'` "
                "(or python ternary_weight_linear_quant_amd/build.py)")
        handle = ctypes.CDLL(_LIB_PATH)
        for name, (args, res) in _SIGNATURES.items():
            fn = getattr(handle, name)
            fn.argtypes = args
            fn.restype = res
        from . import build as _build
        built, tree = handle.bl_source_sha256().decode(), _build.source_sha256()
        if built != tree:
            raise BitLinearError(
                f"{_LIB_PATH} was built from other sources (digest {built[:16]}, tree "
                f"{tree[:16]}): rebuild it with `python -c 'import __graft_entry__ as g; "
                "g.build()'`")
        _lib = handle
    return _lib


def _check(status: int, what: str):
    if status != BL_OK:
        L = lib()
        msg = L.bl_status_string(status).decode()
        if status == BL_ERR_HIP:
            msg += f" (hipError_t {L.bl_last_hip_error()})"
        raise BitLinearError(f"{what}: {msg}")


def _torch():
    import torch
    return torch


def _stream_ptr(t):
    torch = _torch()
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _dev(t, dtype, name):
    torch = _torch()
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise BitLinearError(f"{name} must be a CUDA (HIP) tensor")
    if t.dtype != dtype:
        raise BitLinearError(f"{name} must have dtype {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise BitLinearError(f"{name} must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def packed_bytes(N: int, K: int) -> int:
    return lib().bl_packed_bytes(N, K)


def quantize_weights(W, workspace=None, out=None):
    """W: fp32 [N][K] -> (W_packed int32 [N][K/16] holding the uint32 words,
    gamma fp32 [1]). out: optional (W_packed, gamma) buffers. Calls
    bl_quantize_weights."""
    torch = _torch()
    N, K = W.shape
    L = lib()
    if out is None:
        packed = torch.empty((N, K // 16), dtype=torch.int32, device=W.device)
        gamma = torch.empty(1, dtype=torch.float32, device=W.device)
    else:
        packed, gamma = out
    ws_bytes = L.bl_quantize_weights_workspace_bytes(N, K)
    if workspace is None:
        workspace = torch.empty(max(ws_bytes, 8) // 8, dtype=torch.float64, device=W.device)
    _check(L.bl_quantize_weights(_dev(W, torch.float32, "W"), N, K,
                                 _dev(packed, torch.int32, "W_packed"),
                                 _dev(gamma, torch.float32, "gamma"),
                                 _dev(workspace, workspace.dtype, "workspace"),
                                 workspace.numel() * workspace.element_size(),
                                 _stream_ptr(W)), "bl_quantize_weights")
    return packed, gamma


def quantize_acts(x, rms_gain=None, rms_eps: float = 1e-5, out=None):
    """x: bf16 (or int16 bf16 bits) [M][K] -> (x_q int8 [M][K], x_scale fp32 [M]).
    rms_gain: optional bf16 [K] -> fused RMSNorm. Calls bl_quantize_acts."""
    torch = _torch()
    M, K = x.shape
    if x.dtype == torch.int16:
        x = x.view(torch.bfloat16)
    if out is None:
        xq = torch.empty((M, K), dtype=torch.int8, device=x.device)
        xs = torch.empty(M, dtype=torch.float32, device=x.device)
    else:
        xq, xs = out
    gp = None
    if rms_gain is not None:
        if rms_gain.dtype == torch.int16:
            rms_gain = rms_gain.view(torch.bfloat16)
        gp = _dev(rms_gain, torch.bfloat16, "rms_gain")
    _check(lib().bl_quantize_acts(_dev(x, torch.bfloat16, "x"), M, K, gp, float(rms_eps),
                                  _dev(xq, torch.int8, "x_q"),
                                  _dev(xs, torch.float32, "x_scale"), _stream_ptr(x)),
           "bl_quantize_acts")
    return xq, xs


def quant_bitlinear(x, W_packed, gamma, rms_gain=None, rms_eps: float = 1e-5, out=None):
    """Activation quantisation (optional fused RMSNorm) and the BitLinear product in
    one call: x bf16 [M][K] -> (y fp32 [M][N], x_q int8 [M][K], x_scale fp32 [M]),
    the same bits as quantize_acts followed by bitlinear. out: optional (y, x_q,
    x_scale) buffers. Calls bl_quant_bitlinear."""
    torch = _torch()
    M, K = x.shape
    N = W_packed.shape[0]
    if W_packed.shape[1] * 16 != K:
        raise BitLinearError("W_packed shape does not match K")
    if x.dtype == torch.int16:
        x = x.view(torch.bfloat16)
    if out is None:
        y = torch.empty((M, N), dtype=torch.float32, device=x.device)
        xq = torch.empty((M, K), dtype=torch.int8, device=x.device)
        xs = torch.empty(M, dtype=torch.float32, device=x.device)
    else:
        y, xq, xs = out
    gp = None
    if rms_gain is not None:
        if rms_gain.dtype == torch.int16:
            rms_gain = rms_gain.view(torch.bfloat16)
        gp = _dev(rms_gain, torch.bfloat16, "rms_gain")
    _check(lib().bl_quant_bitlinear(_dev(x, torch.bfloat16, "x"), M, K, gp, float(rms_eps),
                                    _dev(W_packed, torch.int32, "W_packed"),
                                    _dev(gamma, torch.float32, "gamma"), N,
                                    _dev(y, torch.float32, "y"), _dev(xq, torch.int8, "x_q"),
                                    _dev(xs, torch.float32, "x_scale"), _stream_ptr(x)),
           "bl_quant_bitlinear")
    return y, xq, xs


def bitlinear(x_q, x_scale, W_packed, gamma, return_acc: bool = False, path: int = 0,
              out=None, acc_out=None):
    """y[m][n] = (x_q . q^T)[m][n] * x_scale[m] * gamma -> fp32 [M][N].
    path: 0 auto, 1 GEMV, 2 GEMM, 3 wide GEMV (M <= 64), 4 one-token GEMV (M == 1). acc_out: optional int32 [M][N] buffer for the
    exact sums (returned with y, as with return_acc). Calls bl_bitlinear_path."""
    torch = _torch()
    M, K = x_q.shape
    N = W_packed.shape[0]
    if W_packed.shape[1] * 16 != K:
        raise BitLinearError("W_packed shape does not match K")
    y = torch.empty((M, N), dtype=torch.float32, device=x_q.device) if out is None else out
    acc = acc_out
    if acc is None and return_acc:
        acc = torch.empty((M, N), dtype=torch.int32, device=x_q.device)
    _check(lib().bl_bitlinear_path(_dev(x_q, torch.int8, "x_q"),
                                   _dev(x_scale, torch.float32, "x_scale"), M, K,
                                   _dev(W_packed, torch.int32, "W_packed"),
                                   _dev(gamma, torch.float32, "gamma"), N,
                                   _dev(y, torch.float32, "y"),
                                   None if acc is None else _dev(acc, torch.int32, "acc"),
                                   int(path), _stream_ptr(x_q)), "bl_bitlinear")
    return (y, acc) if acc is not None else y


def relu2_glu(gate, up, out=None):
    """h = bf16(relu(gate)^2 * up), same shape. Calls bl_relu2_glu."""
    torch = _torch()
    h = torch.empty(gate.shape, dtype=torch.bfloat16, device=gate.device) if out is None else out
    if gate.shape != up.shape:
        raise BitLinearError("gate and up shapes differ")
    _check(lib().bl_relu2_glu(_dev(gate, torch.float32, "gate"), _dev(up, torch.float32, "up"),
                              gate.numel(), _dev(h, torch.bfloat16, "h"), _stream_ptr(gate)),
           "bl_relu2_glu")
    return h


def bitlinear_pair(x_q, x_scale, W1, gamma1, W2, gamma2, out=None):
    """(y1, y2): two BitLinears sharing x_q in one launch. Calls bl_bitlinear_pair."""
    torch = _torch()
    M, K = x_q.shape
    N1, N2 = W1.shape[0], W2.shape[0]
    if W1.shape[1] * 16 != K or W2.shape[1] * 16 != K:
        raise BitLinearError("packed weight shapes do not match K")
    if out is None:
        y1 = torch.empty((M, N1), dtype=torch.float32, device=x_q.device)
        y2 = torch.empty((M, N2), dtype=torch.float32, device=x_q.device)
    else:
        y1, y2 = out
    _check(lib().bl_bitlinear_pair(_dev(x_q, torch.int8, "x_q"),
                                   _dev(x_scale, torch.float32, "x_scale"), M, K,
                                   _dev(W1, torch.int32, "W1"), _dev(gamma1, torch.float32, "gamma1"),
                                   N1, _dev(y1, torch.float32, "y1"),
                                   _dev(W2, torch.int32, "W2"), _dev(gamma2, torch.float32, "gamma2"),
                                   N2, _dev(y2, torch.float32, "y2"), _stream_ptr(x_q)),
           "bl_bitlinear_pair")
    return y1, y2


def relu2_glu_quant(gate, up, out=None, subln_gain=None, subln_eps: float = 1e-5):
    """(h_q int8, h_scale fp32) of h = bf16(relu(gate)^2 * up). Calls
    bl_relu2_glu_quant, or bl_relu2_glu_subln_quant when subln_gain (bf16
    [K]) is given: the sub-layer RMSNorm before the quantisation."""
    torch = _torch()
    M, K = gate.shape
    if gate.shape != up.shape:
        raise BitLinearError("gate and up shapes differ")
    if out is None:
        hq = torch.empty((M, K), dtype=torch.int8, device=gate.device)
        hs = torch.empty(M, dtype=torch.float32, device=gate.device)
    else:
        hq, hs = out
    args = (_dev(gate, torch.float32, "gate"), _dev(up, torch.float32, "up"), M, K)
    outs = (_dev(hq, torch.int8, "h_q"), _dev(hs, torch.float32, "h_scale"), _stream_ptr(gate))
    if subln_gain is None:
        _check(lib().bl_relu2_glu_quant(*args, *outs), "bl_relu2_glu_quant")
    else:
        if subln_gain.dtype == torch.int16:
            subln_gain = subln_gain.view(torch.bfloat16)
        _check(lib().bl_relu2_glu_subln_quant(*args, _dev(subln_gain, torch.bfloat16, "gain"),
                                              float(subln_eps), *outs),
               "bl_relu2_glu_subln_quant")
    return hq, hs


def _glu_kind(kind) -> int:
    if kind in _GLU_KINDS:
        return _GLU_KINDS[kind]
    if kind in (BL_GLU_RELU2, BL_GLU_SWIGLU):
        return int(kind)
    raise BitLinearError(f"unknown gating kind {kind!r}")


def glu(gate, up, kind="relu2", out=None):
    """h = bf16(act(gate) * up), act = relu^2 ("relu2") or SiLU ("swiglu").
    Calls bl_glu."""
    torch = _torch()
    h = torch.empty(gate.shape, dtype=torch.bfloat16, device=gate.device) if out is None else out
    if gate.shape != up.shape:
        raise BitLinearError("gate and up shapes differ")
    _check(lib().bl_glu(_dev(gate, torch.float32, "gate"), _dev(up, torch.float32, "up"),
                        gate.numel(), _glu_kind(kind), _dev(h, torch.bfloat16, "h"),
                        _stream_ptr(gate)), "bl_glu")
    return h


def glu_quant(gate, up, kind="relu2", subln_gain=None, subln_eps: float = 1e-5, out=None):
    """(h_q int8, h_scale fp32) of the gating of `kind`, with the sub-layer
    RMSNorm when subln_gain (bf16 [K]) is given. Calls bl_glu_quant."""
    torch = _torch()
    M, K = gate.shape
    if gate.shape != up.shape:
        raise BitLinearError("gate and up shapes differ")
    if out is None:
        hq = torch.empty((M, K), dtype=torch.int8, device=gate.device)
        hs = torch.empty(M, dtype=torch.float32, device=gate.device)
    else:
        hq, hs = out
    gp = None
    if subln_gain is not None:
        if subln_gain.dtype == torch.int16:
            subln_gain = subln_gain.view(torch.bfloat16)
        gp = _dev(subln_gain, torch.bfloat16, "gain")
    _check(lib().bl_glu_quant(_dev(gate, torch.float32, "gate"), _dev(up, torch.float32, "up"),
                              M, K, _glu_kind(kind), gp, float(subln_eps),
                              _dev(hq, torch.int8, "h_q"), _dev(hs, torch.float32, "h_scale"),
                              _stream_ptr(gate)), "bl_glu_quant")
    return hq, hs


def ffn_relu2_workspace(M: int, K: int, N_ff: int, device=None):
    """A workspace tensor sized by bl_ffn_relu2_workspace_bytes."""
    torch = _torch()
    n = lib().bl_ffn_relu2_workspace_bytes(M, K, N_ff)
    if n == 0:
        raise BitLinearError("invalid FFN shapes")
    return torch.empty(n, dtype=torch.uint8, device=device)


def ffn_relu2(x, W_gate, gamma_gate, W_up, gamma_up, W_down, gamma_down, workspace=None,
              out=None, subln_gain=None, subln_eps: float = 1e-5):
    """y fp32 [M][K] of one 2B4T-style FFN step on bf16 x. Calls bl_ffn_relu2,
    or bl_ffn_relu2_subln when subln_gain (bf16 [N_ff]) is given: the
    sub-layer RMSNorm on the gated hidden state before the down projection."""
    torch = _torch()
    if x.dtype == torch.int16:
        x = x.view(torch.bfloat16)
    M, K = x.shape
    N_ff = W_gate.shape[0]
    if W_gate.shape[1] * 16 != K or W_up.shape != W_gate.shape or \
            W_down.shape[0] != K or W_down.shape[1] * 16 != N_ff:
        raise BitLinearError("FFN weight shapes do not match")
    if workspace is None:
        workspace = ffn_relu2_workspace(M, K, N_ff, x.device)
    y = torch.empty((M, K), dtype=torch.float32, device=x.device) if out is None else out
    head = (_dev(x, torch.bfloat16, "x"), M, K,
            _dev(W_gate, torch.int32, "W_gate"), _dev(gamma_gate, torch.float32, "gamma_gate"),
            _dev(W_up, torch.int32, "W_up"), _dev(gamma_up, torch.float32, "gamma_up"), N_ff,
            _dev(W_down, torch.int32, "W_down"), _dev(gamma_down, torch.float32, "gamma_down"))
    tail = (_dev(y, torch.float32, "y"), _dev(workspace, torch.uint8, "workspace"),
            workspace.numel(), _stream_ptr(x))
    if subln_gain is None:
        _check(lib().bl_ffn_relu2(*head, *tail), "bl_ffn_relu2")
    else:
        if subln_gain.dtype == torch.int16:
            subln_gain = subln_gain.view(torch.bfloat16)
        _check(lib().bl_ffn_relu2_subln(*head, _dev(subln_gain, torch.bfloat16, "subln_gain"),
                                        float(subln_eps), *tail), "bl_ffn_relu2_subln")
    return y


def ffn_step(x, W_gate, gamma_gate, W_up, gamma_up, W_down, gamma_down, kind="relu2",
             subln_gain=None, subln_eps: float = 1e-5, workspace=None, out=None):
    """y fp32 [M][K] of one gated FFN step with the gating of `kind`
    ("relu2" or "swiglu") and an optional sub-layer RMSNorm. Calls
    bl_ffn_step."""
    torch = _torch()
    if x.dtype == torch.int16:
        x = x.view(torch.bfloat16)
    M, K = x.shape
    N_ff = W_gate.shape[0]
    if W_gate.shape[1] * 16 != K or W_up.shape != W_gate.shape or \
            W_down.shape[0] != K or W_down.shape[1] * 16 != N_ff:
        raise BitLinearError("FFN weight shapes do not match")
    if workspace is None:
        workspace = ffn_relu2_workspace(M, K, N_ff, x.device)
    y = torch.empty((M, K), dtype=torch.float32, device=x.device) if out is None else out
    gp = None
    if subln_gain is not None:
        if subln_gain.dtype == torch.int16:
            subln_gain = subln_gain.view(torch.bfloat16)
        gp = _dev(subln_gain, torch.bfloat16, "subln_gain")
    _check(lib().bl_ffn_step(_dev(x, torch.bfloat16, "x"), M, K,
                             _dev(W_gate, torch.int32, "W_gate"),
                             _dev(gamma_gate, torch.float32, "gamma_gate"),
                             _dev(W_up, torch.int32, "W_up"),
                             _dev(gamma_up, torch.float32, "gamma_up"), N_ff,
                             _dev(W_down, torch.int32, "W_down"),
                             _dev(gamma_down, torch.float32, "gamma_down"), _glu_kind(kind), gp,
                             float(subln_eps), _dev(y, torch.float32, "y"),
                             _dev(workspace, torch.uint8, "workspace"), workspace.numel(),
                             _stream_ptr(x)), "bl_ffn_step")
    return y


def ffn_step_noalloc(x, W_gate, gamma_gate, W_up, gamma_up, W_down, gamma_down, kind="relu2",
                     subln_gain=None, subln_eps: float = 1e-5, out=None):
    """ffn_step without a workspace: the library's fixed per-device scratch
    (up to 8 MiB of FFN workspace). Calls bl_ffn_step_noalloc."""
    torch = _torch()
    if x.dtype == torch.int16:
        x = x.view(torch.bfloat16)
    M, K = x.shape
    N_ff = W_gate.shape[0]
    if W_gate.shape[1] * 16 != K or W_up.shape != W_gate.shape or \
            W_down.shape[0] != K or W_down.shape[1] * 16 != N_ff:
        raise BitLinearError("FFN weight shapes do not match")
    y = torch.empty((M, K), dtype=torch.float32, device=x.device) if out is None else out
    gp = None
    if subln_gain is not None:
        if subln_gain.dtype == torch.int16:
            subln_gain = subln_gain.view(torch.bfloat16)
        gp = _dev(subln_gain, torch.bfloat16, "subln_gain")
    _check(lib().bl_ffn_step_noalloc(_dev(x, torch.bfloat16, "x"), M, K,
                                     _dev(W_gate, torch.int32, "W_gate"),
                                     _dev(gamma_gate, torch.float32, "gamma_gate"),
                                     _dev(W_up, torch.int32, "W_up"),
                                     _dev(gamma_up, torch.float32, "gamma_up"), N_ff,
                                     _dev(W_down, torch.int32, "W_down"),
                                     _dev(gamma_down, torch.float32, "gamma_down"),
                                     _glu_kind(kind), gp, float(subln_eps),
                                     _dev(y, torch.float32, "y"), _stream_ptr(x)),
           "bl_ffn_step_noalloc")
    return y


# ------------------------------------------------- other weight formats ----
# 1 bit per {-1, +1} weight (the original BitNet's binary weights) and five
# ternary weights per byte (1.6 bits); decode products for M <= 16.

def quantize_weights_binary(W, workspace=None, out=None):
    """W fp32 [N][K] -> (W_bits int32 [N][4*ceil(K/128)] holding uint32 words,
    gamma fp32 [1]). out: optional (W_bits, gamma) buffers. Calls
    bl_quantize_weights_binary."""
    torch = _torch()
    N, K = W.shape
    L = lib()
    nbytes = L.bl_packed_bytes_binary(N, K)
    if nbytes == 0:
        raise BitLinearError("invalid weight shape")
    if out is None:
        bits = torch.empty((N, nbytes // (4 * N)), dtype=torch.int32, device=W.device)
        gamma = torch.empty(1, dtype=torch.float32, device=W.device)
    else:
        bits, gamma = out
    ws_bytes = L.bl_quantize_weights_workspace_bytes(N, K)
    if workspace is None:
        workspace = torch.empty(max(ws_bytes, 8) // 8, dtype=torch.float64, device=W.device)
    _check(L.bl_quantize_weights_binary(_dev(W, torch.float32, "W"), N, K,
                                        _dev(bits, torch.int32, "W_bits"),
                                        _dev(gamma, torch.float32, "gamma"),
                                        _dev(workspace, workspace.dtype, "workspace"),
                                        workspace.numel() * workspace.element_size(),
                                        _stream_ptr(W)), "bl_quantize_weights_binary")
    return bits, gamma


def pack_base3(W_packed, K: int, out=None):
    """2-bit packed [N][K/16] -> uint8 [N][16*ceil(ceil(K/5)/16)], five ternary
    weights per byte (into `out` when given). Calls bl_pack_base3."""
    torch = _torch()
    N = W_packed.shape[0]
    L = lib()
    nbytes = L.bl_packed_bytes_base3(N, K)
    if nbytes == 0 or W_packed.shape[1] * 16 != K:
        raise BitLinearError("invalid weight shape")
    if out is None:
        out = torch.empty((N, nbytes // N), dtype=torch.uint8, device=W_packed.device)
    _check(L.bl_pack_base3(_dev(W_packed, torch.int32, "W_packed"), N, K,
                           _dev(out, torch.uint8, "W3"), _stream_ptr(W_packed)), "bl_pack_base3")
    return out


def _other_product(fn, name, x_q, x_scale, W, wdtype, gamma, N, return_acc, out, acc_out=None):
    torch = _torch()
    M, K = x_q.shape
    y = torch.empty((M, N), dtype=torch.float32, device=x_q.device) if out is None else out
    acc = acc_out
    if acc is None and return_acc:
        acc = torch.empty((M, N), dtype=torch.int32, device=x_q.device)
    return_acc = acc is not None
    _check(fn(_dev(x_q, torch.int8, "x_q"), _dev(x_scale, torch.float32, "x_scale"), M, K,
              _dev(W, wdtype, "W"), _dev(gamma, torch.float32, "gamma"), N,
              _dev(y, torch.float32, "y"),
              None if acc is None else _dev(acc, torch.int32, "acc"), _stream_ptr(x_q)), name)
    return (y, acc) if return_acc else y


def bitlinear_binary(x_q, x_scale, W_bits, gamma, return_acc: bool = False, out=None,
                     acc_out=None):
    """BitLinear with 1-bit weights (M <= 16). Calls bl_bitlinear_binary."""
    torch = _torch()
    return _other_product(lib().bl_bitlinear_binary, "bl_bitlinear_binary", x_q, x_scale,
                          W_bits, torch.int32, gamma, W_bits.shape[0], return_acc, out, acc_out)


def bitlinear_base3(x_q, x_scale, W3, gamma, return_acc: bool = False, out=None, acc_out=None):
    """BitLinear with base-3 weights (M <= 16). Calls bl_bitlinear_base3."""
    torch = _torch()
    return _other_product(lib().bl_bitlinear_base3, "bl_bitlinear_base3", x_q, x_scale, W3,
                          torch.uint8, gamma, W3.shape[0], return_acc, out, acc_out)


# ------------------------------------------- straight-through backward ----

def pack_ste_t(W_packed, K: int, out=None):
    """2-bit packed [N][K/16] -> transposed codes uint8 [K][row bytes], four n
    per byte, for the backward pass (into `out` when given). Calls
    bl_pack_ste_t."""
    torch = _torch()
    N = W_packed.shape[0]
    L = lib()
    nbytes = L.bl_ste_t_bytes(N, K)
    if nbytes == 0 or W_packed.shape[1] * 16 != K:
        raise BitLinearError("invalid weight shape")
    qT = torch.empty((K, nbytes // K), dtype=torch.uint8, device=W_packed.device) \
        if out is None else out
    _check(L.bl_pack_ste_t(_dev(W_packed, torch.int32, "W_packed"), N, K,
                           _dev(qT, torch.uint8, "qT"), _stream_ptr(W_packed)), "bl_pack_ste_t")
    return qT


def ste_backward_dx(dy, qT, gamma, N: int, out=None):
    """dx fp32 [M][K] = gamma * dy . q for bf16 dy [M][N]. Calls bl_ste_backward_dx."""
    torch = _torch()
    if dy.dtype == torch.int16:
        dy = dy.view(torch.bfloat16)
    M = dy.shape[0]
    K = qT.shape[0]
    if dy.shape[1] != N:
        raise BitLinearError("dy shape does not match N")
    dx = torch.empty((M, K), dtype=torch.float32, device=dy.device) if out is None else out
    _check(lib().bl_ste_backward_dx(_dev(dy, torch.bfloat16, "dy"), M, N,
                                    _dev(qT, torch.uint8, "qT"),
                                    _dev(gamma, torch.float32, "gamma"), K,
                                    _dev(dx, torch.float32, "dx"), _stream_ptr(dy)),
           "bl_ste_backward_dx")
    return dx


def ste_dw_workspace(M: int, N: int, K: int, device=None):
    """A workspace tensor sized by bl_ste_dw_workspace_bytes."""
    torch = _torch()
    n = lib().bl_ste_dw_workspace_bytes(M, N, K)
    if n == 0:
        raise BitLinearError("invalid STE shapes")
    return torch.empty(n, dtype=torch.uint8, device=device)


def ste_backward_dw(dy, x_q, x_scale, workspace=None, out=None):
    """dW fp32 [N][K] = dy^T . (x_q * x_scale) for bf16 dy [M][N], int8 x_q
    [M][K], fp32 x_scale [M]. Calls bl_ste_backward_dw."""
    torch = _torch()
    if dy.dtype == torch.int16:
        dy = dy.view(torch.bfloat16)
    M, N = dy.shape
    K = x_q.shape[1]
    if x_q.shape[0] != M or x_scale.shape != (M,):
        raise BitLinearError("dy, x_q and x_scale shapes do not match")
    if workspace is None:
        workspace = ste_dw_workspace(M, N, K, dy.device)
    dW = torch.empty((N, K), dtype=torch.float32, device=dy.device) if out is None else out
    _check(lib().bl_ste_backward_dw(_dev(dy, torch.bfloat16, "dy"), M, N,
                                    _dev(x_q, torch.int8, "x_q"),
                                    _dev(x_scale, torch.float32, "x_scale"), K,
                                    _dev(dW, torch.float32, "dW"),
                                    _dev(workspace, torch.uint8, "workspace"),
                                    workspace.numel(), _stream_ptr(dy)), "bl_ste_backward_dw")
    return dW


# ---------------------------------------------------------- calibration ----
# Measured ceilings (a read-only stream, a copy, an int8 matrix-core loop);
# they compute nothing of the method.

def _any_dev(t, name):
    torch = _torch()
    if not isinstance(t, torch.Tensor) or not t.is_cuda or not t.is_contiguous():
        raise BitLinearError(f"{name} must be a contiguous CUDA (HIP) tensor")
    return ctypes.c_void_p(t.data_ptr())


def calib_read(src, sink):
    """Reads every byte of `src` once (bl_calib_read); sink: int32 device tensor."""
    torch = _torch()
    _check(lib().bl_calib_read(_any_dev(src, "src"), src.numel() * src.element_size(),
                               _dev(sink, torch.int32, "sink"), _stream_ptr(src)),
           "bl_calib_read")


def calib_copy(dst, src):
    """dst[:] = src bytewise (bl_calib_copy); equal byte sizes required."""
    nb = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() != nb:
        raise BitLinearError("calib_copy: dst and src sizes differ")
    _check(lib().bl_calib_copy(_any_dev(dst, "dst"), _any_dev(src, "src"), nb,
                               _stream_ptr(src)), "bl_calib_copy")


def calib_mfma_sink(device=None):
    torch = _torch()
    return torch.empty(lib().bl_calib_mfma_i8_sink_elems(), dtype=torch.int32, device=device)


def calib_mfma_i8(iters: int, sink) -> int:
    """Runs the int8 matrix-core loop (bl_calib_mfma_i8); returns its op count."""
    torch = _torch()
    L = lib()
    if sink.numel() < L.bl_calib_mfma_i8_sink_elems():
        raise BitLinearError("calib_mfma_i8: sink too small")
    _check(L.bl_calib_mfma_i8(iters, _dev(sink, torch.int32, "sink"), _stream_ptr(sink)),
           "bl_calib_mfma_i8")
    return L.bl_calib_mfma_i8_ops(iters)
