"""C-ABI checks that need no GPU: the library loads, exports every function
include/bitlinear.h declares, and rejects invalid arguments on the host before
anything is enqueued."""
import ctypes
import os
import re

import pytest

import ternary_weight_linear_quant_amd as bl

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "bitlinear.h")


@pytest.fixture(scope="session")
def L():
    if not os.path.exists(bl.library_path()):
        from ternary_weight_linear_quant_amd import build
        build.build()
    return bl.lib()


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(bl_\w+)\s*\(", text)))


def test_header_declares_the_three_calls():
    names = _declared_functions()
    for n in ("bl_quantize_weights", "bl_quantize_acts", "bl_bitlinear"):
        assert n in names


def test_library_exports_every_declared_symbol(L):
    names = _declared_functions()
    assert len(names) >= 10
    for n in names:
        assert hasattr(L, n), f"{n} not exported"


def test_binding_signatures_cover_header():
    assert set(_declared_functions()) == set(bl._SIGNATURES)


def test_host_helpers(L):
    assert L.bl_packed_bytes(28672, 8192) == 28672 * 8192 // 4
    assert L.bl_packed_bytes(10, 100) == 0
    assert L.bl_packed_bytes(0, 64) == 0
    assert L.bl_quantize_weights_workspace_bytes(2560, 6912) == 8 * 2560
    assert L.bl_status_string(0) == b"BL_OK"
    assert L.bl_status_string(1) == b"BL_ERR_INVALID_ARG"
    assert L.bl_status_string(99) == b"BL_ERR_UNKNOWN"
    assert L.bl_version().startswith(b"bitlinear")


P = ctypes.c_void_p
A = P(0x100000)        # aligned fake address, never dereferenced
MIS = P(0x100001)      # misaligned
# Distinct, non-overlapping fake buffers for the product's operands.
X, S, W, G, Y = (P(0x1000000 * i) for i in range(1, 6))


def test_invalid_arguments_rejected_before_launch(L):
    E = bl.BL_ERR_INVALID_ARG
    # null pointers
    assert L.bl_bitlinear(None, S, 1, 64, W, G, 16, Y, None, None) == E
    assert L.bl_bitlinear(X, S, 1, 64, W, G, 16, None, None, None) == E
    # shapes
    assert L.bl_bitlinear(X, S, 0, 64, W, G, 16, Y, None, None) == E
    assert L.bl_bitlinear(X, S, 1, 100, W, G, 16, Y, None, None) == E
    assert L.bl_bitlinear(X, S, 1, 32, W, G, 16, Y, None, None) == E
    assert L.bl_bitlinear(X, S, 1, 64, W, G, 0, Y, None, None) == E
    assert L.bl_bitlinear(X, S, 1 << 20, 1 << 12, W, G, 16, Y, None, None) == E
    # alignment
    assert L.bl_bitlinear(P(0x1000001), S, 1, 64, W, G, 16, Y, None, None) == E
    assert L.bl_bitlinear(X, S, 1, 64, P(0x3000001), G, 16, Y, None, None) == E
    # outputs aliasing inputs
    assert L.bl_bitlinear(A, P(0x200000), 1, 64, P(0x300000), P(0x400000), 16, A, None, None) == E
    assert L.bl_bitlinear(P(0x100000), P(0x200000), 1, 64, P(0x300000), P(0x400000), 16,
                          P(0x500000), P(0x500020), None) == E
    assert L.bl_bitlinear(P(0x100000), P(0x200000), 1, 64, P(0x300000), P(0x400000), 16,
                          P(0x3000F0), None, None) == E
    # path selection
    assert L.bl_bitlinear_path(X, S, 1, 64, W, G, 16, Y, None, 5, None) == E
    assert L.bl_bitlinear_path(X, S, 1, 64, W, G, 16, Y, None, -1, None) == E
    assert L.bl_bitlinear_path(X, S, 2, 64, W, G, 16, Y, None, 4, None) == E     # one token only
    assert L.bl_bitlinear_path(X, S, 1, 65600, W, G, 16, Y, None, 4, None) == E  # K > 65536
    assert L.bl_bitlinear_path(X, S, 65, 64, W, G, 16, Y, None, 3, None) == E
    assert L.bl_bitlinear_path(X, S, 17, 64, W, G, 16, Y, None, 1, None) == E
    assert L.bl_bitlinear_path(X, S, 16, 16384, W, G, 16, Y, None, 1, None) == E
    # act quant + product in one call: x, gain, W, gamma in; y, x_q, x_scale out
    XB, GN, QO, SO = P(0x6000000), P(0x7000000), P(0x8000000), P(0x9000000)
    assert L.bl_quant_bitlinear(None, 1, 64, None, 0.0, W, G, 16, Y, QO, SO, None) == E
    assert L.bl_quant_bitlinear(XB, 1, 64, None, 0.0, W, G, 16, Y, None, SO, None) == E
    assert L.bl_quant_bitlinear(XB, 1, 64, None, 0.0, W, G, 16, Y, QO, None, None) == E
    assert L.bl_quant_bitlinear(XB, 1, 96, None, 0.0, W, G, 16, Y, QO, SO, None) == E
    assert L.bl_quant_bitlinear(XB, 0, 64, None, 0.0, W, G, 16, Y, QO, SO, None) == E
    assert L.bl_quant_bitlinear(XB, 1, 64, None, 0.0, W, G, 0, Y, QO, SO, None) == E
    assert L.bl_quant_bitlinear(MIS, 1, 64, None, 0.0, W, G, 16, Y, QO, SO, None) == E
    assert L.bl_quant_bitlinear(XB, 1, 64, None, 0.0, W, G, 16, Y, P(0x8000008), SO, None) == E
    assert L.bl_quant_bitlinear(XB, 1, 64, GN, 0.0, W, G, 16, Y, QO, SO, None) == E    # eps
    assert L.bl_quant_bitlinear(XB, 1, 64, MIS, 1e-5, W, G, 16, Y, QO, SO, None) == E
    # outputs overlapping each other or an input
    assert L.bl_quant_bitlinear(XB, 1, 64, None, 0.0, W, G, 16, Y, P(0x5000030), SO, None) == E
    assert L.bl_quant_bitlinear(XB, 1, 64, None, 0.0, W, G, 16, Y, QO, P(0x8000030), None) == E
    assert L.bl_quant_bitlinear(XB, 1, 64, None, 0.0, W, G, 16, P(0x6000070), QO, SO, None) == E
    assert L.bl_quant_bitlinear(XB, 1, 64, GN, 1e-5, W, G, 16, Y, P(0x7000070), SO, None) == E
    assert L.bl_quant_bitlinear(XB, 1, 64, None, 0.0, W, G, 16, Y, QO, P(0x4000000), None) == E
    # weight quantisation
    assert L.bl_quantize_weights(A, 16, 64, A, A, A, 8 * 15, None) == E
    assert L.bl_quantize_weights(A, 16, 64, A, A, P(0x100004), 8 * 16, None) == E
    assert L.bl_quantize_weights(A, 16, 48, A, A, A, 8 * 16, None) == E
    assert L.bl_quantize_weights(None, 16, 64, A, A, A, 8 * 16, None) == E
    # activation quantisation
    assert L.bl_quantize_acts(A, 1, 64, A, 0.0, A, A, None) == E
    assert L.bl_quantize_acts(A, 1, 64, MIS, 1e-5, A, A, None) == E
    assert L.bl_quantize_acts(MIS, 1, 64, None, 0.0, A, A, None) == E
    assert L.bl_quantize_acts(A, 1, 96, None, 0.0, A, A, None) == E
    # glue
    assert L.bl_relu2_glu(A, A, 0, A, None) == E
    assert L.bl_relu2_glu(A, MIS, 4, A, None) == E
    assert L.bl_relu2_glu_quant(A, A, 1, 100, A, A, None) == E
    assert L.bl_relu2_glu_quant(A, A, 0, 64, A, A, None) == E
    assert L.bl_relu2_glu_quant(A, MIS, 1, 64, A, A, None) == E
    assert L.bl_relu2_glu_quant(A, A, 1, 64, A, None, None) == E
    # gating kinds: only BL_GLU_RELU2 (0) and BL_GLU_SWIGLU (1)
    assert L.bl_glu(A, A, 4, 2, A, None) == E
    assert L.bl_glu(A, A, 4, -1, A, None) == E
    assert L.bl_glu(A, A, 0, 1, A, None) == E
    assert L.bl_glu_quant(A, A, 1, 64, 2, None, 0.0, A, A, None) == E
    assert L.bl_glu_quant(A, A, 1, 64, 1, MIS, 1e-5, A, A, None) == E
    assert L.bl_glu_quant(A, A, 1, 64, 1, A, 0.0, A, A, None) == E
    # glue with the sub-layer norm: the gain is required, aligned, eps > 0
    assert L.bl_relu2_glu_subln_quant(A, A, 1, 64, None, 1e-5, A, A, None) == E
    assert L.bl_relu2_glu_subln_quant(A, A, 1, 64, MIS, 1e-5, A, A, None) == E
    assert L.bl_relu2_glu_subln_quant(A, A, 1, 64, A, 0.0, A, A, None) == E
    assert L.bl_relu2_glu_subln_quant(A, A, 1, 100, A, 1e-5, A, A, None) == E
    # fused FFN step
    WS = P(0x200000)  # 256-byte aligned
    need = L.bl_ffn_relu2_workspace_bytes(4, 2560, 6912)
    assert need >= 2 * 4 * 6912
    assert L.bl_ffn_relu2_workspace_bytes(4, 100, 6912) == 0
    assert L.bl_ffn_relu2(A, 4, 2560, A, A, A, A, 6912, A, A, A, WS, need - 1, None) == E
    assert L.bl_ffn_relu2(A, 4, 2560, A, A, A, A, 6912, A, A, A, P(0x200010), need, None) == E
    assert L.bl_ffn_relu2(A, 4, 2560, A, A, None, A, 6912, A, A, A, WS, need, None) == E
    assert L.bl_ffn_relu2(A, 4, 2560, A, A, A, A, 6900, A, A, A, WS, need, None) == E
    assert L.bl_ffn_relu2(MIS, 4, 2560, A, A, A, A, 6912, A, A, A, WS, need, None) == E
    assert L.bl_ffn_relu2_subln(A, 4, 2560, A, A, A, A, 6912, A, A, None, 1e-5, A, WS, need,
                                None) == E
    assert L.bl_ffn_relu2_subln(A, 4, 2560, A, A, A, A, 6912, A, A, MIS, 1e-5, A, WS, need,
                                None) == E
    assert L.bl_ffn_relu2_subln(A, 4, 2560, A, A, A, A, 6912, A, A, A, -1.0, A, WS, need,
                                None) == E
    assert L.bl_ffn_relu2_subln(A, 4, 2560, A, A, A, A, 6912, A, A, A, 1e-5, A, WS, need - 1,
                                None) == E
    assert L.bl_ffn_step(A, 4, 2560, A, A, A, A, 6912, A, A, 3, None, 0.0, A, WS, need,
                         None) == E
    assert L.bl_ffn_step(A, 4, 2560, A, A, A, A, 6912, A, A, 1, A, 0.0, A, WS, need,
                         None) == E
    # no-allocation FFN step: null pointers, bad shapes, workspace past the 8 MiB scratch
    assert L.bl_ffn_step_noalloc(None, 4, 2560, A, A, A, A, 6912, A, A, 0, None, 0.0, A,
                                 None) == E
    assert L.bl_ffn_step_noalloc(A, 4, 2560, A, A, A, A, 6912, A, A, 0, None, 0.0, None,
                                 None) == E
    assert L.bl_ffn_step_noalloc(A, 4, 2560, A, A, A, A, 6900, A, A, 0, None, 0.0, A,
                                 None) == E
    assert L.bl_ffn_step_noalloc(A, 4, 2560, A, A, A, A, 6912, A, A, 3, None, 0.0, A,
                                 None) == E
    assert L.bl_ffn_step_noalloc(A, 26, 8192, A, A, A, A, 28672, A, A, 0, None, 0.0, A,
                                 None) == E
    assert L.bl_ffn_step_noalloc(A, 107, 2560, A, A, A, A, 6912, A, A, 0, None, 0.0, A,
                                 None) == E
    assert L.bl_ffn_step_noalloc(MIS, 4, 2560, A, A, A, A, 6912, A, A, 0, None, 0.0, A,
                                 None) == E
    assert L.bl_ffn_step_noalloc(A, 4, 2560, A, A, A, A, 6912, A, A, 1, A, -1.0, A,
                                 None) == E
    # straight-through weight gradient
    need_dw = L.bl_ste_dw_workspace_bytes(100, 64, 128)
    assert need_dw == 4 * 64 * 128 + 2 * 128 * 128
    # Shapes whose last round of 128 x 256 tiles splits its stages add the
    # fp32 partial tiles: splits x tail row tiles x 128 rows x K x 4 bytes.
    assert L.bl_ste_dw_workspace_bytes(512, 2600, 3328) == \
        4 * 2600 * 512 + 2 * 3328 * 512 + 2 * 256 * 3328 * 4
    assert L.bl_ste_dw_workspace_bytes(4096, 6912, 2560) == \
        4 * 6912 * 4096 + 2 * 2560 * 4096 + 8 * 384 * 2560 * 4
    assert L.bl_ste_dw_workspace_bytes(4096, 2560, 6912) == \
        4 * 2560 * 4096 + 2 * 6912 * 4096 + 4 * 256 * 6912 * 4
    assert L.bl_ste_dw_workspace_bytes(33, 2600, 3328) == 4 * 2600 * 64 + 2 * 3328 * 64
    assert L.bl_ste_dw_workspace_bytes(100, 60, 128) == 0          # N % 8
    assert L.bl_ste_dw_workspace_bytes(100, 64, 96) == 0           # K % 64
    assert L.bl_ste_dw_workspace_bytes(0, 64, 128) == 0
    assert L.bl_ste_backward_dw(None, 100, 64, A, A, 128, A, WS, need_dw, None) == E
    assert L.bl_ste_backward_dw(A, 100, 64, A, A, 128, A, None, need_dw, None) == E
    assert L.bl_ste_backward_dw(A, 100, 64, A, A, 128, A, WS, need_dw - 1, None) == E
    assert L.bl_ste_backward_dw(A, 100, 60, A, A, 128, A, WS, need_dw, None) == E
    assert L.bl_ste_backward_dw(MIS, 100, 64, A, A, 128, A, WS, need_dw, None) == E
    assert L.bl_ste_backward_dw(A, 100, 64, A, A, 128, A, P(0x500010), need_dw, None) == E
    # pair
    assert L.bl_bitlinear_pair(A, A, 1, 64, A, A, 16, A, None, A, 16, A, None) == E
    assert L.bl_bitlinear_pair(A, A, 1, 64, A, A, 16, A, A, A, 0, A, None) == E
    assert L.bl_bitlinear_pair(A, A, 1, 96, A, A, 16, A, A, A, 16, A, None) == E
    assert L.bl_bitlinear_pair(A, A, 1, 64, MIS, A, 16, A, A, A, 16, A, None) == E


def test_other_formats_host_side(L):
    E = bl.BL_ERR_INVALID_ARG
    assert L.bl_packed_bytes_binary(16, 8640) == 16 * 16 * 68
    assert L.bl_packed_bytes_binary(16, 8192) == 16 * 8192 // 8
    assert L.bl_packed_bytes_base3(16, 6912) == 16 * 1392
    assert L.bl_packed_bytes_base3(16, 2560) == 16 * 512
    assert L.bl_packed_bytes_base3(16, 100) == 0
    ws = L.bl_quantize_weights_workspace_bytes(16, 64)
    assert L.bl_quantize_weights_binary(None, 16, 64, W, G, S, ws, None) == E
    assert L.bl_quantize_weights_binary(X, 16, 48, W, G, S, ws, None) == E
    assert L.bl_quantize_weights_binary(X, 16, 64, W, G, S, ws - 1, None) == E
    assert L.bl_pack_base3(W, 16, 64, P(0x3000010), None) == E               # overlapping
    assert L.bl_pack_base3(W, 16, 64, P(0x6000001), None) == E               # misaligned
    for f in (L.bl_bitlinear_binary, L.bl_bitlinear_base3):
        assert f(X, S, 17, 64, W, G, 16, Y, None, None) == E                  # M > 16
        assert f(X, S, 16, 16384, W, G, 16, Y, None, None) == E               # LDS bound
        assert f(X, S, 1, 64, W, G, 16, P(0x3000000), None, None) == E        # y aliases W
        assert f(X, S, 1, 100, W, G, 16, Y, None, None) == E
        assert f(None, S, 1, 64, W, G, 16, Y, None, None) == E


def test_ste_backward_host_side(L):
    E = bl.BL_ERR_INVALID_ARG
    assert L.bl_ste_t_bytes(6912, 2560) == 2560 * 1728
    assert L.bl_ste_t_bytes(37, 64) == 64 * 16
    assert L.bl_ste_t_bytes(16, 100) == 0
    assert L.bl_pack_ste_t(W, 16, 64, P(0x3000010), None) == E                 # overlapping
    assert L.bl_pack_ste_t(W, 16, 48, P(0x6000000), None) == E
    assert L.bl_ste_backward_dx(X, 4, 12, W, G, 64, Y, None) == E              # N % 8
    assert L.bl_ste_backward_dx(X, 4, 0, W, G, 64, Y, None) == E
    assert L.bl_ste_backward_dx(X, 0, 16, W, G, 64, Y, None) == E
    assert L.bl_ste_backward_dx(X, 4, 16, W, G, 96, Y, None) == E              # K % 64
    assert L.bl_ste_backward_dx(P(0x1000008), 4, 16, W, G, 64, Y, None) == E   # misaligned dy
    assert L.bl_ste_backward_dx(X, 4, 16, W, G, 64, P(0x1000040), None) == E   # dx over dy
    assert L.bl_ste_backward_dx(None, 4, 16, W, G, 64, Y, None) == E


def test_calibration_arguments(L):
    E = bl.BL_ERR_INVALID_ARG
    assert L.bl_calib_read(A, 8, A, None) == E
    assert L.bl_calib_read(A, 24, A, None) == E
    assert L.bl_calib_read(MIS, 32, A, None) == E
    assert L.bl_calib_read(None, 32, A, None) == E
    assert L.bl_calib_copy(A, A, 32, None) == E                  # overlapping
    assert L.bl_calib_copy(P(0x100010), A, 32, None) == E       # overlapping
    assert L.bl_calib_copy(P(0x200000), MIS, 32, None) == E
    assert L.bl_calib_mfma_i8(0, A, None) == E
    assert L.bl_calib_mfma_i8((1 << 24) + 1, A, None) == E
    assert L.bl_calib_mfma_i8_ops(0) == 0
    # 8 instructions x 32*32*32 multiply-adds x 2 ops x 4 waves x blocks
    blocks = L.bl_calib_mfma_i8_sink_elems() // 256
    assert L.bl_calib_mfma_i8_ops(10) == 10 * 8 * 2 * 32 ** 3 * 4 * blocks


@pytest.mark.parametrize("M,K,N,path,kernel", [
    (1, 8192, 28672, 0, 4), (1, 28672, 8192, 0, 4), (1, 2560, 2560, 0, 4),
    (1, 8640, 3200, 0, 1),     # one-token GEMV supported but not preferred: the GEMV
    (1, 11008, 4096, 0, 1), (4, 2560, 6912, 0, 1), (16, 6912, 2560, 0, 1),
    (17, 28672, 8192, 0, 3), (24, 8192, 28672, 0, 3), (48, 2560, 6912, 0, 2),
    (64, 8192, 28672, 0, 2), (2048, 8192, 28672, 0, 2),
    (1, 8640, 3200, 4, 4), (1, 8640, 3200, 2, 2), (16, 6912, 2560, 3, 3),
    (1, 100, 16, 0, -1), (2, 64, 16, 4, -1), (17, 64, 16, 1, -1), (1, 64, 16, 5, -1),
    (65, 64, 16, 3, -1), (1, 65600, 16, 4, -1),
])
def test_bitlinear_kernel_choice(L, M, K, N, path, kernel):
    """The automatic rule documented for bl_bitlinear_path, on the host."""
    assert L.bl_bitlinear_choice(M, K, N, path) == kernel


def test_no_device_status(L):
    import torch
    if torch.cuda.device_count() > 0:
        pytest.skip("a GPU is visible; this checks the no-device path")
    D = bl.BL_ERR_NO_DEVICE
    assert L.bl_bitlinear(X, S, 1, 64, W, G, 16, Y, None, None) == D
    assert L.bl_quantize_acts(A, 1, 64, None, 0.0, A, A, None) == D
    assert L.bl_quantize_weights(A, 16, 64, A, A, A, 8 * 16, None) == D
    assert L.bl_relu2_glu(A, A, 4, A, None) == D
    assert L.bl_relu2_glu_quant(A, A, 1, 64, A, A, None) == D
    assert L.bl_bitlinear_pair(A, A, 1, 64, A, A, 16, A, A, A, 16, A, None) == D
    assert L.bl_bitlinear_binary(X, S, 1, 64, W, G, 16, Y, None, None) == D
    assert L.bl_bitlinear_base3(X, S, 1, 64, W, G, 16, Y, None, None) == D
    assert L.bl_pack_base3(W, 16, 64, P(0x6000000), None) == D
    assert L.bl_ste_backward_dx(X, 4, 16, W, G, 64, Y, None) == D
    assert L.bl_pack_ste_t(W, 16, 64, P(0x6000000), None) == D
    need = L.bl_ffn_relu2_workspace_bytes(1, 256, 1024)
    assert L.bl_ffn_relu2(A, 1, 256, A, A, A, A, 1024, A, A, A, P(0x200000), need, None) == D
    assert L.bl_ffn_relu2_subln(A, 1, 256, A, A, A, A, 1024, A, A, A, 1e-5, A, P(0x200000),
                                need, None) == D
    assert L.bl_relu2_glu_subln_quant(A, A, 1, 64, A, 1e-5, A, A, None) == D
    assert L.bl_glu(A, A, 4, 1, A, None) == D
    assert L.bl_glu_quant(A, A, 1, 64, 1, None, 0.0, A, A, None) == D
    assert L.bl_ffn_step(A, 1, 256, A, A, A, A, 1024, A, A, 1, None, 0.0, A, P(0x200000),
                         need, None) == D
    assert L.bl_ffn_step_noalloc(A, 25, 8192, A, A, A, A, 28672, A, A, 0, None, 0.0, A,
                                 None) == D
    need_dw = L.bl_ste_dw_workspace_bytes(100, 64, 128)
    assert L.bl_ste_backward_dw(P(0x100000), 100, 64, P(0x110000), P(0x120000), 128,
                                P(0x130000), P(0x200000), need_dw, None) == D
    assert L.bl_ffn_step_noalloc(A, 106, 2560, A, A, A, A, 6912, A, A, 0, None, 0.0, A,
                                 None) == D
    XB, GN, QO, SO = P(0x6000000), P(0x7000000), P(0x8000000), P(0x9000000)
    assert L.bl_quant_bitlinear(XB, 1, 64, None, 0.0, W, G, 16, Y, QO, SO, None) == D
    assert L.bl_quant_bitlinear(XB, 3, 8192, GN, 1e-5, W, G, 16, Y, QO, SO, None) == D


def test_binding_fails_loudly_without_gpu():
    import torch
    if torch.cuda.device_count() > 0:
        pytest.skip("a GPU is visible")
    with pytest.raises(bl.BitLinearError):
        bl.quantize_weights(torch.zeros(16, 64))


def test_binding_refuses_a_library_built_from_other_sources(monkeypatch):
    """bl.lib() compares the digest embedded at build time with the source
    tree's; a mismatch (a stale build) raises instead of loading."""
    import ternary_weight_linear_quant_amd as blm
    from ternary_weight_linear_quant_amd import build as blbuild
    built = blm.lib().bl_source_sha256().decode()
    assert built == blbuild.source_sha256()
    monkeypatch.setattr(blm, "_lib", None)
    monkeypatch.setattr(blbuild, "source_sha256", lambda: "0" * 64)
    with pytest.raises(blm.BitLinearError, match="built from other sources"):
        blm.lib()


def test_oracle_library_carries_its_source_digest():
    """The oracle's library on disk carries the digest of oracle.c, oracle.h
    and its flags (the loader rebuilds on any difference, not by mtime)."""
    import oracle
    oracle._load()
    assert oracle._built_sha256() == oracle.source_sha256()
