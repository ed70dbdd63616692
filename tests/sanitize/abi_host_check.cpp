// Host-side argument validation of the C ABI under AddressSanitizer and
// UndefinedBehaviorSanitizer. Built from the library's sources compiled for
// the host only (no device code), it calls every entry point with invalid
// arguments (expecting BL_ERR_INVALID_ARG) and with valid ones on a machine
// without a GPU (expecting BL_ERR_NO_DEVICE), including shapes at the edges
// of int64 where a careless size product would overflow. The pointers are
// never dereferenced by the validation. Exit 0 on success, 77 when a GPU is
// visible (the valid calls would launch), 1 on a failed check.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdio>

#include "../../include/bitlinear.h"

static int g_failures = 0;

#define EXPECT(call, want)                                                              \
    do {                                                                                \
        const int got_ = (int)(call);                                                   \
        if (got_ != (want)) {                                                           \
            std::fprintf(stderr, "line %d: %s returned %d, expected %d\n", __LINE__, #call, \
                         got_, (int)(want));                                            \
            ++g_failures;                                                               \
        }                                                                               \
    } while (0)

template <class T = void>
static T* P(uintptr_t a) { return reinterpret_cast<T*>(a); }

int main() {
    int n = 0;
    if (hipGetDeviceCount(&n) == hipSuccess && n > 0) {
        std::puts("a GPU is visible: this check runs where there is none");
        return 77;
    }
    const int E = BL_ERR_INVALID_ARG, D = BL_ERR_NO_DEVICE;
    const int64_t BIG = INT64_MAX, NEG = -5;
    // Distinct, 256-byte aligned stand-ins for device buffers.
    auto* x = P<uint16_t>(0x1000000);
    auto* xq = P<int8_t>(0x2000000);
    auto* xs = P<float>(0x3000000);
    auto* W = P<uint32_t>(0x4000000);
    auto* g = P<float>(0x5000000);
    auto* y = P<float>(0x6000000);
    auto* acc = P<int32_t>(0x7000000);
    auto* ws = P<void>(0x8000000);
    auto* f = P<float>(0x9000000);
    auto* f2 = P<float>(0xA000000);
    auto* h = P<uint16_t>(0xB000000);
    auto* b8 = P<uint8_t>(0xC000000);
    auto* mis = P<uint16_t>(0xD000002);

    // Size helpers at the edges.
    EXPECT(bl_packed_bytes(BIG, BIG), 0);
    EXPECT(bl_packed_bytes(NEG, 64), 0);
    EXPECT(bl_packed_bytes(1, 64), 16);
    EXPECT(bl_quantize_weights_workspace_bytes(BIG, 64), 0);
    EXPECT(bl_packed_bytes_binary(BIG, BIG), 0);
    EXPECT(bl_packed_bytes_base3(BIG, 64), 0);
    EXPECT(bl_ste_t_bytes(BIG, BIG), 0);
    EXPECT(bl_ste_dw_workspace_bytes(BIG, 64, 64), 0);
    EXPECT(bl_ste_dw_workspace_bytes(1, BIG, 64), 0);
    EXPECT(bl_ffn_relu2_workspace_bytes(BIG, 2560, 6912), 0);
    EXPECT(bl_ffn_relu2_workspace_bytes(1, BIG, 6912), 0);
    EXPECT(bl_calib_mfma_i8_ops(BIG), 0);
    EXPECT(bl_calib_mfma_i8_ops(NEG), 0);

    // Weight quantisation.
    const size_t wsb = bl_quantize_weights_workspace_bytes(16, 64);
    EXPECT(bl_quantize_weights(f, 16, 64, W, g, ws, wsb, nullptr), D);
    EXPECT(bl_quantize_weights(nullptr, 16, 64, W, g, ws, wsb, nullptr), E);
    EXPECT(bl_quantize_weights(f, BIG, BIG, W, g, ws, wsb, nullptr), E);
    EXPECT(bl_quantize_weights(f, 16, 48, W, g, ws, wsb, nullptr), E);
    EXPECT(bl_quantize_weights(f, 16, 64, W, g, ws, wsb - 1, nullptr), E);
    EXPECT(bl_quantize_weights_binary(f, 16, 64, W, g, ws, wsb, nullptr), D);
    EXPECT(bl_quantize_weights_binary(f, NEG, 64, W, g, ws, wsb, nullptr), E);

    // Activation quantisation.
    EXPECT(bl_quantize_acts(x, 4, 2560, nullptr, 0.0f, xq, xs, nullptr), D);
    EXPECT(bl_quantize_acts(x, 4, 2560, h, 1e-5f, xq, xs, nullptr), D);
    EXPECT(bl_quantize_acts(x, BIG, 2560, nullptr, 0.0f, xq, xs, nullptr), E);
    EXPECT(bl_quantize_acts(x, 4, BIG, nullptr, 0.0f, xq, xs, nullptr), E);
    EXPECT(bl_quantize_acts(x, 4, 2560, h, -1.0f, xq, xs, nullptr), E);
    EXPECT(bl_quantize_acts(mis, 4, 2560, nullptr, 0.0f, xq, xs, nullptr), E);

    // Products, every path.
    for (int path = 0; path <= 4; ++path)
        EXPECT(bl_bitlinear_path(xq, xs, 1, 2560, W, g, 6912, y, acc, path, nullptr), D);
    EXPECT(bl_bitlinear_path(xq, xs, 1, 2560, W, g, 6912, y, acc, 5, nullptr), E);
    EXPECT(bl_bitlinear_path(xq, xs, 2, 2560, W, g, 6912, y, acc, 4, nullptr), E);
    EXPECT(bl_bitlinear_path(xq, xs, 17, 2560, W, g, 6912, y, acc, 1, nullptr), E);
    // The kernel choice and the act quant + product in one call.
    EXPECT(bl_bitlinear_choice(1, 8640, 3200, 0), 1);
    EXPECT(bl_bitlinear_choice(1, 8192, 28672, 0), 4);
    EXPECT(bl_bitlinear_choice(BIG, 2560, 6912, 0), -1);
    EXPECT(bl_bitlinear_choice(1, BIG, 6912, 0), -1);
    EXPECT(bl_bitlinear_choice(1, 2560, NEG, 0), -1);
    EXPECT(bl_quant_bitlinear(x, 1, 2560, nullptr, 0.0f, W, g, 6912, y, xq, xs, nullptr), D);
    EXPECT(bl_quant_bitlinear(x, 3, 8192, h, 1e-5f, W, g, 6912, y, xq, xs, nullptr), D);
    EXPECT(bl_quant_bitlinear(x, BIG, 2560, nullptr, 0.0f, W, g, 6912, y, xq, xs, nullptr), E);
    EXPECT(bl_quant_bitlinear(x, 1, 2560, nullptr, 0.0f, W, g, BIG, y, xq, xs, nullptr), E);
    EXPECT(bl_quant_bitlinear(x, 1, 2560, h, 0.0f, W, g, 6912, y, xq, xs, nullptr), E);
    EXPECT(bl_quant_bitlinear(x, 1, 2560, nullptr, 0.0f, W, g, 6912, y, xq, P<float>(0x6000100),
                              nullptr), E);
    EXPECT(bl_bitlinear(xq, xs, BIG, 64, W, g, 16, y, nullptr, nullptr), E);
    EXPECT(bl_bitlinear(xq, xs, 1 << 20, 1 << 12, W, g, 1 << 20, y, nullptr, nullptr), E);
    EXPECT(bl_bitlinear(xq, xs, 1, 64, W, g, BIG, y, nullptr, nullptr), E);
    EXPECT(bl_bitlinear(xq, xs, 1, 64, W, g, 16, P<float>(0x2000000), nullptr, nullptr), E);
    EXPECT(bl_bitlinear_pair(xq, xs, 1, 2560, W, g, 6912, y, W, g, 6912, f, nullptr), D);
    EXPECT(bl_bitlinear_pair(xq, xs, 1, 2560, W, g, BIG, y, W, g, 6912, f, nullptr), E);
    EXPECT(bl_bitlinear_binary(xq, xs, 1, 2560, W, g, 6912, y, acc, nullptr), D);
    EXPECT(bl_bitlinear_base3(xq, xs, 1, 2560, b8, g, 6912, y, acc, nullptr), D);
    EXPECT(bl_bitlinear_base3(xq, xs, 64, 2560, b8, g, 6912, y, acc, nullptr), E);
    EXPECT(bl_pack_base3(W, 6912, 2560, b8, nullptr), D);
    EXPECT(bl_pack_base3(W, BIG, 2560, b8, nullptr), E);

    // Gating and the FFN step.
    EXPECT(bl_relu2_glu(f, f2, 4096, h, nullptr), D);
    EXPECT(bl_relu2_glu(f, f2, NEG, h, nullptr), E);
    EXPECT(bl_glu(f, f2, 4096, BL_GLU_SWIGLU, h, nullptr), D);
    EXPECT(bl_glu(f, f2, 4096, 7, h, nullptr), E);
    EXPECT(bl_glu_quant(f, f2, 4, 6912, BL_GLU_RELU2, nullptr, 0.0f, xq, xs, nullptr), D);
    EXPECT(bl_glu_quant(f, f2, 4, 6912, BL_GLU_RELU2, h, 0.0f, xq, xs, nullptr), E);
    EXPECT(bl_relu2_glu_quant(f, f2, 4, 6912, xq, xs, nullptr), D);
    EXPECT(bl_relu2_glu_subln_quant(f, f2, 4, 6912, h, 1e-5f, xq, xs, nullptr), D);
    EXPECT(bl_relu2_glu_subln_quant(f, f2, 4, 6912, nullptr, 1e-5f, xq, xs, nullptr), E);
    const size_t fws = bl_ffn_relu2_workspace_bytes(4, 2560, 6912);
    EXPECT(bl_ffn_relu2(x, 4, 2560, W, g, W, g, 6912, W, g, y, ws, fws, nullptr), D);
    EXPECT(bl_ffn_relu2(x, 4, 2560, W, g, W, g, 6912, W, g, y, ws, fws - 1, nullptr), E);
    EXPECT(bl_ffn_relu2(x, BIG, 2560, W, g, W, g, 6912, W, g, y, ws, fws, nullptr), E);
    EXPECT(bl_ffn_relu2_subln(x, 4, 2560, W, g, W, g, 6912, W, g, h, 1e-5f, y, ws, fws, nullptr),
           D);
    EXPECT(bl_ffn_step(x, 4, 2560, W, g, W, g, 6912, W, g, BL_GLU_SWIGLU, nullptr, 0.0f, y, ws,
                       fws, nullptr), D);
    EXPECT(bl_ffn_step(x, 4, 2560, W, g, W, g, 6912, W, g, 9, nullptr, 0.0f, y, ws, fws, nullptr),
           E);
    EXPECT(bl_ffn_step_noalloc(x, 25, 8192, W, g, W, g, 28672, W, g, BL_GLU_RELU2, nullptr, 0.0f,
                               y, nullptr), D);
    EXPECT(bl_ffn_step_noalloc(x, 26, 8192, W, g, W, g, 28672, W, g, BL_GLU_RELU2, nullptr, 0.0f,
                               y, nullptr), E);
    EXPECT(bl_ffn_step_noalloc(x, BIG, BIG, W, g, W, g, BIG, W, g, BL_GLU_RELU2, nullptr, 0.0f, y,
                               nullptr), E);

    // Straight-through backward.
    EXPECT(bl_pack_ste_t(W, 6912, 2560, b8, nullptr), D);
    EXPECT(bl_pack_ste_t(W, BIG, 2560, b8, nullptr), E);
    EXPECT(bl_ste_backward_dx(x, 4096, 6912, b8, g, 2560, f, nullptr), D);
    EXPECT(bl_ste_backward_dx(x, 4096, 6913, b8, g, 2560, f, nullptr), E);
    EXPECT(bl_ste_backward_dx(x, BIG, 6912, b8, g, 2560, f, nullptr), E);
    const size_t dws = bl_ste_dw_workspace_bytes(100, 64, 128);
    EXPECT(bl_ste_backward_dw(x, 100, 64, xq, xs, 128, f, ws, dws, nullptr), D);
    EXPECT(bl_ste_backward_dw(x, 100, 64, xq, xs, 128, f, ws, dws - 1, nullptr), E);
    EXPECT(bl_ste_backward_dw(x, BIG, 64, xq, xs, 128, f, ws, dws, nullptr), E);
    EXPECT(bl_ste_backward_dw(x, 100, 64, xq, xs, 128, f, P<void>(0x8000010), dws, nullptr), E);

    // Calibration.
    EXPECT(bl_calib_read(W, 1 << 20, P<uint32_t>(0xE000000), nullptr), D);
    EXPECT(bl_calib_read(W, 15, P<uint32_t>(0xE000000), nullptr), E);
    EXPECT(bl_calib_copy(f, W, 1 << 20, nullptr), D);
    EXPECT(bl_calib_copy(f, f, 1 << 20, nullptr), E);
    EXPECT(bl_calib_mfma_i8(10, acc, nullptr), D);
    EXPECT(bl_calib_mfma_i8(0, acc, nullptr), E);

    // Status strings.
    for (int s = -1; s <= 5; ++s)
        if (bl_status_string(s) == nullptr) ++g_failures;
    if (g_failures) {
        std::fprintf(stderr, "%d check(s) failed\n", g_failures);
        return 1;
    }
    std::puts("abi host checks: ok");
    return 0;
}
