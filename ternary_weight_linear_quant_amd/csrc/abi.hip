// C ABI of the BitLinear library: host-side validation and kernel dispatch.
// The entry points and their contracts are declared in include/bitlinear.h.
#include <atomic>
#include <cstdint>

#include "../../include/bitlinear.h"
#include "launch.hpp"

namespace {

thread_local int g_last_hip_error = 0;
std::atomic<int> g_device_count{-1};

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool shape_ok(int64_t rows, int64_t K) {
    if (rows < 1 || K < 64 || (K % 64) != 0) return false;
    if (rows > (int64_t{1} << 31) / K) return false;  // rows*K < 2^31
    return true;
}

int device_status() {
    int n = g_device_count.load(std::memory_order_relaxed);
    if (n < 0) {
        if (hipGetDeviceCount(&n) != hipSuccess) n = 0;
        (void)hipGetLastError();
        g_device_count.store(n, std::memory_order_relaxed);
    }
    return n > 0 ? BL_OK : BL_ERR_NO_DEVICE;
}

int hip_status(hipError_t e) {
    if (e == hipSuccess) return BL_OK;
    g_last_hip_error = (int)e;
    return BL_ERR_HIP;
}

hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

}  // namespace

extern "C" {

const char* bl_status_string(int status) {
    switch (status) {
        case BL_OK: return "BL_OK";
        case BL_ERR_INVALID_ARG: return "BL_ERR_INVALID_ARG";
        case BL_ERR_HIP: return "BL_ERR_HIP";
        case BL_ERR_NO_DEVICE: return "BL_ERR_NO_DEVICE";
        default: return "BL_ERR_UNKNOWN";
    }
}

int bl_last_hip_error(void) { return g_last_hip_error; }

const char* bl_version(void) { return "bitlinear-gfx950 0.1.0"; }

size_t bl_packed_bytes(int64_t N, int64_t K) {
    if (!shape_ok(N, K)) return 0;
    return (size_t)(N * (K / 4));
}

size_t bl_quantize_weights_workspace_bytes(int64_t N, int64_t K) {
    if (!shape_ok(N, K)) return 0;
    return (size_t)N * sizeof(double);
}

int bl_quantize_weights(const float* W, int64_t N, int64_t K, uint32_t* W_packed, float* gamma,
                        void* workspace, size_t workspace_bytes, void* stream) {
    if (!W || !W_packed || !gamma || !workspace) return BL_ERR_INVALID_ARG;
    if (!shape_ok(N, K)) return BL_ERR_INVALID_ARG;
    if (!aligned16(W) || !aligned16(W_packed)) return BL_ERR_INVALID_ARG;
    if ((reinterpret_cast<uintptr_t>(workspace) & 7u) != 0) return BL_ERR_INVALID_ARG;
    if (workspace_bytes < bl_quantize_weights_workspace_bytes(N, K)) return BL_ERR_INVALID_ARG;
    if (int s = device_status()) return s;
    return hip_status(bl::launch_quantize_weights(W, N, K, W_packed, gamma,
                                                  static_cast<double*>(workspace),
                                                  as_stream(stream)));
}

int bl_quantize_acts(const uint16_t* x, int64_t M, int64_t K, const uint16_t* rms_gain,
                     float rms_eps, int8_t* x_q, float* x_scale, void* stream) {
    if (!x || !x_q || !x_scale) return BL_ERR_INVALID_ARG;
    if (!shape_ok(M, K)) return BL_ERR_INVALID_ARG;
    if (!aligned16(x) || !aligned16(x_q)) return BL_ERR_INVALID_ARG;
    if (rms_gain && (!aligned16(rms_gain) || !(rms_eps > 0.0f))) return BL_ERR_INVALID_ARG;
    if (int s = device_status()) return s;
    return hip_status(bl::launch_quantize_acts(x, M, K, rms_gain, rms_eps, x_q, x_scale,
                                               as_stream(stream)));
}

int bl_bitlinear_path(const int8_t* x_q, const float* x_scale, int64_t M, int64_t K,
                      const uint32_t* W_packed, const float* gamma, int64_t N, float* y,
                      int32_t* acc, int path, void* stream) {
    if (!x_q || !x_scale || !W_packed || !gamma || !y) return BL_ERR_INVALID_ARG;
    if (!shape_ok(M, K) || !shape_ok(N, K)) return BL_ERR_INVALID_ARG;
    if (M > (int64_t{1} << 31) / N) return BL_ERR_INVALID_ARG;  // M*N < 2^31
    if (!aligned16(x_q) || !aligned16(W_packed)) return BL_ERR_INVALID_ARG;
    if (path < 0 || path > 2) return BL_ERR_INVALID_ARG;
    const bool gemv_ok = bl::gemv_supported(M, K);
    if (path == 1 && !gemv_ok) return BL_ERR_INVALID_ARG;
    if (int s = device_status()) return s;
    const bool use_gemv = path == 1 || (path == 0 && gemv_ok);
    hipStream_t st = as_stream(stream);
    if (use_gemv)
        return hip_status(bl::launch_gemv(x_q, x_scale, (int)M, (int)K, W_packed, gamma, (int)N,
                                          y, acc, st));
    return hip_status(bl::launch_gemm(x_q, x_scale, (int)M, (int)K, W_packed, gamma, (int)N, y,
                                      acc, st));
}

int bl_bitlinear(const int8_t* x_q, const float* x_scale, int64_t M, int64_t K,
                 const uint32_t* W_packed, const float* gamma, int64_t N, float* y, int32_t* acc,
                 void* stream) {
    return bl_bitlinear_path(x_q, x_scale, M, K, W_packed, gamma, N, y, acc, 0, stream);
}

int bl_bitlinear_pair(const int8_t* x_q, const float* x_scale, int64_t M, int64_t K,
                      const uint32_t* W1, const float* gamma1, int64_t N1, float* y1,
                      const uint32_t* W2, const float* gamma2, int64_t N2, float* y2,
                      void* stream) {
    if (!x_q || !x_scale || !W1 || !gamma1 || !y1 || !W2 || !gamma2 || !y2)
        return BL_ERR_INVALID_ARG;
    if (!shape_ok(M, K) || !shape_ok(N1, K) || !shape_ok(N2, K)) return BL_ERR_INVALID_ARG;
    if (M > (int64_t{1} << 31) / N1 || M > (int64_t{1} << 31) / N2) return BL_ERR_INVALID_ARG;
    if (!aligned16(x_q) || !aligned16(W1) || !aligned16(W2)) return BL_ERR_INVALID_ARG;
    if (int s = device_status()) return s;
    hipStream_t st = as_stream(stream);
    if (bl::gemv_supported(M, K))
        return hip_status(bl::launch_gemv_pair(x_q, x_scale, (int)M, (int)K, W1, gamma1, (int)N1,
                                               y1, W2, gamma2, (int)N2, y2, st));
    int e = hip_status(bl::launch_gemm(x_q, x_scale, (int)M, (int)K, W1, gamma1, (int)N1, y1,
                                       nullptr, st));
    if (e) return e;
    return hip_status(bl::launch_gemm(x_q, x_scale, (int)M, (int)K, W2, gamma2, (int)N2, y2,
                                      nullptr, st));
}

int bl_relu2_glu_quant(const float* gate, const float* up, int64_t M, int64_t K, int8_t* h_q,
                       float* h_scale, void* stream) {
    if (!gate || !up || !h_q || !h_scale) return BL_ERR_INVALID_ARG;
    if (!shape_ok(M, K)) return BL_ERR_INVALID_ARG;
    if (!aligned16(gate) || !aligned16(up) || !aligned16(h_q)) return BL_ERR_INVALID_ARG;
    if (int s = device_status()) return s;
    return hip_status(bl::launch_relu2_glu_quant(gate, up, M, K, h_q, h_scale, as_stream(stream)));
}

int bl_relu2_glu(const float* gate, const float* up, int64_t count, uint16_t* h, void* stream) {
    if (!gate || !up || !h || count < 1) return BL_ERR_INVALID_ARG;
    if (count > (int64_t{1} << 40)) return BL_ERR_INVALID_ARG;
    if (!aligned16(gate) || !aligned16(up) || !aligned16(h)) return BL_ERR_INVALID_ARG;
    if (int s = device_status()) return s;
    return hip_status(bl::launch_relu2_glu(gate, up, count, h, as_stream(stream)));
}

}  // extern "C"
