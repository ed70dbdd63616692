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

// Every entry point calls this after validating its arguments and before
// enqueuing anything. It also clears the thread's pending HIP error, so that
// the hipGetLastError() after each launch reports that launch, not an error
// left by an earlier, unrelated call.
int device_status() {
    int n = g_device_count.load(std::memory_order_relaxed);
    if (n < 0) {
        if (hipGetDeviceCount(&n) != hipSuccess) n = 0;
        g_device_count.store(n, std::memory_order_relaxed);
    }
    (void)hipGetLastError();
    return n > 0 ? BL_OK : BL_ERR_NO_DEVICE;
}

// A failure is recorded for bl_last_hip_error() and taken off HIP's pending
// error, so it does not resurface in the caller's next, unrelated check.
int hip_status(hipError_t e) {
    if (e == hipSuccess) return BL_OK;
    g_last_hip_error = (int)e;
    (void)hipGetLastError();
    return BL_ERR_HIP;
}

hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

// Workspace of bl_ffn_relu2: 256-byte aligned segments.
struct FfnWorkspace {
    size_t h, xq, xs, yg, yu, hq, hs, total;
};
size_t align256(size_t v) { return (v + 255) & ~size_t(255); }
FfnWorkspace ffn_layout(int64_t M, int64_t K, int64_t N) {
    FfnWorkspace w;
    size_t o = 0;
    w.h = o;  o += align256((size_t)(2 * M * N));
    w.xq = o; o += align256((size_t)(M * K));
    w.xs = o; o += align256((size_t)(4 * M));
    w.yg = o; o += align256((size_t)(4 * M * N));
    w.yu = o; o += align256((size_t)(4 * M * N));
    w.hq = o; o += align256((size_t)(M * N));
    w.hs = o; o += align256((size_t)(4 * M));
    w.total = o;
    return w;
}

// True when the byte ranges [a, a+na) and [b, b+nb) intersect.
bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
    const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
    return x < y + nb && y < x + na;
}

bool ffn_shapes_ok(int64_t M, int64_t K, int64_t N) {
    return shape_ok(M, K) && shape_ok(M, N) && shape_ok(N, K) && shape_ok(K, N) &&
           M <= (int64_t{1} << 31) / N;
}

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

#ifndef BL_SOURCE_SHA256
#define BL_SOURCE_SHA256 "unknown"
#endif
const char* bl_source_sha256(void) { return BL_SOURCE_SHA256; }

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

int bl_bitlinear_choice(int64_t M, int64_t K, int64_t N, int path) {
    if (!shape_ok(M, K) || !shape_ok(N, K)) return -1;
    const bool one_ok = bl::gemv1_supported(M, K);
    const bool gemv_ok = bl::gemv_supported(M, K);
    const bool wide_ok = bl::gemv_wide_supported(M, K);
    switch (path) {
        case 1: return gemv_ok ? 1 : -1;
        case 2: return 2;
        case 3: return wide_ok ? 3 : -1;
        case 4: return one_ok ? 4 : -1;
        case 0: break;
        default: return -1;
    }
    if (bl::gemv1_preferred(M, K)) return 4;
    if (gemv_ok) return 1;
    if (bl::gemv_wide_preferred(M, N, K)) return 3;
    return 2;
}

int bl_bitlinear_path(const int8_t* x_q, const float* x_scale, int64_t M, int64_t K,
                      const uint32_t* W_packed, const float* gamma, int64_t N, float* y,
                      int32_t* acc, int path, void* stream) {
    if (!x_q || !x_scale || !W_packed || !gamma || !y) return BL_ERR_INVALID_ARG;
    if (!shape_ok(M, K) || !shape_ok(N, K)) return BL_ERR_INVALID_ARG;
    if (M > (int64_t{1} << 31) / N) return BL_ERR_INVALID_ARG;  // M*N < 2^31
    if (!aligned16(x_q) || !aligned16(W_packed)) return BL_ERR_INVALID_ARG;
    if (path < 0 || path > 4) return BL_ERR_INVALID_ARG;
    // The outputs may not alias an input (y holds partial sums mid-call).
    const size_t ny = (size_t)(M * N) * 4;
    if (overlaps(y, ny, x_q, (size_t)(M * K)) || overlaps(y, ny, x_scale, (size_t)M * 4) ||
        overlaps(y, ny, W_packed, (size_t)(N * K) / 4) || overlaps(y, ny, gamma, 4))
        return BL_ERR_INVALID_ARG;
    if (acc && (overlaps(acc, ny, y, ny) || overlaps(acc, ny, x_q, (size_t)(M * K)) ||
                overlaps(acc, ny, x_scale, (size_t)M * 4) ||
                overlaps(acc, ny, W_packed, (size_t)(N * K) / 4) || overlaps(acc, ny, gamma, 4)))
        return BL_ERR_INVALID_ARG;
    const int chosen = bl_bitlinear_choice(M, K, N, path);
    if (chosen < 0) return BL_ERR_INVALID_ARG;
    if (int s = device_status()) return s;
    const bool use_one = chosen == 4, use_gemv = chosen == 1, use_wide = chosen == 3;
    hipStream_t st = as_stream(stream);
    if (use_one)
        return hip_status(bl::launch_gemv1(x_q, x_scale, (int)K, W_packed, gamma, (int)N, y, acc,
                                           st));
    if (use_gemv)
        return hip_status(bl::launch_gemv(x_q, x_scale, (int)M, (int)K, W_packed, gamma, (int)N,
                                          y, acc, st));
    if (use_wide)
        return hip_status(bl::launch_gemv_wide(x_q, x_scale, (int)M, (int)K, W_packed, gamma,
                                               (int)N, y, acc, st));
    return hip_status(bl::launch_gemm(x_q, x_scale, (int)M, (int)K, W_packed, gamma, (int)N, y,
                                      acc, st));
}

int bl_bitlinear(const int8_t* x_q, const float* x_scale, int64_t M, int64_t K,
                 const uint32_t* W_packed, const float* gamma, int64_t N, float* y, int32_t* acc,
                 void* stream) {
    return bl_bitlinear_path(x_q, x_scale, M, K, W_packed, gamma, N, y, acc, 0, stream);
}

int bl_quant_bitlinear(const uint16_t* x, int64_t M, int64_t K, const uint16_t* rms_gain,
                       float rms_eps, const uint32_t* W_packed, const float* gamma, int64_t N,
                       float* y, int8_t* x_q, float* x_scale, void* stream) {
    if (!x || !W_packed || !gamma || !y || !x_q || !x_scale) return BL_ERR_INVALID_ARG;
    if (!shape_ok(M, K) || !shape_ok(N, K)) return BL_ERR_INVALID_ARG;
    if (M > (int64_t{1} << 31) / N) return BL_ERR_INVALID_ARG;  // M*N < 2^31
    if (!aligned16(x) || !aligned16(x_q) || !aligned16(x_scale) || !aligned16(W_packed) ||
        !aligned16(y))
        return BL_ERR_INVALID_ARG;
    if (rms_gain && (!aligned16(rms_gain) || !(rms_eps > 0.0f))) return BL_ERR_INVALID_ARG;
    // No output may overlap another output or an input.
    const size_t ny = (size_t)(M * N) * 4, nq = (size_t)(M * K), ns = (size_t)M * 4;
    const void* outs[3] = {y, x_q, x_scale};
    const size_t out_n[3] = {ny, nq, ns};
    const void* ins[4] = {x, rms_gain, W_packed, gamma};
    const size_t in_n[4] = {(size_t)(M * K) * 2, rms_gain ? (size_t)K * 2 : 0,
                            (size_t)(N * K) / 4, 4};
    for (int i = 0; i < 3; ++i) {
        for (int j = i + 1; j < 3; ++j)
            if (overlaps(outs[i], out_n[i], outs[j], out_n[j])) return BL_ERR_INVALID_ARG;
        for (int j = 0; j < 4; ++j)
            if (ins[j] && overlaps(outs[i], out_n[i], ins[j], in_n[j])) return BL_ERR_INVALID_ARG;
    }
    if (int s = device_status()) return s;
    hipStream_t st = as_stream(stream);
    if (bl::gemv1_quant_supported(M, K, rms_gain != nullptr))
        return hip_status(bl::launch_gemv1_quant(x, rms_gain, rms_eps, (int)K, W_packed, gamma,
                                                 (int)N, y, x_q, x_scale, st));
    if (int s = bl_quantize_acts(x, M, K, rms_gain, rms_eps, x_q, x_scale, stream)) return s;
    return bl_bitlinear_path(x_q, x_scale, M, K, W_packed, gamma, N, y, nullptr, 0, stream);
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

size_t bl_ffn_relu2_workspace_bytes(int64_t M, int64_t K, int64_t N_ff) {
    if (!ffn_shapes_ok(M, K, N_ff)) return 0;
    return ffn_layout(M, K, N_ff).total;
}

}  // extern "C"

namespace {

bool glu_kind_ok(int kind) { return kind == BL_GLU_RELU2 || kind == BL_GLU_SWIGLU; }

constexpr int64_t kFfnSplitDownM = 16;

// One FFN step; subln_gain (bf16 [N_ff]) null for none.
int ffn_step(const uint16_t* x, int64_t M, int64_t K, const uint32_t* W_gate,
             const float* gamma_gate, const uint32_t* W_up, const float* gamma_up, int64_t N_ff,
             const uint32_t* W_down, const float* gamma_down, int kind,
             const uint16_t* subln_gain, float subln_eps, float* y, void* workspace,
             size_t workspace_bytes, void* stream) {
    if (!glu_kind_ok(kind)) return BL_ERR_INVALID_ARG;
    if (!x || !W_gate || !gamma_gate || !W_up || !gamma_up || !W_down || !gamma_down || !y ||
        !workspace)
        return BL_ERR_INVALID_ARG;
    if (!ffn_shapes_ok(M, K, N_ff)) return BL_ERR_INVALID_ARG;
    if (!aligned16(x) || !aligned16(W_gate) || !aligned16(W_up) || !aligned16(W_down) ||
        !aligned16(y) || (reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
        return BL_ERR_INVALID_ARG;
    if (subln_gain && (!aligned16(subln_gain) || !(subln_eps > 0.0f))) return BL_ERR_INVALID_ARG;
    const FfnWorkspace L = ffn_layout(M, K, N_ff);
    if (workspace_bytes < L.total) return BL_ERR_INVALID_ARG;
    if (int s = device_status()) return s;
    hipStream_t st = as_stream(stream);
    uint8_t* ws = static_cast<uint8_t*>(workspace);
    auto* h = reinterpret_cast<uint16_t*>(ws + L.h);
    auto* hq = reinterpret_cast<int8_t*>(ws + L.hq);
    auto* hs = reinterpret_cast<float*>(ws + L.hs);
    // From kFfnSplitDownM tokens the down projection's fused launch, whose
    // every workgroup reads and quantises all of h, costs more than one act
    // quant launch followed by the plain GEMV on the int8 codes.
    if (M >= kFfnSplitDownM && bl::ffn_gate_up_supported(M, K, N_ff) &&
        bl::gemv_supported(M, N_ff)) {
        hipError_t e = bl::launch_ffn_gate_up(x, (int)M, (int)K, W_gate, gamma_gate, W_up,
                                              gamma_up, (int)N_ff, h, kind, st);
        if (e == hipSuccess)
            e = bl::launch_quantize_acts(h, M, N_ff, subln_gain, subln_eps, hq, hs, st);
        if (e == hipSuccess)
            e = bl::launch_gemv(hq, hs, (int)M, (int)N_ff, W_down, gamma_down, (int)K, y,
                                nullptr, st);
        return hip_status(e);
    }
    if (bl::ffn_fused_supported(M, K, N_ff, subln_gain != nullptr))
        return hip_status(bl::launch_ffn_fused(x, (int)M, (int)K, W_gate, gamma_gate, W_up,
                                               gamma_up, (int)N_ff, W_down, gamma_down, h, y,
                                               kind, subln_gain, subln_eps, st));
    // Unfused sequence: act quant -> gate/up -> gating (+ norm) + act quant -> down.
    auto* xq = reinterpret_cast<int8_t*>(ws + L.xq);
    auto* xs = reinterpret_cast<float*>(ws + L.xs);
    auto* yg = reinterpret_cast<float*>(ws + L.yg);
    auto* yu = reinterpret_cast<float*>(ws + L.yu);
    const int m = (int)M, k = (int)K, n = (int)N_ff;
    hipError_t e = bl::launch_quantize_acts(x, M, K, nullptr, 0.0f, xq, xs, st);
    if (e == hipSuccess) {
        if (bl::gemv_supported(M, K)) {
            e = bl::launch_gemv_pair(xq, xs, m, k, W_gate, gamma_gate, n, yg, W_up, gamma_up, n,
                                     yu, st);
        } else {
            e = bl::launch_gemm(xq, xs, m, k, W_gate, gamma_gate, n, yg, nullptr, st);
            if (e == hipSuccess)
                e = bl::launch_gemm(xq, xs, m, k, W_up, gamma_up, n, yu, nullptr, st);
        }
    }
    if (e == hipSuccess)
        e = bl::launch_glu_quant(yg, yu, M, N_ff, kind, subln_gain, subln_eps, hq, hs, st);
    if (e == hipSuccess) {
        if (bl::gemv_supported(M, N_ff))
            e = bl::launch_gemv(hq, hs, m, n, W_down, gamma_down, k, y, nullptr, st);
        else
            e = bl::launch_gemm(hq, hs, m, n, W_down, gamma_down, k, y, nullptr, st);
    }
    return hip_status(e);
}

int glu_quant(const float* gate, const float* up, int64_t M, int64_t K, int kind,
              const uint16_t* gain, float rms_eps, int8_t* h_q, float* h_scale, void* stream) {
    if (!gate || !up || !h_q || !h_scale || !glu_kind_ok(kind)) return BL_ERR_INVALID_ARG;
    if (!shape_ok(M, K)) return BL_ERR_INVALID_ARG;
    if (!aligned16(gate) || !aligned16(up) || !aligned16(h_q)) return BL_ERR_INVALID_ARG;
    if (gain && (!aligned16(gain) || !(rms_eps > 0.0f))) return BL_ERR_INVALID_ARG;
    if (int s = device_status()) return s;
    return hip_status(
        bl::launch_glu_quant(gate, up, M, K, kind, gain, rms_eps, h_q, h_scale, as_stream(stream)));
}

}  // namespace

extern "C" {

int bl_ffn_relu2(const uint16_t* x, int64_t M, int64_t K, const uint32_t* W_gate,
                 const float* gamma_gate, const uint32_t* W_up, const float* gamma_up,
                 int64_t N_ff, const uint32_t* W_down, const float* gamma_down, float* y,
                 void* workspace, size_t workspace_bytes, void* stream) {
    return ffn_step(x, M, K, W_gate, gamma_gate, W_up, gamma_up, N_ff, W_down, gamma_down,
                    BL_GLU_RELU2, nullptr, 0.0f, y, workspace, workspace_bytes, stream);
}

int bl_ffn_relu2_subln(const uint16_t* x, int64_t M, int64_t K, const uint32_t* W_gate,
                       const float* gamma_gate, const uint32_t* W_up, const float* gamma_up,
                       int64_t N_ff, const uint32_t* W_down, const float* gamma_down,
                       const uint16_t* subln_gain, float subln_eps, float* y, void* workspace,
                       size_t workspace_bytes, void* stream) {
    if (!subln_gain) return BL_ERR_INVALID_ARG;
    return ffn_step(x, M, K, W_gate, gamma_gate, W_up, gamma_up, N_ff, W_down, gamma_down,
                    BL_GLU_RELU2, subln_gain, subln_eps, y, workspace, workspace_bytes, stream);
}

int bl_ffn_step(const uint16_t* x, int64_t M, int64_t K, const uint32_t* W_gate,
                const float* gamma_gate, const uint32_t* W_up, const float* gamma_up,
                int64_t N_ff, const uint32_t* W_down, const float* gamma_down, int glu_kind,
                const uint16_t* subln_gain, float subln_eps, float* y, void* workspace,
                size_t workspace_bytes, void* stream) {
    return ffn_step(x, M, K, W_gate, gamma_gate, W_up, gamma_up, N_ff, W_down, gamma_down,
                    glu_kind, subln_gain, subln_eps, y, workspace, workspace_bytes, stream);
}

}  // extern "C"

namespace {

// Fixed scratch of bl_ffn_step_noalloc. Every device that runs the library
// holds its own copy of this array until the process ends. Host code never
// passes the array's name to a kernel (on the host it is only a stand-in):
// it uses the device address that hipGetSymbolAddress returns on each device.
constexpr size_t kNoAllocScratchBytes = size_t{8} << 20;
__device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];

constexpr int kMaxCachedDevices = 64;
std::atomic<uintptr_t> g_scratch_addr[kMaxCachedDevices];  // 0 until resolved

// The current device's copy of `scratch`, resolved on the first call on that
// device (with the device current) and kept; devices past the cache are
// resolved on every call. Two threads racing on a first call store the same
// address.
int current_scratch(uint8_t** out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_status(e);
    const bool cached = dev >= 0 && dev < kMaxCachedDevices;
    uintptr_t addr = cached ? g_scratch_addr[dev].load(std::memory_order_acquire) : 0;
    if (addr == 0) {
        void* ptr = nullptr;
        e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return hip_status(e);
        if (ptr == nullptr) return hip_status(hipErrorInvalidSymbol);
        addr = reinterpret_cast<uintptr_t>(ptr);
        if (cached) g_scratch_addr[dev].store(addr, std::memory_order_release);
    }
    *out = reinterpret_cast<uint8_t*>(addr);
    return BL_OK;
}

}  // namespace

extern "C" {

int bl_ffn_step_noalloc(const uint16_t* x, int64_t M, int64_t K, const uint32_t* W_gate,
                        const float* gamma_gate, const uint32_t* W_up, const float* gamma_up,
                        int64_t N_ff, const uint32_t* W_down, const float* gamma_down,
                        int glu_kind, const uint16_t* subln_gain, float subln_eps, float* y,
                        void* stream) {
    // Every argument check of ffn_step, before the device is touched.
    if (!glu_kind_ok(glu_kind)) return BL_ERR_INVALID_ARG;
    if (!ffn_shapes_ok(M, K, N_ff)) return BL_ERR_INVALID_ARG;
    if (ffn_layout(M, K, N_ff).total > kNoAllocScratchBytes) return BL_ERR_INVALID_ARG;
    if (!x || !W_gate || !gamma_gate || !W_up || !gamma_up || !W_down || !gamma_down || !y)
        return BL_ERR_INVALID_ARG;
    if (!aligned16(x) || !aligned16(W_gate) || !aligned16(W_up) || !aligned16(W_down) ||
        !aligned16(y))
        return BL_ERR_INVALID_ARG;
    if (subln_gain && (!aligned16(subln_gain) || !(subln_eps > 0.0f))) return BL_ERR_INVALID_ARG;
    if (int s = device_status()) return s;
    uint8_t* ws = nullptr;
    if (int s = current_scratch(&ws)) return s;
    return ffn_step(x, M, K, W_gate, gamma_gate, W_up, gamma_up, N_ff, W_down, gamma_down,
                    glu_kind, subln_gain, subln_eps, y, ws, kNoAllocScratchBytes, stream);
}

int bl_relu2_glu_quant(const float* gate, const float* up, int64_t M, int64_t K, int8_t* h_q,
                       float* h_scale, void* stream) {
    return glu_quant(gate, up, M, K, BL_GLU_RELU2, nullptr, 0.0f, h_q, h_scale, stream);
}

int bl_relu2_glu_subln_quant(const float* gate, const float* up, int64_t M, int64_t K,
                             const uint16_t* gain, float rms_eps, int8_t* h_q, float* h_scale,
                             void* stream) {
    if (!gain) return BL_ERR_INVALID_ARG;
    return glu_quant(gate, up, M, K, BL_GLU_RELU2, gain, rms_eps, h_q, h_scale, stream);
}

int bl_glu_quant(const float* gate, const float* up, int64_t M, int64_t K, int glu_kind,
                 const uint16_t* gain, float rms_eps, int8_t* h_q, float* h_scale, void* stream) {
    return glu_quant(gate, up, M, K, glu_kind, gain, rms_eps, h_q, h_scale, stream);
}

int bl_glu(const float* gate, const float* up, int64_t count, int glu_kind, uint16_t* h,
           void* stream) {
    if (!gate || !up || !h || count < 1 || !glu_kind_ok(glu_kind)) return BL_ERR_INVALID_ARG;
    if (count > (int64_t{1} << 40)) return BL_ERR_INVALID_ARG;
    if (!aligned16(gate) || !aligned16(up) || !aligned16(h)) return BL_ERR_INVALID_ARG;
    if (int s = device_status()) return s;
    return hip_status(bl::launch_glu(gate, up, count, glu_kind, h, as_stream(stream)));
}

int bl_relu2_glu(const float* gate, const float* up, int64_t count, uint16_t* h, void* stream) {
    return bl_glu(gate, up, count, BL_GLU_RELU2, h, stream);
}

size_t bl_packed_bytes_binary(int64_t N, int64_t K) {
    if (!shape_ok(N, K)) return 0;
    return (size_t)N * (size_t)bl::packed_row_bytes_binary(K);
}

size_t bl_packed_bytes_base3(int64_t N, int64_t K) {
    if (!shape_ok(N, K)) return 0;
    return (size_t)N * (size_t)bl::packed_row_bytes_base3(K);
}

int bl_quantize_weights_binary(const float* W, int64_t N, int64_t K, uint32_t* W_bits,
                               float* gamma, void* workspace, size_t workspace_bytes,
                               void* stream) {
    if (!W || !W_bits || !gamma || !workspace) return BL_ERR_INVALID_ARG;
    if (!shape_ok(N, K)) return BL_ERR_INVALID_ARG;
    if (!aligned16(W) || !aligned16(W_bits)) return BL_ERR_INVALID_ARG;
    if ((reinterpret_cast<uintptr_t>(workspace) & 7u) != 0) return BL_ERR_INVALID_ARG;
    if (workspace_bytes < bl_quantize_weights_workspace_bytes(N, K)) return BL_ERR_INVALID_ARG;
    if (int s = device_status()) return s;
    return hip_status(bl::launch_quantize_weights_binary(
        W, N, K, W_bits, bl::packed_row_bytes_binary(K) / 4, gamma,
        static_cast<double*>(workspace), as_stream(stream)));
}

int bl_pack_base3(const uint32_t* W_packed, int64_t N, int64_t K, uint8_t* W3, void* stream) {
    if (!W_packed || !W3) return BL_ERR_INVALID_ARG;
    if (!shape_ok(N, K)) return BL_ERR_INVALID_ARG;
    if (!aligned16(W_packed) || !aligned16(W3)) return BL_ERR_INVALID_ARG;
    if (overlaps(W3, bl_packed_bytes_base3(N, K), W_packed, (size_t)(N * K) / 4))
        return BL_ERR_INVALID_ARG;
    if (int s = device_status()) return s;
    return hip_status(bl::launch_pack_base3(W_packed, N, K, W3, bl::packed_row_bytes_base3(K),
                                            as_stream(stream)));
}

namespace {

// Validation shared by the decode products of the other weight formats.
int other_format_args(const int8_t* x_q, const float* x_scale, int64_t M, int64_t K,
                      const void* W, size_t w_bytes, const float* gamma, int64_t N, float* y,
                      int32_t* acc, bool fits) {
    if (!x_q || !x_scale || !W || !gamma || !y) return BL_ERR_INVALID_ARG;
    if (!shape_ok(M, K) || !shape_ok(N, K)) return BL_ERR_INVALID_ARG;
    if (M > (int64_t{1} << 31) / N) return BL_ERR_INVALID_ARG;
    if (!aligned16(x_q) || !aligned16(W)) return BL_ERR_INVALID_ARG;
    if (!fits) return BL_ERR_INVALID_ARG;
    const size_t ny = (size_t)(M * N) * 4;
    if (overlaps(y, ny, x_q, (size_t)(M * K)) || overlaps(y, ny, x_scale, (size_t)M * 4) ||
        overlaps(y, ny, W, w_bytes) || overlaps(y, ny, gamma, 4))
        return BL_ERR_INVALID_ARG;
    if (acc && (overlaps(acc, ny, y, ny) || overlaps(acc, ny, x_q, (size_t)(M * K)) ||
                overlaps(acc, ny, x_scale, (size_t)M * 4) || overlaps(acc, ny, W, w_bytes) ||
                overlaps(acc, ny, gamma, 4)))
        return BL_ERR_INVALID_ARG;
    return device_status();
}

}  // namespace

int bl_bitlinear_binary(const int8_t* x_q, const float* x_scale, int64_t M, int64_t K,
                        const uint32_t* W_bits, const float* gamma, int64_t N, float* y,
                        int32_t* acc, void* stream) {
    const bool fits = shape_ok(M, K) && bl::gemv_binary_supported(M, K);
    if (int s = other_format_args(x_q, x_scale, M, K, W_bits, bl_packed_bytes_binary(N, K),
                                  gamma, N, y, acc, fits))
        return s;
    return hip_status(bl::launch_gemv_binary(x_q, x_scale, (int)M, (int)K, W_bits, gamma, (int)N,
                                             y, acc, as_stream(stream)));
}

int bl_bitlinear_base3(const int8_t* x_q, const float* x_scale, int64_t M, int64_t K,
                       const uint8_t* W3, const float* gamma, int64_t N, float* y, int32_t* acc,
                       void* stream) {
    const bool fits = shape_ok(M, K) && bl::gemv_base3_supported(M, K);
    if (int s = other_format_args(x_q, x_scale, M, K, W3, bl_packed_bytes_base3(N, K), gamma,
                                  N, y, acc, fits))
        return s;
    return hip_status(bl::launch_gemv_base3(x_q, x_scale, (int)M, (int)K, W3, gamma, (int)N, y,
                                            acc, as_stream(stream)));
}

size_t bl_ste_t_bytes(int64_t N, int64_t K) {
    if (!shape_ok(N, K)) return 0;
    return (size_t)K * (size_t)bl::ste_t_row_bytes(N);
}

int bl_pack_ste_t(const uint32_t* W_packed, int64_t N, int64_t K, uint8_t* qT, void* stream) {
    if (!W_packed || !qT) return BL_ERR_INVALID_ARG;
    if (!shape_ok(N, K)) return BL_ERR_INVALID_ARG;
    if (!aligned16(W_packed) || !aligned16(qT)) return BL_ERR_INVALID_ARG;
    if (overlaps(qT, bl_ste_t_bytes(N, K), W_packed, (size_t)(N * K) / 4))
        return BL_ERR_INVALID_ARG;
    if (int s = device_status()) return s;
    return hip_status(bl::launch_pack_ste_t(W_packed, N, K, qT, as_stream(stream)));
}

int bl_ste_backward_dx(const uint16_t* dy, int64_t M, int64_t N, const uint8_t* qT,
                       const float* gamma, int64_t K, float* dx, void* stream) {
    if (!dy || !qT || !gamma || !dx) return BL_ERR_INVALID_ARG;
    if (M < 1 || N < 8 || (N % 8) != 0 || !shape_ok(N, K)) return BL_ERR_INVALID_ARG;
    if (M > (int64_t{1} << 31) / N || M > (int64_t{1} << 31) / K) return BL_ERR_INVALID_ARG;
    if (!aligned16(dy) || !aligned16(qT)) return BL_ERR_INVALID_ARG;
    const size_t ndx = (size_t)(M * K) * 4;
    if (overlaps(dx, ndx, dy, (size_t)(M * N) * 2) || overlaps(dx, ndx, qT, bl_ste_t_bytes(N, K)) ||
        overlaps(dx, ndx, gamma, 4))
        return BL_ERR_INVALID_ARG;
    if (int s = device_status()) return s;
    return hip_status(bl::launch_ste_dx(dy, (int)M, (int)N, qT, gamma, (int)K, dx,
                                        as_stream(stream)));
}


size_t bl_ste_dw_workspace_bytes(int64_t M, int64_t N, int64_t K) {
    if (M < 1 || N < 8 || (N % 8) != 0 || !shape_ok(N, K)) return 0;
    if (M > (int64_t{1} << 31) / N || M > (int64_t{1} << 31) / K) return 0;
    const int64_t Mp = bl::ste_dw_padded_tokens(M);
    if (2 * Mp > (int64_t{1} << 31) / N) return 0;   // operand rows of 2 Mp values
    return bl::ste_dw_workspace_bytes(M, N, K);
}

int bl_ste_backward_dw(const uint16_t* dy, int64_t M, int64_t N, const int8_t* x_q,
                       const float* x_scale, int64_t K, float* dW, void* workspace,
                       size_t workspace_bytes, void* stream) {
    if (!dy || !x_q || !x_scale || !dW || !workspace) return BL_ERR_INVALID_ARG;
    const size_t need = bl_ste_dw_workspace_bytes(M, N, K);
    if (need == 0 || workspace_bytes < need) return BL_ERR_INVALID_ARG;
    if (!aligned16(dy) || !aligned16(x_q) || !aligned16(dW) ||
        (reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
        return BL_ERR_INVALID_ARG;
    const size_t ndw = (size_t)(N * K) * 4;
    if (overlaps(dW, ndw, dy, (size_t)(M * N) * 2) || overlaps(dW, ndw, x_q, (size_t)(M * K)) ||
        overlaps(dW, ndw, x_scale, (size_t)M * 4) || overlaps(dW, ndw, workspace, need) ||
        overlaps(workspace, need, dy, (size_t)(M * N) * 2) ||
        overlaps(workspace, need, x_q, (size_t)(M * K)) ||
        overlaps(workspace, need, x_scale, (size_t)M * 4))
        return BL_ERR_INVALID_ARG;
    if (int s = device_status()) return s;
    return hip_status(bl::launch_ste_dw(dy, (int)M, (int)N, x_q, x_scale, (int)K, dW, workspace,
                                        as_stream(stream)));
}

int bl_calib_read(const void* src, size_t bytes, uint32_t* sink, void* stream) {
    if (!src || !sink || bytes < 16 || (bytes % 16) != 0 || !aligned16(src))
        return BL_ERR_INVALID_ARG;
    if (int st = device_status()) return st;
    return hip_status(bl::launch_calib_read(src, bytes, sink, as_stream(stream)));
}

int bl_calib_copy(void* dst, const void* src, size_t bytes, void* stream) {
    if (!src || !dst || bytes < 16 || (bytes % 16) != 0 || !aligned16(src) || !aligned16(dst))
        return BL_ERR_INVALID_ARG;
    const uintptr_t a = reinterpret_cast<uintptr_t>(src), b = reinterpret_cast<uintptr_t>(dst);
    if (a < b + bytes && b < a + bytes) return BL_ERR_INVALID_ARG;
    if (int st = device_status()) return st;
    return hip_status(bl::launch_calib_copy(dst, src, bytes, as_stream(stream)));
}

int64_t bl_calib_mfma_i8_ops(int64_t iters) {
    if (iters < 1 || iters > (int64_t{1} << 24)) return 0;
    return bl::calib_mfma_ops(iters);
}

size_t bl_calib_mfma_i8_sink_elems(void) { return (size_t)bl::kCalibMfmaBlocks * 256; }

int bl_calib_mfma_i8(int64_t iters, int32_t* sink, void* stream) {
    if (!sink || iters < 1 || iters > (int64_t{1} << 24)) return BL_ERR_INVALID_ARG;
    if (int st = device_status()) return st;
    return hip_status(bl::launch_calib_mfma((int)iters, sink, as_stream(stream)));
}

}  // extern "C"
