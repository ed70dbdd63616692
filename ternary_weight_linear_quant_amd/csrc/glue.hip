// Squared-ReLU gating between the gate/up and down BitLinears of a 2B4T-style
// FFN: h = bf16_rne((relu(gate)^2) * up), fp32 arithmetic.
//
// Source: inferownia.pl, "BitNet b1.58: era 1-bitowych LLM-ów", section "Zrób
// to sam — Microsoft wypuścił konkretny model", and kripta.biz (BitNet b1.58
// 2B4T article): the 2B4T FFN uses squared ReLU. Elementwise, HBM-bound:
// 8 B read + 2 B written per element.
#include "common.hpp"
#include "launch.hpp"

namespace bl {

__device__ __forceinline__ uint32_t relu2_gate(float g, float u) {
    const float r = g > 0.0f ? g : 0.0f;
    const float sq = r * r;
    return f32_to_bf16_rne(sq * u);
}

__global__ __launch_bounds__(256) void k_relu2_glu(const float* __restrict__ g,
                                                   const float* __restrict__ u, int64_t count,
                                                   uint16_t* __restrict__ h) {
    const int64_t nvec = count / 4;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < nvec; i += stride) {
        const float4 gv = reinterpret_cast<const float4*>(g)[i];
        const float4 uv = reinterpret_cast<const float4*>(u)[i];
        const uint32_t lo = relu2_gate(gv.x, uv.x) | (relu2_gate(gv.y, uv.y) << 16);
        const uint32_t hi = relu2_gate(gv.z, uv.z) | (relu2_gate(gv.w, uv.w) << 16);
        reinterpret_cast<uint2*>(h)[i] = make_uint2(lo, hi);
    }
    if (blockIdx.x == 0) {
        for (int64_t i = 4 * nvec + threadIdx.x; i < count; i += blockDim.x)
            h[i] = (uint16_t)relu2_gate(g[i], u[i]);
    }
}

hipError_t launch_relu2_glu(const float* g, const float* u, int64_t count, uint16_t* h,
                            hipStream_t stream) {
    const int threads = 256;
    int64_t blocks = (count / 4 + threads - 1) / threads;
    if (blocks < 1) blocks = 1;
    if (blocks > 8192) blocks = 8192;
    hipLaunchKernelGGL(k_relu2_glu, dim3((unsigned)blocks), dim3(threads), 0, stream, g, u, count,
                       h);
    return hipGetLastError();
}

}  // namespace bl
