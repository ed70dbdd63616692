// Gating between the gate/up and down BitLinears of a gated FFN:
// h = bf16_rne(act(gate) * up), fp32 arithmetic, act = relu^2 or SiLU.
//
// Source: inferownia.pl, "BitNet b1.58: era 1-bitowych LLM-ów", section "Zrób
// to sam — Microsoft wypuścił konkretny model", and kripta.biz (BitNet b1.58
// 2B4T article): the 2B4T FFN uses squared ReLU; comrad404.com, "BitNet
// b1.58: что показала работа Microsoft об «эре 1-битных LLM»", section
// «Метод: как устроен BitNet b1.58»: the b1.58 variant keeps the LLaMA
// stack's SwiGLU. Elementwise, HBM-bound: 8 B read + 2 B written per element.
#include "common.hpp"
#include "launch.hpp"

namespace bl {

template <int KIND>
__global__ __launch_bounds__(256) void k_glu(const float* __restrict__ g,
                                             const float* __restrict__ u, int64_t count,
                                             uint16_t* __restrict__ h) {
    const int64_t nvec = count / 4;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < nvec; i += stride) {
        const float4 gv = reinterpret_cast<const float4*>(g)[i];
        const float4 uv = reinterpret_cast<const float4*>(u)[i];
        const uint32_t lo = glu_bits<KIND>(gv.x, uv.x) | (glu_bits<KIND>(gv.y, uv.y) << 16);
        const uint32_t hi = glu_bits<KIND>(gv.z, uv.z) | (glu_bits<KIND>(gv.w, uv.w) << 16);
        reinterpret_cast<uint2*>(h)[i] = make_uint2(lo, hi);
    }
    if (blockIdx.x == 0) {
        for (int64_t i = 4 * nvec + threadIdx.x; i < count; i += blockDim.x)
            h[i] = (uint16_t)glu_bits<KIND>(g[i], u[i]);
    }
}

hipError_t launch_glu(const float* g, const float* u, int64_t count, int kind, uint16_t* h,
                      hipStream_t stream) {
    const int threads = 256;
    int64_t blocks = (count / 4 + threads - 1) / threads;
    if (blocks < 1) blocks = 1;
    if (blocks > 8192) blocks = 8192;
    if (kind == kGluSwiglu)
        hipLaunchKernelGGL(k_glu<kGluSwiglu>, dim3((unsigned)blocks), dim3(threads), 0, stream, g,
                           u, count, h);
    else
        hipLaunchKernelGGL(k_glu<kGluRelu2>, dim3((unsigned)blocks), dim3(threads), 0, stream, g,
                           u, count, h);
    return hipGetLastError();
}

}  // namespace bl
