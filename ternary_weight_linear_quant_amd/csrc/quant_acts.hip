// Per-token absmax int8 activation quantisation, optionally fused with the
// RMSNorm that precedes BitLinear.
//
// Source: comrad404.com, "BitNet b1.58: что показала работа Microsoft об
// «эре 1-битных LLM»", section «Метод: как устроен BitNet b1.58»: activations
// are carried as 8-bit integers, and the input is normalised (RMSNorm) before
// it is quantised.
//
// One workgroup per token. Pass 1 reduces max|z| (exact, order-free) and, when
// fused, sum x^2 in fp64; pass 2 re-reads the token (L2-resident) and writes
// the codes. Codes: rne(z * (127/a)) clamped to [-127, 127] in fp32; since a
// positive per-token factor cancels in absmax quantisation, the codes of
// RMSNorm(x) are those of z = x*g (exact in fp32) and 1/rms goes into the
// scale. Roofline: HBM, 2 B read + 1 B written per element.
#include "common.hpp"
#include "launch.hpp"

namespace bl {

constexpr int kActThreads = 256;

template <bool FUSED>
__global__ __launch_bounds__(kActThreads) void k_act_quant(
    const uint16_t* __restrict__ x, int64_t K, const uint16_t* __restrict__ gain,
    float rms_eps, int8_t* __restrict__ xq, float* __restrict__ scale) {
    const int64_t m = blockIdx.x;
    const uint4* row = reinterpret_cast<const uint4*>(x + m * K);
    const uint4* grow = reinterpret_cast<const uint4*>(gain);
    const int tid = threadIdx.x;
    const int64_t nvec = K / 8;  // 8 bf16 per 16 bytes

    float amax = 0.0f;
    double ss = 0.0;
    for (int64_t v = tid; v < nvec; v += kActThreads) {
        const uint4 d = row[v];
        const uint32_t dw[4] = {d.x, d.y, d.z, d.w};
        uint32_t gw[4] = {0, 0, 0, 0};
        if (FUSED) {
            const uint4 g = grow[v];
            gw[0] = g.x; gw[1] = g.y; gw[2] = g.z; gw[3] = g.w;
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const float xf = bf16_to_f32((dw[i] >> (16 * h)) & 0xFFFFu);
                float z = xf;
                if (FUSED) {
                    z = xf * bf16_to_f32((gw[i] >> (16 * h)) & 0xFFFFu);
                    ss += (double)xf * (double)xf;
                }
                amax = fmaxf(amax, fabsf(z));
            }
        }
    }

    __shared__ float s_max[kActThreads / kWave];
    __shared__ double s_ss[kActThreads / kWave];
    amax = wave_max(amax);
    if (FUSED) ss = wave_sum(ss);
    const int wave = tid / kWave;
    if ((tid % kWave) == 0) {
        s_max[wave] = amax;
        if (FUSED) s_ss[wave] = ss;
    }
    __syncthreads();
    amax = s_max[0];
    double ss_tot = FUSED ? s_ss[0] : 0.0;
#pragma unroll
    for (int w = 1; w < kActThreads / kWave; ++w) {
        amax = fmaxf(amax, s_max[w]);
        if (FUSED) ss_tot += s_ss[w];
    }
    const float a = amax > 1e-5f ? amax : 1e-5f;
    const float inv = 127.0f / a;  // correctly rounded

    uint2* out = reinterpret_cast<uint2*>(xq + m * K);
    for (int64_t v = tid; v < nvec; v += kActThreads) {
        const uint4 d = row[v];
        const uint32_t dw[4] = {d.x, d.y, d.z, d.w};
        uint32_t gw[4] = {0, 0, 0, 0};
        if (FUSED) {
            const uint4 g = grow[v];
            gw[0] = g.x; gw[1] = g.y; gw[2] = g.z; gw[3] = g.w;
        }
        uint32_t packed[2] = {0, 0};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                float z = bf16_to_f32((dw[i] >> (16 * h)) & 0xFFFFu);
                if (FUSED) z = z * bf16_to_f32((gw[i] >> (16 * h)) & 0xFFFFu);
                float t = __builtin_rintf(z * inv);
                t = fminf(fmaxf(t, -127.0f), 127.0f);
                const uint32_t b = (uint32_t)((int)t) & 0xFFu;
                const int e = 2 * i + h;  // element 0..7 of the vector
                packed[e / 4] |= b << (8 * (e % 4));
            }
        }
        out[v] = make_uint2(packed[0], packed[1]);
    }
    if (tid == 0) {
        if (FUSED) {
            const double rms = sqrt(ss_tot / (double)K + (double)rms_eps);
            scale[m] = (float)((double)a / (127.0 * rms));
        } else {
            scale[m] = a / 127.0f;
        }
    }
}

hipError_t launch_quantize_acts(const uint16_t* x, int64_t M, int64_t K, const uint16_t* gain,
                                float rms_eps, int8_t* xq, float* scale, hipStream_t stream) {
    if (gain)
        hipLaunchKernelGGL(k_act_quant<true>, dim3((unsigned)M), dim3(kActThreads), 0, stream, x,
                           K, gain, rms_eps, xq, scale);
    else
        hipLaunchKernelGGL(k_act_quant<false>, dim3((unsigned)M), dim3(kActThreads), 0, stream, x,
                           K, gain, rms_eps, xq, scale);
    return hipGetLastError();
}

}  // namespace bl
