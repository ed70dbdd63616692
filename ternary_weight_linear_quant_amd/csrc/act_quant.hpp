// Device helpers of the per-token absmax activation quantisation, shared by
// the stand-alone quantiser (k_act_quant) and the one-token GEMV that
// quantises its own input: both take the same decisions in the same order, so
// they produce the same codes and the same scale bit for bit.
//
// Source: comrad404.com, "BitNet b1.58: что показала работа Microsoft об
// «эре 1-битных LLM»", section «Метод: как устроен BitNet b1.58»: activations
// are carried as 8-bit integers and the input is normalised (RMSNorm) before it
// is quantised. Codes: rne(z * (127/a)) clamped to [-127, 127] in fp32, with
// z = x (plain) or z = x*g (RMSNorm gain g: a positive per-token factor cancels
// in absmax quantisation, so 1/rms goes into the scale), a = max(max|z|,
// 1e-5); scale a/127, or a / (127 * rms) with rms = sqrt(sum x^2 / K + eps)
// and sum x^2 in fp64.
#pragma once

#include "common.hpp"

namespace bl {

constexpr int kActThreads = 256;  // threads that hold one token's values

// Reduction over the first kActThreads threads of the workgroup, in a fixed
// order: a butterfly within each wave, then waves 0, 1, 2, 3 in turn (for the
// fp64 sum of squares the order decides the rounding). Every thread of the
// workgroup calls it, since it holds a barrier; threads past kActThreads pass
// a neutral value and are left out. The result reaches every thread.
// `scratch` holds kActThreads / 64 entries.
template <typename T, bool MAX>
__device__ __forceinline__ T act_reduce(T v, T* scratch) {
    const int wave = threadIdx.x / kWave;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        const T other = __shfl_xor(v, o, kWave);
        v = MAX ? (v > other ? v : other) : v + other;
    }
    if ((threadIdx.x % kWave) == 0 && wave < kActThreads / kWave) scratch[wave] = v;
    __syncthreads();
    T r = scratch[0];
#pragma unroll
    for (int w = 1; w < kActThreads / kWave; ++w) r = MAX ? (r > scratch[w] ? r : scratch[w]) : r + scratch[w];
    return r;
}

// Running max|z| (and, with a gain, sum x^2 in fp64) over 8 bf16 values (one
// 16-byte vector `d`, gain vector `gv`), in element order.
template <bool NORM>
__device__ __forceinline__ void act_scan8(const uint4 d, const uint4 gv, float& amax, double& ss) {
    const uint32_t dw[4] = {d.x, d.y, d.z, d.w};
    const uint32_t gw[4] = {gv.x, gv.y, gv.z, gv.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const float xf = bf16_to_f32((dw[i] >> (16 * h)) & 0xFFFFu);
            float z = xf;
            if (NORM) {
                z = xf * bf16_to_f32((gw[i] >> (16 * h)) & 0xFFFFu);
                ss += (double)xf * (double)xf;
            }
            amax = fmaxf(amax, fabsf(z));
        }
    }
}

// 8 bf16 values (one 16-byte vector) -> 8 int8 codes packed in a uint2.
template <bool NORM>
__device__ __forceinline__ uint2 act_quant8(const uint4 d, const uint4 gv, float inv) {
    const uint32_t dw[4] = {d.x, d.y, d.z, d.w};
    const uint32_t gw[4] = {gv.x, gv.y, gv.z, gv.w};
    uint32_t packed[2] = {0, 0};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            float z = bf16_to_f32((dw[i] >> (16 * h)) & 0xFFFFu);
            if (NORM) z = z * bf16_to_f32((gw[i] >> (16 * h)) & 0xFFFFu);
            float t = __builtin_rintf(z * inv);
            t = fminf(fmaxf(t, -127.0f), 127.0f);
            const uint32_t b = (uint32_t)((int)t) & 0xFFu;
            const int e = 2 * i + h;
            packed[e / 4] |= b << (8 * (e % 4));
        }
    }
    return make_uint2(packed[0], packed[1]);
}

// a = max(max|z|, 1e-5); the codes' multiplier 127/a (correctly rounded).
__device__ __forceinline__ float act_clamped_max(float amax) { return amax > 1e-5f ? amax : 1e-5f; }

// The dequantisation scale of a token.
template <bool NORM>
__device__ __forceinline__ float act_scale(float a, double ss_tot, int64_t K, float rms_eps) {
    if (NORM) {
        const double rms = sqrt(ss_tot / (double)K + (double)rms_eps);
        return (float)((double)a / (127.0 * rms));
    }
    return a / 127.0f;
}

}  // namespace bl
