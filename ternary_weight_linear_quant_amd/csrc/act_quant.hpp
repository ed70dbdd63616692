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

#include <type_traits>

#include "common.hpp"

namespace bl {

constexpr int kActThreads = 256;  // threads that hold one token's values

// Reduction over the first NW waves of the workgroup, in a fixed order: a
// butterfly within each wave, then waves 0, 1, ..., NW-1 in turn (for the fp64
// sum of squares the order decides the rounding). Every thread of the
// workgroup calls it, since it holds a barrier; threads of later waves pass a
// neutral value and are left out. The result reaches every thread. `scratch`
// holds NW entries. The max (of magnitudes: finite and at least +0, where the
// float order is the unsigned order of the bits) runs on DPP instead of the
// butterfly; a max is exact in any order.
template <typename T, bool MAX, int NW = kActThreads / kWave>
__device__ __forceinline__ T act_reduce(T v, T* scratch) {
    const int wave = threadIdx.x / kWave;
    if constexpr (MAX && std::is_same<T, float>::value) {
        v = __uint_as_float(wave_max_u32(__float_as_uint(v)));
    } else {
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) {
            const T other = __shfl_xor(v, o, kWave);
            v = MAX ? (v > other ? v : other) : v + other;
        }
    }
    if ((threadIdx.x % kWave) == 0 && wave < NW) scratch[wave] = v;
    __syncthreads();
    T r = scratch[0];
#pragma unroll
    for (int w = 1; w < NW; ++w) r = MAX ? (r > scratch[w] ? r : scratch[w]) : r + scratch[w];
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

// Plain quantisation's max|x| on the raw bits: for finite bf16 values the
// magnitude order is the integer order of the low 15 bits, so a packed
// 16-bit integer max over (bits & 0x7FFF) per half finds the largest
// magnitude exactly (one AND and one max per two values). `m2` accumulates
// both halves; act_bits_max turns it into the float max|x|.
typedef unsigned short act_u16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ void act_scan8_bits(const uint4 d, act_u16x2& m2) {
    const uint32_t dw[4] = {d.x, d.y, d.z, d.w};
#pragma unroll
    for (int i = 0; i < 4; ++i)
        m2 = __builtin_elementwise_max(m2, __builtin_bit_cast(act_u16x2, dw[i] & 0x7FFF7FFFu));
}

__device__ __forceinline__ float act_bits_max(act_u16x2 m2) {
    return bf16_to_f32(m2.x > m2.y ? m2.x : m2.y);
}

// 8 bf16 values (one 16-byte vector) -> 8 int8 codes packed in a uint2.
// t = z * inv in fp32 (|t| <= 127 (1 + 2^-24)^2 since |z| <= a and inv =
// fl(127/a), so the [-127, 127] clamp can never act); pack_codes4 rounds each
// t to nearest even with the 1.5 * 2^23 add, the result of rintf.
template <bool NORM>
__device__ __forceinline__ uint2 act_quant8(const uint4 d, const uint4 gv, float inv) {
    const uint32_t dw[4] = {d.x, d.y, d.z, d.w};
    const uint32_t gw[4] = {gv.x, gv.y, gv.z, gv.w};
    float t[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        // bf16 pair -> fp32: the low half shifted up, the high half masked.
        float z0 = __uint_as_float(dw[i] << 16), z1 = __uint_as_float(dw[i] & 0xFFFF0000u);
        if (NORM) {
            z0 = z0 * __uint_as_float(gw[i] << 16);
            z1 = z1 * __uint_as_float(gw[i] & 0xFFFF0000u);
        }
        t[2 * i] = z0 * inv;
        t[2 * i + 1] = z1 * inv;
    }
    return make_uint2(pack_codes4(t[0], t[1], t[2], t[3]), pack_codes4(t[4], t[5], t[6], t[7]));
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
