// Absmean ternary weight quantisation and 2-bit packing (offline, per matrix).
//
// Source: inferownia.pl, "BitNet b1.58: era 1-bitowych LLM-ów", section
// "„Trenowany od zera” — i czemu to nie jest zwykła kwantyzacja": the whole
// matrix is scaled by its mean absolute value, then each entry goes to the
// nearest integer of {-1, 0, +1}; section "Skąd te 1,58 bita": a ternary value
// is stored in two bits in practice.
//
// gamma is defined with a fixed fp64 summation order so that it is bit-exact
// and shard-invariant: one fp64 chain per row in increasing k, then one chain
// over the row sums in increasing n. Weights are read once per pass; the
// passes are offline and bound by reading the fp32 matrix (4 B/weight).
#include "common.hpp"
#include "launch.hpp"

namespace bl {

// R[n] = sum_k |W[n][k]|, fp64, k increasing. One thread per row.
__global__ __launch_bounds__(64) void k_absmean_rowsum(
    const float* __restrict__ W, int64_t N, int64_t K, double* __restrict__ R) {
    const int64_t n = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (n >= N) return;
    const float4* row = reinterpret_cast<const float4*>(W + n * K);
    const int64_t K4 = K / 4;
    double s = 0.0;
#pragma unroll 8
    for (int64_t j = 0; j < K4; ++j) {
        const float4 v = row[j];
        s += (double)fabsf(v.x);
        s += (double)fabsf(v.y);
        s += (double)fabsf(v.z);
        s += (double)fabsf(v.w);
    }
    R[n] = s;
}

// gamma = (float)((sum_n R[n], n increasing) / (N*K)). One thread.
__global__ __launch_bounds__(64) void k_gamma_finalize(
    const double* __restrict__ R, int64_t N, int64_t K, float* __restrict__ gamma) {
    if (threadIdx.x != 0) return;
    double s = 0.0;
#pragma unroll 8
    for (int64_t n = 0; n < N; ++n) s += R[n];
    *gamma = (float)(s / (double)(N * K));
}

// One thread per packed word: 16 consecutive weights of one row.
// q = clamp(rne(w / (gamma + 1e-5f)), -1, 1); code c = q + 1 at bit
// 8*(i%4) + 2*(i/4) for weight i of the word.
__global__ __launch_bounds__(256) void k_ternarize_pack(
    const float* __restrict__ W, int64_t total_words, const float* __restrict__ gamma,
    uint32_t* __restrict__ out) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= total_words) return;
    const float s = *gamma + 1e-5f;
    const float4* src = reinterpret_cast<const float4*>(W) + 4 * i;
    uint32_t word = 0;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
        const float4 f = src[v];
        const float e[4] = {f.x, f.y, f.z, f.w};
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            // IEEE division (correctly rounded; the library is built with
            // -fhip-fp32-correctly-rounded-divide-sqrt and no fast-math).
            float q = __builtin_rintf(e[t] / s);
            q = fminf(fmaxf(q, -1.0f), 1.0f);
            const uint32_t c = (uint32_t)((int)q + 1);
            // weight index within the word is 4v + t: byte t, bit-pair v.
            word |= c << (8 * t + 2 * v);
        }
    }
    out[i] = word;
}

hipError_t launch_quantize_weights(const float* W, int64_t N, int64_t K, uint32_t* packed,
                                   float* gamma, double* rowsums, hipStream_t stream) {
    {
        const int threads = 64;
        const int64_t blocks = (N + threads - 1) / threads;
        hipLaunchKernelGGL(k_absmean_rowsum, dim3((unsigned)blocks), dim3(threads), 0, stream,
                           W, N, K, rowsums);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(k_gamma_finalize, dim3(1), dim3(64), 0, stream, rowsums, N, K, gamma);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    {
        const int threads = 256;
        const int64_t words = N * (K / 16);
        const int64_t blocks = (words + threads - 1) / threads;
        hipLaunchKernelGGL(k_ternarize_pack, dim3((unsigned)blocks), dim3(threads), 0, stream,
                           W, words, gamma, packed);
    }
    return hipGetLastError();
}

}  // namespace bl
