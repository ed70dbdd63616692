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

// R[n] = sum_k |W[n][k]|, fp64, k increasing. A workgroup takes 32 rows and
// walks K in tiles of 256 columns: all 256 threads load a tile with
// coalesced 16-byte loads (64 lanes per 1 KB row segment) into LDS (rows
// padded to 260 floats, so the 32 readers of one column offset hit distinct
// banks), then thread r runs row r's chain over the tile while the next
// tile's loads are in flight.
constexpr int kRsRows = 32, kRsTK = 256, kRsThreads = 256;
constexpr int kRsPitch = kRsTK + 4;
constexpr int kRsLoads = kRsRows * kRsTK / 4 / kRsThreads;  // float4 per thread per tile

__global__ __launch_bounds__(kRsThreads) void k_absmean_rowsum(
    const float* __restrict__ W, int64_t N, int64_t K, double* __restrict__ R) {
    __shared__ __align__(16) float tile[kRsRows * kRsPitch];
    const int tid = threadIdx.x;
    const int64_t n0 = (int64_t)blockIdx.x * kRsRows;
    float4 reg[kRsLoads];
    auto load = [&](int64_t k0) {
#pragma unroll
        for (int i = 0; i < kRsLoads; ++i) {
            const int f = tid + kRsThreads * i;
            const int r = f / (kRsTK / 4), c4 = f % (kRsTK / 4);
            const int64_t row = n0 + r, col = k0 + 4 * c4;
            reg[i] = (row < N && col < K)
                         ? *reinterpret_cast<const float4*>(W + row * K + col)
                         : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
        }
    };
    double s = 0.0;
    load(0);
    for (int64_t k0 = 0; k0 < K; k0 += kRsTK) {
#pragma unroll
        for (int i = 0; i < kRsLoads; ++i) {
            const int f = tid + kRsThreads * i;
            const int r = f / (kRsTK / 4), c4 = f % (kRsTK / 4);
            *reinterpret_cast<float4*>(&tile[r * kRsPitch + 4 * c4]) = reg[i];
        }
        __syncthreads();
        if (k0 + kRsTK < K) load(k0 + kRsTK);
        if (tid < kRsRows) {
            // K % 64 == 0: the tile holds a whole number of float4.
            const int cnt4 = (int)((K - k0 < kRsTK ? K - k0 : kRsTK) / 4);
            const float* row = &tile[tid * kRsPitch];
#pragma unroll 8
            for (int c = 0; c < cnt4; ++c) {
                const float4 v = *reinterpret_cast<const float4*>(row + 4 * c);
                s += (double)fabsf(v.x);
                s += (double)fabsf(v.y);
                s += (double)fabsf(v.z);
                s += (double)fabsf(v.w);
            }
        }
        __syncthreads();
    }
    if (tid < kRsRows && n0 + tid < N) R[n0 + tid] = s;
}

// gamma = (float)((sum_n R[n], n increasing) / (N*K)). The row sums are
// staged through LDS by the whole block in coalesced tiles; thread 0 adds
// them in order, reading each batch of 16 from LDS while it adds the
// previous one. The last batch of a tile is padded with +0.0, which leaves
// the (non-negative) running sum unchanged bit for bit.
__global__ __launch_bounds__(256) void k_gamma_finalize(
    const double* __restrict__ R, int64_t N, int64_t K, float* __restrict__ gamma) {
    constexpr int kTile = 4096, kB = 16;
    __shared__ double tile[kTile];
    double s = 0.0;
    for (int64_t base = 0; base < N; base += kTile) {
        const int cnt = (int)((N - base) < kTile ? (N - base) : kTile);
        const int padded = (cnt + kB - 1) / kB * kB;
        for (int i = threadIdx.x; i < padded; i += blockDim.x)
            tile[i] = i < cnt ? R[base + i] : 0.0;
        __syncthreads();
        if (threadIdx.x == 0) {
            double cur[kB];
#pragma unroll
            for (int j = 0; j < kB; ++j) cur[j] = tile[j];
            for (int i = 0; i < padded; i += kB) {
                double nxt[kB];
                const int nb = i + kB < padded ? i + kB : i;  // last batch: harmless re-read
#pragma unroll
                for (int j = 0; j < kB; ++j) nxt[j] = tile[nb + j];
#pragma unroll
                for (int j = 0; j < kB; ++j) s += cur[j];
#pragma unroll
                for (int j = 0; j < kB; ++j) cur[j] = nxt[j];
            }
        }
        __syncthreads();
    }
    if (threadIdx.x == 0) *gamma = (float)(s / (double)(N * K));
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
        const int64_t blocks = (N + kRsRows - 1) / kRsRows;
        hipLaunchKernelGGL(k_absmean_rowsum, dim3((unsigned)blocks), dim3(kRsThreads), 0, stream,
                           W, N, K, rowsums);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(k_gamma_finalize, dim3(1), dim3(256), 0, stream, rowsums, N, K, gamma);
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

// Binary weights of the original BitNet (inferownia.pl page above, section
// "Dlaczego akurat ternarne, a nie czyste zero-jeden": only -1 and +1): the
// sign of the latent weight, W >= 0 (either zero) giving +1, stored at one
// bit per weight -- word k/32 of the row, bit 8*(i%4) + i/4 for i = k%32, so
// that (w >> p) & 0x01010101 holds four consecutive weights. Rows are
// row_words words (16-byte multiples); bits past K are 0. One thread per
// word.
__global__ __launch_bounds__(256) void k_binarize_pack(
    const float* __restrict__ W, int64_t N, int64_t K, int64_t row_words,
    uint32_t* __restrict__ out) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= N * row_words) return;
    const int64_t n = i / row_words, j = i - n * row_words;
    uint32_t word = 0;
    if (32 * j < K) {  // K % 64 == 0: a word is wholly inside or past the row
        const float4* src = reinterpret_cast<const float4*>(W + n * K + 32 * j);
#pragma unroll
        for (int v = 0; v < 8; ++v) {
            const float4 f = src[v];
            const float e[4] = {f.x, f.y, f.z, f.w};
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const int b = 4 * v + t;  // weight index within the word
                if (e[t] >= 0.0f) word |= 1u << (8 * (b % 4) + b / 4);
            }
        }
    }
    out[i] = word;
}

// Ternary codes at five per byte (same page, section "Skąd te 1,58 bita":
// log2(3) bits carry a ternary value): byte j of a row is the base-3 number
// sum_{i<5} c_i 3^i of codes c = q + 1 at k = 5j + i (least significant
// digit first), read from the 2-bit packing; positions k >= K count as
// weight 0 (c = 1), so padding bytes are 121. One thread per output byte.
__global__ __launch_bounds__(256) void k_pack_base3(
    const uint32_t* __restrict__ P2, int64_t N, int64_t K, int64_t row_bytes,
    uint8_t* __restrict__ out) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= N * row_bytes) return;
    const int64_t n = i / row_bytes, j = i - n * row_bytes;
    const uint32_t* row = P2 + n * (K / 16);
    int v = 0;
#pragma unroll
    for (int d = 4; d >= 0; --d) {  // Horner, most significant digit first
        const int64_t k = 5 * j + d;
        int c = 1;
        if (k < K) {
            const int t = (int)(k % 16);
            c = (int)((row[k / 16] >> (8 * (t % 4) + 2 * (t / 4))) & 3u);
        }
        v = 3 * v + c;
    }
    out[i] = (uint8_t)v;
}

hipError_t launch_quantize_weights_binary(const float* W, int64_t N, int64_t K, uint32_t* packed,
                                          int64_t row_words, float* gamma, double* rowsums,
                                          hipStream_t stream) {
    {
        const int64_t blocks = (N + kRsRows - 1) / kRsRows;
        hipLaunchKernelGGL(k_absmean_rowsum, dim3((unsigned)blocks), dim3(kRsThreads), 0, stream,
                           W, N, K, rowsums);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(k_gamma_finalize, dim3(1), dim3(256), 0, stream, rowsums, N, K, gamma);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int threads = 256;
    const int64_t blocks = (N * row_words + threads - 1) / threads;
    hipLaunchKernelGGL(k_binarize_pack, dim3((unsigned)blocks), dim3(threads), 0, stream, W, N, K,
                       row_words, packed);
    return hipGetLastError();
}

hipError_t launch_pack_base3(const uint32_t* packed2, int64_t N, int64_t K, uint8_t* out,
                             int64_t row_bytes, hipStream_t stream) {
    const int threads = 256;
    const int64_t blocks = (N * row_bytes + threads - 1) / threads;
    hipLaunchKernelGGL(k_pack_base3, dim3((unsigned)blocks), dim3(threads), 0, stream, packed2, N,
                       K, row_bytes, out);
    return hipGetLastError();
}

}  // namespace bl
