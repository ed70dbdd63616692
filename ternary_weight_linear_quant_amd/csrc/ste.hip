// Straight-through backward of BitLinear with respect to its input.
//
// Source: juhe.plus (Habr repost), the section on training that follows
// BinaryConnect: the rounding function has no useful derivative, so the
// forward pass rounds and the backward pass lets the gradient through as if
// there were no rounding (straight-through estimator); comrad404.com,
// "BitNet b1.58: что показала работа Microsoft об «эре 1-битных LLM»",
// section «Метод: как устроен BitNet b1.58»: gradients stay in high
// precision. For y = x~ . (gamma q)^T this gives
//     dx[m][k] = gamma * sum_n dy[m][n] * q[n][k]
// with dy in bf16: the transposed ternary product, rescaled.
//
// The ternary weights enter the bf16 matrix cores directly: q is first
// transposed once (offline, like the forward packing) into rows of k with
// four consecutive n per byte, so a 2-byte read gives the 8 reduction values
// of one lane of a v_mfma_f32_32x32x16_bf16 B fragment, decoded through a
// 256-entry LDS table of four bf16 values {-1, 0, +1}. Products of bf16 by
// {-1, 0, +1} are exact; the sums accumulate in fp32.
//
// Tile: 128 (tokens) x 128 (input features), 4 waves in a 2 x 2 grid of
// 64 x 64, reduction steps of 32 n double-buffered through registers into
// LDS. dy rows in LDS are padded to 80 bytes, which keeps the 16-byte
// fragment reads of 8 consecutive rows on distinct banks.
//
// Roofline: MFMA (bf16). Work per call = 2*M*N*K flops.
#include "common.hpp"
#include "launch.hpp"

namespace bl {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kSteBM = 128, kSteBN = 128, kSteBR = 32;
constexpr int kSteThreads = 256;
constexpr int kSteARow = kSteBR * 2 + 16;  // bytes per padded dy row in LDS
constexpr int kSteBRow = kSteBR / 4;       // code bytes per qT row per step

int64_t ste_t_row_bytes(int64_t N) { return 16 * (((N + 3) / 4 + 15) / 16); }

// qT[k][j] = codes (q[4j+i][k] + 1) at bits 2i, i < 4, from the 2-bit
// forward packing (word k/16 of row n, bits 8*(t%4) + 2*(t/4), t = k%16);
// n >= N gives code 1 (weight 0). One thread per output byte, k fastest so
// that a wave reads few distinct words.
__global__ __launch_bounds__(256) void k_pack_ste_t(const uint32_t* __restrict__ P2, int64_t N,
                                                    int64_t K, int64_t row_bytes,
                                                    uint8_t* __restrict__ qT) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= K * row_bytes) return;
    const int64_t j = i / K, k = i - j * K;
    const int t = (int)(k % 16);
    const int shift = 8 * (t % 4) + 2 * (t / 4);
    uint32_t v = 0;
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) {
        const int64_t n = 4 * j + ii;
        const uint32_t c = n < N ? (P2[n * (K / 16) + k / 16] >> shift) & 3u : 1u;
        v |= c << (2 * ii);
    }
    qT[k * row_bytes + j] = (uint8_t)v;
}

__device__ __forceinline__ uint32_t bf16_of_code(uint32_t c) {
    return c == 0 ? 0xBF80u : c == 2 ? 0x3F80u : 0u;  // weight c - 1; code 3 unused -> 0
}

__global__ __launch_bounds__(kSteThreads, 2) void k_ste_dx(
    const uint16_t* __restrict__ dy, int M, int N, const uint8_t* __restrict__ qT, int RBT,
    const float* __restrict__ gamma_p, int K, float* __restrict__ dx) {
    __shared__ __align__(16) uint8_t As[2][kSteBM * kSteARow];
    __shared__ __align__(16) uint8_t Bs[2][kSteBN * kSteBRow];
    __shared__ uint2 lut[256];

    const int tid = threadIdx.x;
    const int lane = tid % kWave;
    const int wave = tid / kWave;
    const int wm0 = (wave % 2) * 64, wn0 = (wave / 2) * 64;
    const int tilesN = (K + kSteBN - 1) / kSteBN;
    const int m0 = ((int)blockIdx.x / tilesN) * kSteBM;
    const int k0 = ((int)blockIdx.x % tilesN) * kSteBN;

    // Table: byte b -> four bf16 weights of its codes, low code first.
    {
        const uint32_t b = (uint32_t)tid;
        const uint32_t lo = bf16_of_code(b & 3u) | (bf16_of_code((b >> 2) & 3u) << 16);
        const uint32_t hi = bf16_of_code((b >> 4) & 3u) | (bf16_of_code((b >> 6) & 3u) << 16);
        lut[b] = make_uint2(lo, hi);
    }

    // Stage loads: dy 128 rows x 64 bytes (two 16-byte chunks per thread),
    // qT 128 rows x 8 bytes (threads 0..127). Rows past M or K are clamped
    // (their results are not stored); chunks past N are zero.
    const int steps = (N + kSteBR - 1) / kSteBR;
    uint4 ra[2];
    uint2 rb = make_uint2(0x55555555u, 0x55555555u);
    auto load = [&](int st) {
        const int n0 = st * kSteBR;
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int c = tid + kSteThreads * i;  // chunk 0..511: row c/4, part c%4
            const int row = min(m0 + c / 4, M - 1);
            const int n = n0 + 8 * (c % 4);
            ra[i] = n < N ? *reinterpret_cast<const uint4*>(dy + (size_t)row * N + n)
                          : make_uint4(0, 0, 0, 0);
        }
        if (tid < kSteBN) {
            const int krow = min(k0 + tid, K - 1);
            rb = *reinterpret_cast<const uint2*>(qT + (size_t)krow * RBT + n0 / 4);
        }
    };
    auto store = [&](int buf) {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int c = tid + kSteThreads * i;
            *reinterpret_cast<uint4*>(&As[buf][(c / 4) * kSteARow + 16 * (c % 4)]) = ra[i];
        }
        if (tid < kSteBN) *reinterpret_cast<uint2*>(&Bs[buf][tid * kSteBRow]) = rb;
    };

    f32x16 acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

    const int fr = lane % 32, fg = lane / 32;
    load(0);
    store(0);
    __syncthreads();
    for (int st = 0; st < steps; ++st) {
        const int buf = st & 1;
        if (st + 1 < steps) load(st + 1);
#pragma unroll
        for (int s = 0; s < kSteBR / 16; ++s) {
            // A: dy row, reduction n = 16s + 8*fg .. +8 (16 bytes).
            bf16x8 a[2], b[2];
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const int r = wm0 + 32 * i + fr;
                const uint4 v = *reinterpret_cast<const uint4*>(
                    &As[buf][r * kSteARow + 32 * s + 16 * fg]);
                a[i] = __builtin_bit_cast(bf16x8, v);
            }
            // B: qT row k, the same 8 n as two code bytes -> 8 bf16.
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const int kr = wn0 + 32 * j + fr;
                const uint32_t two = *reinterpret_cast<const uint16_t*>(
                    &Bs[buf][kr * kSteBRow + 4 * s + 2 * fg]);
                const uint2 e0 = lut[two & 0xFFu], e1 = lut[two >> 8];
                b[j] = __builtin_bit_cast(bf16x8, make_uint4(e0.x, e0.y, e1.x, e1.y));
            }
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0,
                                                                        0, 0);
        }
        if (st + 1 < steps) {
            store(buf ^ 1);
        }
        __syncthreads();
    }

    // C layout of the 32x32 MFMA: lane l, register v holds row
    // 8*(v/4) + 4*(l/32) + v%4 (token) and column l%32 (input feature).
    const float g = *gamma_p;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            const int m = m0 + wm0 + 32 * i + 8 * (v / 4) + 4 * (lane / 32) + (v % 4);
            if (m < M) {
#pragma unroll
                for (int j = 0; j < 2; ++j) {
                    const int k = k0 + wn0 + 32 * j + (lane % 32);
                    if (k < K) dx[(size_t)m * K + k] = acc[i][j][v] * g;
                }
            }
        }
}

hipError_t launch_pack_ste_t(const uint32_t* packed2, int64_t N, int64_t K, uint8_t* qT,
                             hipStream_t stream) {
    const int64_t rb = ste_t_row_bytes(N);
    const int64_t total = K * rb;
    hipLaunchKernelGGL(k_pack_ste_t, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, stream,
                       packed2, N, K, rb, qT);
    return hipGetLastError();
}

hipError_t launch_ste_dx(const uint16_t* dy, int M, int N, const uint8_t* qT, const float* gamma,
                         int K, float* dx, hipStream_t stream) {
    const int tiles = ((M + kSteBM - 1) / kSteBM) * ((K + kSteBN - 1) / kSteBN);
    hipLaunchKernelGGL(k_ste_dx, dim3(tiles), dim3(kSteThreads), 0, stream, dy, M, N, qT,
                       (int)ste_t_row_bytes(N), gamma, K, dx);
    return hipGetLastError();
}

}  // namespace bl
