// Prefill BitLinear (many tokens): int8 MFMA GEMM over ternary tiles expanded
// to int8 in LDS.
//
// Source: inferownia.pl, "BitNet b1.58: era 1-bitowych LLM-ów", section
// "Mnożenie? Jakie mnożenie", and juhe.plus (Habr repost), section «Когда - три
// лучше двух»: a ternary weight turns each multiply into an add, a subtract or
// nothing. At prefill the work is compute-bound (2*M*N*K int8 operations over
// 2 bits of weight and M*K bytes of activations), so the add/subtract is
// carried out by the int8 matrix cores on weights expanded to {-1, 0, +1}
// bytes: every product is exact and the int32 sums are exact.
//
// y = x_q . q^T: the MFMA A operand is the activation tile (rows = tokens), the
// B operand the weight tile (rows = output features); both are k-contiguous.
// Workgroup: 256 threads = 4 waves in a 2 x 2 grid, block tile BM x BN, K step
// 64, v_mfma_i32_32x32x32_i8. Per K step each thread loads its share of the
// activation tile (16 B chunks) and of the packed weight tile (one 16 B load =
// 64 weights of one row), expands the weights with byte permutes, and stores
// both into the idle half of a double-buffered LDS tile (16 B chunks XOR-
// swizzled by row against bank conflicts). The epilogue scales the exact int32
// sums by x_scale[m] * gamma and stores fp32 rows of 128 contiguous bytes.
//
// Roofline: MFMA (int8). Algorithmic work per call = 2*M*N*K operations.
#include "common.hpp"
#include "launch.hpp"

namespace bl {

constexpr int kGemmThreads = 256;
constexpr int kBK = 64;

// 16-byte chunk c (0..3) of LDS row r lives at chunk position c ^ swz(r).
__device__ __forceinline__ int swz(int r) { return (r >> 1) & 3; }

template <int BM, int BN>
__global__ __launch_bounds__(kGemmThreads) void k_gemm(
    const int8_t* __restrict__ xq, const float* __restrict__ xs, int M, int K,
    const uint32_t* __restrict__ Wp, const float* __restrict__ gamma_p, int N,
    float* __restrict__ y, int32_t* __restrict__ acc_out) {
    constexpr int WM = BM / 2, WN = BN / 2;
    constexpr int TM = WM / 32, TN = WN / 32;
    constexpr int A_PER = BM * 4 / kGemmThreads;  // 16 B activation chunks per thread
    static_assert(A_PER >= 1 && BN <= kGemmThreads, "tile shape");

    __shared__ __align__(16) int8_t As[2][BM * kBK];
    __shared__ __align__(16) int8_t Bs[2][BN * kBK];

    const int tid = threadIdx.x;
    const int wave = tid / kWave, lane = tid % kWave;
    const int wm0 = (wave % 2) * WM, wn0 = (wave / 2) * WN;

    // Tile order: hand each XCD (workgroups are dealt round-robin to the 8
    // XCDs) a contiguous range of tile ids, then walk tiles in groups of 8
    // row tiles so neighbouring workgroups share activation and weight tiles
    // in the XCD's L2.
    const int nM = (M + BM - 1) / BM, nN = (N + BN - 1) / BN;
    const int total = nM * nN;
    const int b = blockIdx.x;
    const int xcd = b % 8, idx = b / 8;
    const int t = xcd * (total / 8) + min(xcd, total % 8) + idx;
    constexpr int G = 8;
    const int group = t / (G * nN);
    const int first_m = group * G;
    const int gsize = min(nM - first_m, G);
    const int bm = first_m + (t % (G * nN)) % gsize;
    const int bn = (t % (G * nN)) / gsize;
    const int m0 = bm * BM, n0 = bn * BN;

    // Global -> register staging assignments.
    const int8_t* a_src[A_PER];
    int a_lds[A_PER];
#pragma unroll
    for (int i = 0; i < A_PER; ++i) {
        const int id = tid + kGemmThreads * i;
        const int r = id / 4, c = id % 4;
        const int gm = min(m0 + r, M - 1);
        a_src[i] = xq + (size_t)gm * K + 16 * c;
        a_lds[i] = r * kBK + 16 * (c ^ swz(r));
    }
    const bool b_ld = tid < BN;
    const int b_row = tid;
    const uint32_t* b_src = Wp + (size_t)min(n0 + b_row, N - 1) * (K / 16);

    uint4 a_reg[A_PER];
    uint4 b_reg = make_uint4(0, 0, 0, 0);

    auto gload = [&](int kt) {
#pragma unroll
        for (int i = 0; i < A_PER; ++i)
            a_reg[i] = *reinterpret_cast<const uint4*>(a_src[i] + (size_t)kt * kBK);
        if (b_ld) b_reg = *reinterpret_cast<const uint4*>(b_src + 4 * kt);
    };
    auto lstore = [&](int buf) {
#pragma unroll
        for (int i = 0; i < A_PER; ++i)
            *reinterpret_cast<uint4*>(&As[buf][a_lds[i]]) = a_reg[i];
        if (b_ld) {
            const uint32_t w4[4] = {b_reg.x, b_reg.y, b_reg.z, b_reg.w};
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const v4i e = expand_word(w4[c]);
                *reinterpret_cast<v4i*>(&Bs[buf][b_row * kBK + 16 * (c ^ swz(b_row))]) = e;
            }
        }
    };

    v16i acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[i][j][v] = 0;

    const int KT = K / kBK;
    gload(0);
    lstore(0);
    __syncthreads();

    const int fr = lane % 32, fg = lane / 32;
    for (int kt = 0; kt < KT; ++kt) {
        const int buf = kt & 1;
        if (kt + 1 < KT) gload(kt + 1);
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            const int c = 2 * s + fg;
            v4i af[TM], bf[TN];
#pragma unroll
            for (int i = 0; i < TM; ++i) {
                const int r = wm0 + 32 * i + fr;
                af[i] = *reinterpret_cast<const v4i*>(&As[buf][r * kBK + 16 * (c ^ swz(r))]);
            }
#pragma unroll
            for (int j = 0; j < TN; ++j) {
                const int r = wn0 + 32 * j + fr;
                bf[j] = *reinterpret_cast<const v4i*>(&Bs[buf][r * kBK + 16 * (c ^ swz(r))]);
            }
#pragma unroll
            for (int i = 0; i < TM; ++i)
#pragma unroll
                for (int j = 0; j < TN; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(af[i], bf[j], acc[i][j],
                                                                      0, 0, 0);
        }
        if (kt + 1 < KT) lstore(buf ^ 1);
        __syncthreads();
    }

    // Epilogue. C layout of the 32x32 MFMA: lane l, register v holds row
    // 8*(v/4) + 4*(l/32) + v%4 (token) and column l%32 (output feature).
    const float gm = *gamma_p;
#pragma unroll
    for (int i = 0; i < TM; ++i) {
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            const int m = m0 + wm0 + 32 * i + 8 * (v / 4) + 4 * (lane / 32) + (v % 4);
            if (m >= M) continue;
            const float sc = xs[m] * gm;
#pragma unroll
            for (int j = 0; j < TN; ++j) {
                const int n = n0 + wn0 + 32 * j + (lane % 32);
                if (n < N) {
                    y[(size_t)m * N + n] = (float)acc[i][j][v] * sc;
                    if (acc_out) acc_out[(size_t)m * N + n] = acc[i][j][v];
                }
            }
        }
    }
}

template <int BM, int BN>
static hipError_t launch_gemm_tile(const int8_t* xq, const float* xs, int M, int K,
                                   const uint32_t* Wp, const float* gamma, int N, float* y,
                                   int32_t* acc, hipStream_t stream) {
    const int blocks = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
    hipLaunchKernelGGL((k_gemm<BM, BN>), dim3(blocks), dim3(kGemmThreads), 0, stream, xq, xs, M,
                       K, Wp, gamma, N, y, acc);
    return hipGetLastError();
}

hipError_t launch_gemm(const int8_t* xq, const float* xs, int M, int K, const uint32_t* Wp,
                       const float* gamma, int N, float* y, int32_t* acc, hipStream_t stream) {
    auto tiles = [&](int bm, int bn) {
        return (int64_t)((M + bm - 1) / bm) * ((N + bn - 1) / bn);
    };
    constexpr int kCUs = 256;
    if (tiles(256, 256) >= kCUs) return launch_gemm_tile<256, 256>(xq, xs, M, K, Wp, gamma, N, y, acc, stream);
    if (tiles(256, 128) >= kCUs) return launch_gemm_tile<256, 128>(xq, xs, M, K, Wp, gamma, N, y, acc, stream);
    if (tiles(128, 128) >= kCUs) return launch_gemm_tile<128, 128>(xq, xs, M, K, Wp, gamma, N, y, acc, stream);
    return launch_gemm_tile<64, 128>(xq, xs, M, K, Wp, gamma, N, y, acc, stream);
}

}  // namespace bl
