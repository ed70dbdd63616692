// Straight-through backward of BitLinear with respect to its latent weights.
//
// Source: juhe.plus (Habr repost), the section on training that follows
// BinaryConnect: the forward pass rounds and the backward pass lets the
// gradient through as if there were no rounding, so the latent full-precision
// weights receive the gradient of an ordinary linear layer; comrad404.com,
// "BitNet b1.58: что показала работа Microsoft об «эре 1-битных LLM»",
// section «Метод: как устроен BitNet b1.58»: gradients stay in high
// precision. The forward multiplies the dequantised activations
// x~ = x_q * s_x, so
//     dW[n][k] = sum_m dy[m][n] * x_q[m][k] * s_x[m]
// with dy in bf16 and dW in fp32.
//
// The per-token scale sits inside the sum over tokens, so it cannot be
// applied after the product. Each p = dy[m][n] * s_x[m] is formed in fp32
// and split exactly into two bf16 numbers: hi = p with its low 16 bits
// cleared, lo = p - hi rounded to bf16 (|hi + lo - p| < 2^-16 |p|). x_q is
// exact in bf16. The contraction then runs over 2 * Mp values (hi block, lo
// block; Mp = M rounded up to 64, zero past M) on the bf16 matrix cores,
// where every product is exact and the sums accumulate in fp32:
//     |dW - exact| <= (2^-16 + 2^-24 + 2 Mp 2^-24) * sum_m |dy s_x x_q|.
//
// Both operands are needed with the token index contiguous, so two prep
// kernels transpose them through LDS tiles: A = [hi | lo] as bf16 [N][2 Mp]
// and B = x_q as bf16 [K][Mp] (read at column j mod Mp). The GEMM mirrors the
// forward one: C tile (rows n, columns k), v_mfma_f32_32x32x16_bf16, a
// STAGES-deep LDS ring filled with global_load_lds_dwordx4, XOR-swizzled rows.
//
// Roofline: MFMA (bf16). Algorithmic work per call = 2*M*N*K flops (the
// matrix cores run twice that, the hi and the lo halves).
#include <type_traits>

#include "common.hpp"
#include "launch.hpp"

namespace bl {

namespace {

typedef __bf16 bf16x8_dw __attribute__((ext_vector_type(8)));
typedef float f32x16_dw __attribute__((ext_vector_type(16)));

constexpr int kDwPad = 64;  // token padding of the contraction

}  // namespace

int64_t ste_dw_padded_tokens(int64_t M) { return (M + kDwPad - 1) / kDwPad * kDwPad; }

// A[n][j] for a 64 x 64 (token x feature) tile of dy: hi at j = m, lo at
// j = Mp + m. Loads 16 bytes (8 features) per thread along n, stores 16
// bytes (8 tokens) per thread along m. N % 8 == 0.
__global__ __launch_bounds__(256) void k_dw_prep_a(const uint16_t* __restrict__ dy,
                                                   const float* __restrict__ xs, int M, int N,
                                                   int Mp, uint16_t* __restrict__ A) {
    __shared__ uint16_t hi_t[64][64 + 8], lo_t[64][64 + 8];
    const int m0 = blockIdx.y * 64, n0 = blockIdx.x * 64;
    const int tid = threadIdx.x;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int c = tid + 256 * i;           // 512 chunks: 64 rows x 8
        const int r = c / 8, ch = c % 8;
        const int m = m0 + r, n = n0 + 8 * ch;
        uint4 v = make_uint4(0, 0, 0, 0);
        float s = 0.0f;
        if (m < M && n < N) {
            v = *reinterpret_cast<const uint4*>(dy + (size_t)m * N + n);
            s = xs[m];
        }
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float p = bf16_to_f32((w[e / 2] >> (16 * (e % 2))) & 0xFFFFu) * s;
            const uint32_t hb = __float_as_uint(p) >> 16;       // truncated: exact high part
            const float rem = p - __uint_as_float(hb << 16);    // exact
            hi_t[r][8 * ch + e] = (uint16_t)hb;
            lo_t[r][8 * ch + e] = (uint16_t)f32_to_bf16_rne(rem);
        }
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int c = tid + 256 * i;           // 512 chunks: 64 features x 8
        const int nl = c / 8, ch = c % 8;
        const int n = n0 + nl;
        if (n >= N) continue;
        uint32_t h[4], l[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            h[e] = hi_t[8 * ch + 2 * e][nl] | ((uint32_t)hi_t[8 * ch + 2 * e + 1][nl] << 16);
            l[e] = lo_t[8 * ch + 2 * e][nl] | ((uint32_t)lo_t[8 * ch + 2 * e + 1][nl] << 16);
        }
        uint16_t* row = A + (size_t)n * (2 * (size_t)Mp) + m0 + 8 * ch;
        *reinterpret_cast<uint4*>(row) = make_uint4(h[0], h[1], h[2], h[3]);
        *reinterpret_cast<uint4*>(row + Mp) = make_uint4(l[0], l[1], l[2], l[3]);
    }
}

// B[k][m] = bf16(x_q[m][k]) (exact) for a 64 x 64 tile; zeros past M.
__global__ __launch_bounds__(256) void k_dw_prep_b(const int8_t* __restrict__ xq, int M, int K,
                                                   int Mp, uint16_t* __restrict__ B) {
    __shared__ uint16_t t[64][64 + 8];
    const int m0 = blockIdx.y * 64, k0 = blockIdx.x * 64;
    const int tid = threadIdx.x;
    {
        const int r = tid / 4, ch = tid % 4;   // 256 chunks: 64 rows x 4 x 16 codes
        const int m = m0 + r;
        uint4 v = make_uint4(0, 0, 0, 0);
        if (m < M) v = *reinterpret_cast<const uint4*>(xq + (size_t)m * K + k0 + 16 * ch);
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            const float f = (float)(int8_t)((w[e / 4] >> (8 * (e % 4))) & 0xFFu);
            t[r][16 * ch + e] = (uint16_t)(__float_as_uint(f) >> 16);   // exact in bf16
        }
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int c = tid + 256 * i;           // 512 chunks: 64 features x 8
        const int kl = c / 8, ch = c % 8;
        uint32_t h[4];
#pragma unroll
        for (int e = 0; e < 4; ++e)
            h[e] = t[8 * ch + 2 * e][kl] | ((uint32_t)t[8 * ch + 2 * e + 1][kl] << 16);
        *reinterpret_cast<uint4*>(B + (size_t)(k0 + kl) * Mp + m0 + 8 * ch) =
            make_uint4(h[0], h[1], h[2], h[3]);
    }
}

// Physical 16-byte chunk of logical chunk c in an LDS row of CH chunks, so
// that the 8 lanes of one fragment-read pass (8 consecutive rows) hit 8
// distinct 16-byte bank groups.
template <int CH>
__device__ __forceinline__ int dw_swz(int r) {
    if constexpr (CH == 4) return (r >> 1) & 3;
    else if constexpr (CH == 8) return swz_a(r);
    else return r & 15;
}

// C[n][k] = sum_{j < 2 Mp} A[n][j] * B[k][j mod Mp]: BM x BN tiles of WGM x
// WGN waves, BR contraction values per stage (2 * BR bytes per operand row).
// PART: workgroup (t, s) sums only stages [s * kt_per, (s + 1) * kt_per) of
// tile t and stores that partial tile to part + s * N * K (layout of dW).
template <int BM, int BN, int WGM, int WGN, int BR, int STAGES, int WPE, bool PART = false>
__global__ __launch_bounds__(64 * WGM * WGN, WPE) void k_ste_dw(
    const uint16_t* __restrict__ A, const uint16_t* __restrict__ B, int N, int K, int Mp,
    float* __restrict__ dW, int kt_per, float* __restrict__ part) {
    constexpr int NW = WGM * WGN;
    constexpr int WM = BM / WGM, WN = BN / WGN;
    constexpr int TM = WM / 32, TN = WN / 32;
    constexpr int ROW = 2 * BR, CH = ROW / 16;     // bytes / chunks per row per stage
    constexpr int SUB = BR / 16;                    // MFMA substeps per stage
    constexpr int A_STAGE = BM * ROW, STAGE = (BM + BN) * ROW;
    constexpr int RPI = 64 / CH;                    // rows per DMA instruction
    constexpr int A_INSTR = BM / NW / RPI, B_INSTR = BN / NW / RPI;
    constexpr int LOADS = A_INSTR + B_INSTR;
    static_assert(CH == 4 || CH == 8 || CH == 16, "stage width");
    static_assert(TM >= 1 && TN >= 1 && A_INSTR >= 1 && B_INSTR >= 1, "tile shape");
    static_assert((BM / NW) % RPI == 0 && (BN / NW) % RPI == 0, "tile shape");
    static_assert(STAGES >= 3 && LOADS * (STAGES - 1) < 64, "pipeline depth");

    extern __shared__ __align__(16) uint8_t smem[];
    const int tid = threadIdx.x;
    const int lane = tid % kWave;
    const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int wm0 = (wave % WGM) * WM, wn0 = (wave / WGM) * WN;

    // Tile order: a contiguous range of tiles per XCD, walked in groups of 8
    // row tiles (as the forward GEMM).
    const int nM = (N + BM - 1) / BM, nN = (K + BN - 1) / BN;
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
    const int n0 = bm * BM, k0 = bn * BN;

    // Stages; Mp % BR == 0, so none straddles the halves.
    const int kt0 = PART ? (int)blockIdx.y * kt_per : 0;
    const int NK = PART ? min(kt_per, 2 * Mp / BR - kt0) : 2 * Mp / BR;

    // Lane l of a DMA instruction fills physical chunk l % CH of row l / CH,
    // so it loads the logical chunk the swizzle maps there. Rows past N or
    // K are clamped (their results are not stored).
    const uint16_t* a_src[A_INSTR];
#pragma unroll
    for (int i = 0; i < A_INSTR; ++i) {
        const int r = wave * (BM / NW) + RPI * i + lane / CH;
        const int c = (lane % CH) ^ dw_swz<CH>(r);
        a_src[i] = A + (size_t)min(n0 + r, N - 1) * (2 * (size_t)Mp) + 8 * c;
    }
    const uint16_t* b_src[B_INSTR];
#pragma unroll
    for (int i = 0; i < B_INSTR; ++i) {
        const int r = wave * (BN / NW) + RPI * i + lane / CH;
        const int c = (lane % CH) ^ dw_swz<CH>(r);
        b_src[i] = B + (size_t)min(k0 + r, K - 1) * Mp + 8 * c;
    }
    const uint32_t smem_base = (uint32_t)(size_t)(lds_u8_t*)smem;
    auto issue = [&](int kt) {
        const uint32_t st = smem_base + (uint32_t)((kt % STAGES) * STAGE);
        const int ja = (kt0 + kt) * BR, jb = ja < Mp ? ja : ja - Mp;
#pragma unroll
        for (int i = 0; i < A_INSTR; ++i)
            lds_dma16(a_src[i] + ja, st + (wave * (BM / NW) + RPI * i) * ROW);
#pragma unroll
        for (int i = 0; i < B_INSTR; ++i)
            lds_dma16(b_src[i] + jb, st + A_STAGE + (wave * (BN / NW) + RPI * i) * ROW);
    };

    f32x16_dw acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

    const int fr = lane % 32, fg = lane / 32;
    // Fragments of substep s: row r, contraction 16s + 8g .. +8 = logical
    // chunk 2s + g.
    auto read_frags = [&](bf16x8_dw* f, int kt, int s, int base, int r0, auto tiles) {
        const uint8_t* S = smem + (kt % STAGES) * STAGE + base;
#pragma unroll
        for (int i = 0; i < decltype(tiles)::value; ++i) {
            const int r = r0 + 32 * i + fr;
            f[i] = *reinterpret_cast<const bf16x8_dw*>(S + r * ROW +
                                                       16 * ((2 * s + fg) ^ dw_swz<CH>(r)));
        }
    };
    using TMc = std::integral_constant<int, TM>;
    using TNc = std::integral_constant<int, TN>;

#pragma unroll
    for (int st = 0; st < STAGES - 1; ++st)
        if (st < NK) issue(st);
    {
        wait_stages<LOADS, STAGES - 2>(min(STAGES - 2, NK - 1));
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
    }
    bf16x8_dw af[TM], an[TM], bf[TN], bfn[TN];
    read_frags(af, 0, 0, 0, wm0, TMc());
    read_frags(bf, 0, 0, A_STAGE, wn0, TNc());

    // One K step; in the steady state (the STAGES - 1 steps after kt exist)
    // every bound is a constant, so that body carries no compare-and-branch
    // chains. Both bodies do the same loads, waits and MFMAs in the same order.
    auto step = [&](auto steady_c, int kt) {
        constexpr bool STEADY = decltype(steady_c)::value;
        const bool more = STEADY || kt + 1 < NK;
#pragma unroll
        for (int s = 0; s < SUB; ++s) {
            // The next substep's fragments (this stage, or the first of the
            // next once it is visible) are read ahead of this one's MFMAs.
            if (s == SUB - 1 && more) {
                // Stage kt+1 landed once only the stages issued after it are
                // outstanding; the barrier also proves every wave is done
                // with stage kt-1, whose buffer is refilled now.
                wait_stages<LOADS, STAGES - 3>(STEADY ? STAGES - 3 : min(STAGES - 3, NK - 2 - kt));
                __builtin_amdgcn_s_barrier();
                asm volatile("" ::: "memory");
                if (STEADY || kt + STAGES - 1 < NK) issue(kt + STAGES - 1);
            }
            if (s < SUB - 1) {
                read_frags(an, kt, s + 1, 0, wm0, TMc());
                read_frags(bfn, kt, s + 1, A_STAGE, wn0, TNc());
            } else if (more) {
                read_frags(an, kt + 1, 0, 0, wm0, TMc());
                read_frags(bfn, kt + 1, 0, A_STAGE, wn0, TNc());
            }
#pragma unroll
            for (int i = 0; i < TM; ++i)
#pragma unroll
                for (int j = 0; j < TN; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bf[j], acc[i][j],
                                                                        0, 0, 0);
#pragma unroll
            for (int i = 0; i < TM; ++i) af[i] = an[i];
#pragma unroll
            for (int j = 0; j < TN; ++j) bf[j] = bfn[j];
            __builtin_amdgcn_sched_barrier(0);
        }
    };
    int kt = 0;
    for (; kt < NK - (STAGES - 1); ++kt) step(std::true_type(), kt);
    for (; kt < NK; ++kt) step(std::false_type(), kt);

    // C layout of the 32x32 MFMA: lane l, register v holds row
    // 8*(v/4) + 4*(l/32) + v%4 (output feature n) and column l%32 (input
    // feature k).
#pragma unroll
    for (int i = 0; i < TM; ++i) {
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            const int n = n0 + wm0 + 32 * i + 8 * (v / 4) + 4 * (lane / 32) + (v % 4);
            if (n < N) {
#pragma unroll
                for (int j = 0; j < TN; ++j) {
                    const int k = k0 + wn0 + 32 * j + (lane % 32);
                    if (k >= K) continue;
                    // Partial tiles are read back at once by k_dw_reduce.
                    if constexpr (PART)
                        part[(size_t)blockIdx.y * N * K + (size_t)n * K + k] = acc[i][j][v];
                    else
                        __builtin_nontemporal_store(acc[i][j][v], dW + (size_t)n * K + k);
                }
            }
            __builtin_amdgcn_sched_barrier(0);
        }
    }
}

// dW[rows][K] = sum over s < S of part[s][rows][K], added in order of s.
__global__ __launch_bounds__(256) void k_dw_reduce(const float* __restrict__ part, int S,
                                                   size_t count, float* __restrict__ dW) {
    typedef float f4 __attribute__((ext_vector_type(4)));
    const size_t stride = (size_t)gridDim.x * 256;
    for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < count / 4; i += stride) {
        f4 a = reinterpret_cast<const f4*>(part)[i];
        for (int s = 1; s < S; ++s) {
            const f4 b = reinterpret_cast<const f4*>(part + (size_t)s * count)[i];
            a.x += b.x;
            a.y += b.y;
            a.z += b.z;
            a.w += b.w;
        }
        __builtin_nontemporal_store(a, reinterpret_cast<f4*>(dW) + i);
    }
}

namespace {

constexpr int kDwCUs = 256, kDwBM = 128, kDwBN = 256, kDwBR = 64;

// The last round of 128 x 256 tiles, when at most half full, is not run as
// such. Its row tiles (rows) either split their 2 Mp / 64 stages over
// `splits` workgroups each (at least 8 stages per split, the grid at most one
// round), their partial tiles kept in the workspace and added in a third
// launch; or, where fewer than two splits would result, run as 64 x 64 tiles.
struct DwPlan {
    int rows = 0;    // rows of the tail (0: one launch covers dW)
    int splits = 1;  // > 1: split tail, else 64 x 64 tail
    int per = 0;     // stages per split
};

DwPlan dw_plan(int64_t N, int64_t K, int64_t Mp) {
    DwPlan p;
    const int64_t nM = (N + kDwBM - 1) / kDwBM, nN = (K + kDwBN - 1) / kDwBN;
    const int64_t tiles = nM * nN, tail = tiles % kDwCUs;
    const int64_t rem = (tail + nN - 1) / nN;
    if (!(tiles > kDwCUs && tail > 0 && 2 * tail <= kDwCUs && rem < nM)) return p;
    p.rows = (int)(rem * kDwBM);
    const int64_t NK = 2 * Mp / kDwBR;
    const int64_t s = std::min<int64_t>(kDwCUs / (rem * nN), NK / 8);
    if (s >= 2) {
        p.per = (int)((NK + s - 1) / s);
        p.splits = (int)((NK + p.per - 1) / p.per);
    }
    return p;
}

}  // namespace

size_t ste_dw_workspace_bytes(int64_t M, int64_t N, int64_t K) {
    const int64_t Mp = ste_dw_padded_tokens(M);
    const DwPlan p = dw_plan(N, K, Mp);
    const int64_t part = p.splits > 1 ? (int64_t)p.splits * p.rows * K * 4 : 0;
    // bf16 A [N][2 Mp] and B [K][Mp], then the split tail's fp32 partial tiles.
    return (size_t)(2 * N * 2 * Mp + 2 * K * Mp + part);
}

template <int BM, int BN, int WGM, int WGN, int BR, int STAGES, int WPE, bool PART = false>
static hipError_t launch_dw_tile(const uint16_t* A, const uint16_t* B, int N, int K, int Mp,
                                 float* dW, hipStream_t stream, int splits = 1, int per = 0,
                                 float* part = nullptr) {
    constexpr size_t lds = (size_t)STAGES * (BM + BN) * 2 * BR;
    static_assert(lds <= 160 * 1024, "a workgroup holds at most 160 KiB of LDS");
    auto kern = &k_ste_dw<BM, BN, WGM, WGN, BR, STAGES, WPE, PART>;
    static std::atomic<uint64_t> lds_set{0};
    {
        hipError_t e = allow_dynamic_lds(reinterpret_cast<const void*>(kern), lds, lds_set);
        if (e != hipSuccess) return e;
    }
    const int tiles = ((N + BM - 1) / BM) * ((K + BN - 1) / BN);
    hipLaunchKernelGGL(kern, dim3(tiles, PART ? splits : 1), dim3(64 * WGM * WGN), lds, stream, A,
                       B, N, K, Mp, dW, per, part);
    return hipGetLastError();
}

hipError_t launch_ste_dw(const uint16_t* dy, int M, int N, const int8_t* xq, const float* xs,
                         int K, float* dW, void* workspace, hipStream_t stream) {
    const int Mp = (int)ste_dw_padded_tokens(M);
    uint16_t* A = static_cast<uint16_t*>(workspace);
    uint16_t* B = A + (size_t)N * 2 * Mp;
    hipLaunchKernelGGL(k_dw_prep_a, dim3((N + 63) / 64, Mp / 64), dim3(256), 0, stream, dy, xs,
                       M, N, Mp, A);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k_dw_prep_b, dim3(K / 64, Mp / 64), dim3(256), 0, stream, xq, M, K, Mp, B);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    // 128 x 256 tiles of 8 waves of 64 x 64 (two per SIMD): 8-9% faster on
    // the 4096-token projections than 4 waves of 128 x 64 (one per SIMD, whose
    // LDS and barrier latencies stall its matrix core), and than 8 waves of
    // 128 x 64 on 128 x 512 or 256 x 256 tiles (32-wide stages to fit the LDS,
    // twice the barriers) or 16 waves of 64 x 64.
    //
    // One such tile per CU (144 KB of LDS): when the last round of tiles is
    // at most half full, the last row tiles (dw_plan) leave the first launch
    // so that no round runs on a few CUs. With enough stages they stay
    // 128 x 256 tiles whose stages are split over several workgroups each
    // (the grid at most one round); each split stores its fp32 partial tile
    // in the workspace and k_dw_reduce adds the partials in split order, so
    // the result is the same from call to call, and each output is the sum
    // of the same products, grouped by split. The 4096-token projections
    // have 540 tiles (two rounds and 28): their last 3 and 2 row tiles take
    // 8 and 4 splits of 16 and 32 stages. Otherwise the tail runs as 64 x 64
    // tiles (48 KB, several per CU), in the same stage order as the first
    // launch (same bits): 383 -> 328 us on 6912 x 2560 and 366 -> 312 us on
    // 2560 x 6912 against one launch (a remainder of 64 x 128 tiles: 339 /
    // 321; of 128 x 128: 345 / 335).
    static_assert(kDwBM == 128 && kDwBN == 256 && kDwBR == 64, "tile of the plan");
    const DwPlan plan = dw_plan(N, K, Mp);
    if (plan.rows > 0) {
        const int n1 = ((N + kDwBM - 1) / kDwBM - plan.rows / kDwBM) * kDwBM;  // first tail row
        const int nt = N - n1;
        e = launch_dw_tile<128, 256, 2, 4, 64, 3, 2>(A, B, n1, K, Mp, dW, stream);
        if (e != hipSuccess) return e;
        const uint16_t* At = A + (size_t)n1 * 2 * Mp;
        float* dWt = dW + (size_t)n1 * K;
        if (plan.splits < 2)
            return launch_dw_tile<64, 64, 2, 2, 64, 3, 4>(At, B, nt, K, Mp, dWt, stream);
        float* part = reinterpret_cast<float*>(B + (size_t)K * Mp);
        e = launch_dw_tile<128, 256, 2, 4, 64, 3, 2, true>(At, B, nt, K, Mp, dWt, stream,
                                                           plan.splits, plan.per, part);
        if (e != hipSuccess) return e;
        const size_t count = (size_t)nt * K;
        const int blocks = (int)std::min<size_t>((count / 4 + 255) / 256, 2048);
        hipLaunchKernelGGL(k_dw_reduce, dim3(blocks), dim3(256), 0, stream, part, plan.splits,
                           count, dWt);
        return hipGetLastError();
    }
    return launch_dw_tile<128, 256, 2, 4, 64, 3, 2>(A, B, N, K, Mp, dW, stream);
}

}  // namespace bl
