// Decode BitLinear for one token: the packed weights streamed as 1 KB pieces.
//
// Source: inferownia.pl, "BitNet b1.58: era 1-bitowych LLM-ów", section
// "Mnożenie? Jakie mnożenie", and juhe.plus (Habr repost), section «Когда - три
// лучше двух»: with weights in {-1, 0, +1} the product is the sum of the inputs
// whose weight is +1 minus the sum of those whose weight is -1; zero weights
// add nothing. At one token the call reads every packed weight once and does
// little arithmetic per byte, so its bound is HBM bandwidth.
//
// Each wave owns RW whole rows (output features) and streams them in order:
// one load instruction per 1 KB piece of a row (16 bytes per lane, 64 lanes
// over contiguous memory; the last piece of a row may be partial). A 16-byte
// load that spreads over 16 rows x 64 bytes, the MFMA operand shape of the
// multi-token GEMV, measured 7-8% slower than contiguous loads of the same
// bytes here.
//
// Arithmetic: the stored codes are c = q + 1 in {0, 1, 2}, four consecutive
// weights per byte position (bit pair p of byte b holds weight 4p + b of its
// 16-weight word). Masking a word in place, without shifting the fields down,
// gives four dwords of byte operands:
//   w & 0x03030303          =      c of weights 0..3
//   w & 0x0C0C0C0C          =  4 * c of weights 4..7
//   w & 0x30303030          = 16 * c of weights 8..11
//   (w >> 2) & 0x30303030   = 16 * c of weights 12..15
// (every byte below 128, so signed bytes read them correctly). v_dot4 of each
// with the four matching activation bytes accumulates 1x, 4x and 16x sums; the
// latter two are exact multiples of 4 and 16, so shifting them right is exact
// division. Their total is sum_k c_k x_k = sum_k q_k x_k + sum_k x_k, and the
// activation sum is subtracted once per row. Five VALU operations expand 16
// weights (the sign-select permute of the multi-token kernels takes nine).
//
// Activations: one token of K int8 values, staged in LDS so that lane l's 64
// bytes for piece j lie at (4j + s) * 1024 + 16 l, s = 0..3 (conflict-free
// 16-byte reads; zeros past K). Two variants:
//   k_gemv1_cached  K <= 4096 * S (S = 1 or 2 pieces per row): the block is
//                   loaded by direct global-to-LDS transfers and each lane
//                   keeps its 64 * S bytes in registers; every wave sums its
//                   own lanes' bytes (no extra barrier);
//   k_gemv1_stream  longer rows (one row per wave): the block goes through
//                   registers, summed on the way, one barrier; each piece
//                   reads its activations from LDS.
// Waves are independent after the staging barrier (no barrier at the end).
//
// Roofline: HBM. Algorithmic bytes per call = N * K/4 (packed weights) + K
// (activations) + 4 (scale) + 4 (gamma) + 4 * N (y).
#include "common.hpp"
#include "launch.hpp"

namespace bl {

namespace {

constexpr int kPiece = 1024;                        // packed bytes per piece
constexpr int kPieceK = 4 * kPiece;                 // weights per piece
constexpr int kStreamMaxK = 16 * kPieceK;           // 64 KiB of staged activations
constexpr uint32_t kZeroCodes = 0x55555555u;        // sixteen weights of 0

// Sum over one 16-byte piece of (masked codes) x (activations), exact.
__device__ __forceinline__ int piece_dot(const uint4 wv, const uint4 (&a)[4]) {
    const uint32_t w[4] = {wv.x, wv.y, wv.z, wv.w};
    int v0 = 0, v1 = 0, v2 = 0;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
        v0 = __builtin_amdgcn_sdot4((int)(w[s] & 0x03030303u), (int)a[s].x, v0, false);
        v1 = __builtin_amdgcn_sdot4((int)(w[s] & 0x0C0C0C0Cu), (int)a[s].y, v1, false);
        v2 = __builtin_amdgcn_sdot4((int)(w[s] & 0x30303030u), (int)a[s].z, v2, false);
        v2 = __builtin_amdgcn_sdot4((int)((w[s] >> 2) & 0x30303030u), (int)a[s].w, v2, false);
    }
    return v0 + (v1 >> 2) + (v2 >> 4);
}

__device__ __forceinline__ int bytes_sum(const uint4 a, int s) {
    s = __builtin_amdgcn_sdot4((int)a.x, 0x01010101, s, false);
    s = __builtin_amdgcn_sdot4((int)a.y, 0x01010101, s, false);
    s = __builtin_amdgcn_sdot4((int)a.z, 0x01010101, s, false);
    return __builtin_amdgcn_sdot4((int)a.w, 0x01010101, s, false);
}

__device__ __forceinline__ void store_row(float* y, int32_t* acc_out, int n, int a, float sc) {
    y[n] = (float)a * sc;
    if (acc_out) acc_out[n] = a;
}

}  // namespace

// S pieces per row (K <= 4096 S), RW rows per wave, R loads in flight per lane,
// WPB waves per workgroup. Requires N >= RW.
template <int S, int RW, int R, int WPB>
__global__ __launch_bounds__(64 * WPB) void k_gemv1_cached(
    const int8_t* __restrict__ xq, const float* __restrict__ xs, int K,
    const uint8_t* __restrict__ W, const float* __restrict__ gamma_p, int N, float* __restrict__ y,
    int32_t* __restrict__ acc_out) {
    constexpr int L = S * RW;  // pieces per wave
    __shared__ __align__(16) uint8_t smem[S * kPieceK];
    const int tid = threadIdx.x, lane = tid % kWave;
    const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int RB = K / 4;

    // 1. Activations straight into LDS: transfer q = 4j + s moves, for each
    //    lane l, x[4096 j + 64 l + 16 s, +16) to q * 1024 + 16 l; lanes past
    //    K store zeros instead.
    const uint32_t xbase = lds_offset(smem);
    for (int q = wave; q < 4 * S; q += WPB) {
        const int k0 = kPieceK * (q / 4) + 64 * lane;
        if (k0 < K)
            lds_dma16(xq + k0 + 16 * (q % 4), xbase + q * kPiece);
        else
            *reinterpret_cast<uint4*>(smem + q * kPiece + 16 * lane) = make_uint4(0, 0, 0, 0);
    }
    asm volatile("" ::: "memory");

    // 2. The wave's rows nb .. nb+RW-1 (the last wave of the grid shifts back
    //    to stay inside N and stores only rows from n0 on).
    const int n0 = (blockIdx.x * WPB + wave) * RW;
    const int nb = min(n0, N - RW);
    const uint8_t* wrow = W + (size_t)nb * RB + 16 * lane;
    auto load = [&](int i) -> uint4 {
        const int r = i / S, j = i % S;
        return kPiece * j + 16 * lane < RB
                   ? *reinterpret_cast<const uint4*>(wrow + (size_t)r * RB + kPiece * j)
                   : make_uint4(kZeroCodes, kZeroCodes, kZeroCodes, kZeroCodes);
    };
    uint4 wb[R];
#pragma unroll
    for (int u = 0; u < R; ++u)
        if (u < L) wb[u] = load(u);
    asm volatile("" ::: "memory");

    // 3. This wave's transfers landed (the weight loads, issued after them,
    //    may still be in flight); then every wave's are visible.
    wait_vmcnt_le8(L < R ? L : R);
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __syncthreads();

    uint4 act[S][4];
    int sx = 0;
#pragma unroll
    for (int j = 0; j < S; ++j)
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            act[j][s] = *reinterpret_cast<const uint4*>(smem + (4 * j + s) * kPiece + 16 * lane);
            sx = bytes_sum(act[j][s], sx);
        }

    int acc[RW];
#pragma unroll
    for (int r = 0; r < RW; ++r) acc[r] = 0;
#pragma unroll
    for (int i = 0; i < L; ++i) {
        const int u = i % R;
        acc[i / S] += piece_dot(wb[u], act[i % S]);
        if (i + R < L) wb[u] = load(i + R);
    }

    const float sc = xs[0] * (*gamma_p);
#pragma unroll
    for (int r = 0; r < RW; ++r) {
        // Each lane subtracts its own share of sum x, so one reduction gives
        // sum q x.
        const int a = wave_sum_i32(acc[r] - sx);
        const int n = nb + r;
        if (lane == r && n >= n0) store_row(y, acc_out, n, a, sc);
    }
}

// One row per wave, R loads in flight per lane. SP > 0: exactly SP whole
// pieces per row (K = 4096 SP), every bound known at compile time; SP = 0:
// any K up to kStreamMaxK, the last piece possibly partial.
template <int SP, int R, int WPB>
__global__ __launch_bounds__(64 * WPB) void k_gemv1_stream(
    const int8_t* __restrict__ xq, const float* __restrict__ xs, int K_arg,
    const uint8_t* __restrict__ W, const float* __restrict__ gamma_p, int N, float* __restrict__ y,
    int32_t* __restrict__ acc_out) {
    constexpr int NT = 64 * WPB;
    constexpr int XPT = SP > 0 ? (SP * (kPieceK / 16) + NT - 1) / NT : 4;  // slots per thread
    extern __shared__ __align__(16) uint8_t smem[];
    __shared__ int wsum[WPB];
    const int tid = threadIdx.x, lane = tid % kWave;
    const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int K = SP > 0 ? SP * kPieceK : K_arg;
    const int RB = K / 4;
    const int NP = SP > 0 ? SP : (RB + kPiece - 1) / kPiece;  // pieces per row
    const int XP = NP * (kPieceK / 16);  // 16-byte activation slots, zero past K

    // 1. This thread's activation slots t = tid + NT i: x[16 t, +16) lands at
    //    (4j + s) * 1024 + 16 l with t = 256 j + 4 l + s.
    uint4 xv[XPT];
#pragma unroll
    for (int i = 0; i < XPT; ++i) {
        const int t = tid + NT * i;
        xv[i] = 16 * t < K ? *reinterpret_cast<const uint4*>(xq + 16 * t) : make_uint4(0, 0, 0, 0);
    }
    asm volatile("" ::: "memory");

    // 2. The wave's row (the grid's last waves repeat row N-1 and store nothing).
    const int n0 = blockIdx.x * WPB + wave;
    const int n = min(n0, N - 1);
    const uint8_t* wrow = W + (size_t)n * RB + 16 * lane;
    auto load = [&](int j) -> uint4 {
        if (SP > 0) return *reinterpret_cast<const uint4*>(wrow + kPiece * j);
        return kPiece * j + 16 * lane < RB
                   ? *reinterpret_cast<const uint4*>(wrow + kPiece * j)
                   : make_uint4(kZeroCodes, kZeroCodes, kZeroCodes, kZeroCodes);
    };
    uint4 wb[R];
#pragma unroll
    for (int u = 0; u < R; ++u)
        if (u < NP) wb[u] = load(u);
    asm volatile("" ::: "memory");

    // 3. Only the weight loads may remain in flight; store the slots and sum them.
    wait_vmcnt_le8(NP < R ? NP : R);
    auto slot = [&](int t) { return smem + (4 * (t / 256) + t % 4) * kPiece + 16 * ((t / 4) % 64); };
    int s = 0;
#pragma unroll
    for (int i = 0; i < XPT; ++i) {
        const int t = tid + NT * i;
        if (t < XP) {
            *reinterpret_cast<uint4*>(slot(t)) = xv[i];
            s = bytes_sum(xv[i], s);
        }
    }
    for (int t = tid + NT * XPT; SP == 0 && t < XP; t += NT) {  // more slots than XPT per thread
        const uint4 v =
            16 * t < K ? *reinterpret_cast<const uint4*>(xq + 16 * t) : make_uint4(0, 0, 0, 0);
        *reinterpret_cast<uint4*>(slot(t)) = v;
        s = bytes_sum(v, s);
    }
    s = wave_sum_i32(s);
    if (lane == 0) wsum[wave] = s;
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __syncthreads();
    int sx = 0;
#pragma unroll
    for (int w = 0; w < WPB; ++w) sx += wsum[w];

    // 4. Ring of R pieces: consume piece j, then refill its slot with j + R.
    int acc = 0;
    for (int b0 = 0; b0 < NP; b0 += R) {
#pragma unroll
        for (int u = 0; u < R; ++u) {
            const int j = b0 + u;
            if (j < NP) {
                uint4 a[4];
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    a[q] = *reinterpret_cast<const uint4*>(smem + (4 * j + q) * kPiece + 16 * lane);
                acc += piece_dot(wb[u], a);
                if (j + R < NP) wb[u] = load(j + R);
            }
        }
    }
    const int a = wave_sum_i32(acc) - sx;
    if (lane == 0 && n == n0) store_row(y, acc_out, n, a, xs[0] * (*gamma_p));
}

template <int S, int RW, int R, int WPB>
static hipError_t launch_cached(const int8_t* xq, const float* xs, int K, const uint32_t* Wp,
                                const float* gamma, int N, float* y, int32_t* acc,
                                hipStream_t stream) {
    const int waves = (N + RW - 1) / RW;
    const int blocks = (waves + WPB - 1) / WPB;
    hipLaunchKernelGGL((k_gemv1_cached<S, RW, R, WPB>), dim3(blocks), dim3(64 * WPB), 0, stream,
                       xq, xs, K, reinterpret_cast<const uint8_t*>(Wp), gamma, N, y, acc);
    return hipGetLastError();
}

template <int SP, int R, int WPB>
static hipError_t launch_stream(const int8_t* xq, const float* xs, int K, const uint32_t* Wp,
                                const float* gamma, int N, float* y, int32_t* acc,
                                hipStream_t stream) {
    const int NP = (K / 4 + kPiece - 1) / kPiece;
    const size_t lds = (size_t)NP * kPieceK;
    const int blocks = (N + WPB - 1) / WPB;
    hipLaunchKernelGGL((k_gemv1_stream<SP, R, WPB>), dim3(blocks), dim3(64 * WPB), lds, stream,
                       xq, xs, K, reinterpret_cast<const uint8_t*>(Wp), gamma, N, y, acc);
    return hipGetLastError();
}

bool gemv1_supported(int64_t M, int64_t K) { return M == 1 && K <= kStreamMaxK; }

// The automatic choice at one token: every shape except rows longer than two
// pieces that end in a partial one (8640 -> 3200 and 11008 -> 4096 measured
// level with the multi-token GEMV there).
bool gemv1_preferred(int64_t M, int64_t K) {
    return gemv1_supported(M, K) && (K <= 2 * kPieceK || K % kPieceK == 0);
}

// Shapes measured on 8192 -> 28672 (two pieces per row: two rows per wave,
// two loads in flight, 4-wave workgroups) and 28672 -> 8192 (seven pieces:
// one row per wave, 8-wave workgroups).
hipError_t launch_gemv1(const int8_t* xq, const float* xs, int K, const uint32_t* Wp,
                        const float* gamma, int N, float* y, int32_t* acc, hipStream_t stream) {
    if (K > kStreamMaxK) return hipErrorInvalidValue;
    if (K <= kPieceK) {
        if (N >= 4) return launch_cached<1, 4, 4, 4>(xq, xs, K, Wp, gamma, N, y, acc, stream);
        return launch_cached<1, 1, 1, 4>(xq, xs, K, Wp, gamma, N, y, acc, stream);
    }
    if (K <= 2 * kPieceK) {
        if (N >= 2) return launch_cached<2, 2, 2, 4>(xq, xs, K, Wp, gamma, N, y, acc, stream);
        return launch_cached<2, 1, 2, 4>(xq, xs, K, Wp, gamma, N, y, acc, stream);
    }
    // Whole pieces: the piece count as a template (all of a row's loads in flight).
    switch (K % kPieceK == 0 ? K / kPieceK : 0) {
        case 3: return launch_stream<3, 3, 8>(xq, xs, K, Wp, gamma, N, y, acc, stream);
        case 4: return launch_stream<4, 4, 8>(xq, xs, K, Wp, gamma, N, y, acc, stream);
        case 5: return launch_stream<5, 5, 8>(xq, xs, K, Wp, gamma, N, y, acc, stream);
        case 6: return launch_stream<6, 6, 8>(xq, xs, K, Wp, gamma, N, y, acc, stream);
        case 7: return launch_stream<7, 7, 8>(xq, xs, K, Wp, gamma, N, y, acc, stream);
        case 8: return launch_stream<8, 8, 8>(xq, xs, K, Wp, gamma, N, y, acc, stream);
        default: return launch_stream<0, 8, 8>(xq, xs, K, Wp, gamma, N, y, acc, stream);
    }
}

}  // namespace bl
