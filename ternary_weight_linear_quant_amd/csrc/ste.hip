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
// four consecutive n per byte. The GEMM mirrors the forward one: A = dy tile
// (rows = tokens, n-contiguous), B = code tile (rows = input features k),
// v_mfma_f32_32x32x16_bf16, a STAGES-deep LDS ring filled with
// global_load_lds_dwordx4, reduction steps of 64 n (128 bytes of dy and 16
// bytes of codes per row). Products of bf16 by {-1, 0, +1} are exact; the
// sums accumulate in fp32.
//
// Codes are decoded in registers: the 16 bits of codes that feed one B
// fragment (8 n of one k) become 4 dwords of bf16 pairs with a byte
// replicate, a packed 16-bit shift, a mask and a byte permute through the
// table {0xBF, 0x00, 0x3F} (high bytes) / {0x80, 0x00, 0x80} (low bytes):
// about 3.5 VALU instructions per MFMA, which the matrix cores overlap.
//
// Roofline: MFMA (bf16). Work per call = 2*M*N*K flops.
#include "common.hpp"
#include "launch.hpp"

namespace bl {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));


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

// Source of the dy chunks past N (N % 64 != 0): sixteen zero bytes, so the
// padded products are exact zeros whatever the codes there.
__device__ __align__(16) const uint32_t kSteZero16[4] = {0u, 0u, 0u, 0u};

// One B fragment: bytes b and b+1 of `w` hold the codes of 8 consecutive n
// (code c = q + 1 of the i-th at bits 2i). rep_lo / rep_hi replicate byte b
// / b+1 into all four bytes (selectors 0x01010101 * b, * (b+1)).
__device__ __forceinline__ bf16x8 decode_codes8(uint32_t w, uint32_t rep_lo, uint32_t rep_hi) {
    const uint32_t hi_tab = 0x003F00BFu;  // sel 0 -> 0xBF, 1 -> 0x00, 2 -> 0x3F
    const uint32_t lo_tab = 0x00800080u;  // sel 4 -> 0x80, 5 -> 0x00, 6 -> 0x80
    const uint32_t d0 = __builtin_amdgcn_perm(0u, w, rep_lo);
    const uint32_t d1 = __builtin_amdgcn_perm(0u, w, rep_hi);
    // Per 16-bit half: the two bytes of a bf16 both carry one code, and the
    // low byte's selector gets +4 (the second table).
    auto pair = [&](uint32_t d, unsigned sa, unsigned sb) -> uint32_t {
        const u16x2 sh = __builtin_bit_cast(u16x2, d) >> (u16x2){(unsigned short)sa,
                                                                  (unsigned short)sb};
        const uint32_t sel = (__builtin_bit_cast(uint32_t, sh) & 0x03030303u) | 0x00040004u;
        return __builtin_amdgcn_perm(lo_tab, hi_tab, sel);
    };
    return __builtin_bit_cast(bf16x8, make_uint4(pair(d0, 0, 2), pair(d0, 4, 6), pair(d1, 0, 2),
                                                 pair(d1, 4, 6)));
}

// Physical 16-byte chunk of logical chunk c of LDS row r. dy rows of 8
// chunks use the forward GEMM's swizzle; rows of 16 chunks XOR with r % 16,
// so any 16 aligned consecutive rows read one logical chunk from 16
// distinct bank groups. Code rows of 2 chunks swap halves every 8 rows.
template <int CH>
__device__ __forceinline__ int ste_swz_a(int r) {
    if constexpr (CH == 8) return swz_a(r);
    else return r & 15;
}
template <int CH>
__device__ __forceinline__ int ste_swz_b(int r) {
    if constexpr (CH == 1) return 0;
    else return (r >> 3) & 1;
}

// BR: n per reduction stage (64 or 128): 2*BR bytes of dy and BR/4 bytes of
// codes per row.
template <int BM, int BN, int WGM, int WGN, int BR, int STAGES, int WPE>
__global__ __launch_bounds__(64 * WGM * WGN, WPE) void k_ste_dx(
    const uint16_t* __restrict__ dy, int M, int N, const uint8_t* __restrict__ qT, int RBT,
    const float* __restrict__ gamma_p, int K, float* __restrict__ dx) {
    constexpr int NW = WGM * WGN;
    constexpr int WM = BM / WGM, WN = BN / WGN;
    constexpr int TM = WM / 32, TN = WN / 32;
    constexpr int AROW = 2 * BR, BROW = BR / 4;   // bytes per row per stage
    constexpr int CH_A = AROW / 16, CH_B = BROW / 16;
    constexpr int SUB = BR / 16;                  // MFMA substeps per stage
    constexpr int A_STAGE = BM * AROW;
    constexpr int B_STAGE = BN * BROW;
    constexpr int STAGE = A_STAGE + B_STAGE;
    constexpr int A_RPI = 64 / CH_A, B_RPI = 64 / CH_B;  // rows per DMA instruction
    constexpr int A_ROWS = BM / NW, B_ROWS = BN / NW;    // rows loaded per wave
    constexpr int A_INSTR = A_ROWS / A_RPI, B_INSTR = B_ROWS / B_RPI;
    constexpr int LOADS = A_INSTR + B_INSTR;
    static_assert(BR == 64 || BR == 128, "stage width");
    static_assert(TM >= 1 && TN >= 1 && A_INSTR >= 1 && B_INSTR >= 1, "tile shape");
    static_assert(A_ROWS % A_RPI == 0 && B_ROWS % B_RPI == 0, "tile shape");
    static_assert(STAGES >= 3 && LOADS * (STAGES - 1) < 64, "pipeline depth");

    extern __shared__ __align__(16) uint8_t smem[];

    const int tid = threadIdx.x;
    const int lane = tid % kWave;
    const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int wm0 = (wave % WGM) * WM, wn0 = (wave / WGM) * WN;

    // Tile order as in the forward GEMM: a contiguous range of tiles per XCD,
    // walked in groups of 8 row tiles.
    const int nM = (M + BM - 1) / BM, nN = (K + BN - 1) / BN;
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
    const int m0 = bm * BM, k0 = bn * BN;

    const int NK = (N + BR - 1) / BR;

    // Stage loads. The DMA puts lane l's 16 bytes at physical chunk l % CH of
    // row l / CH of the instruction's rows, so each lane loads the logical
    // chunk that the swizzle maps there. dy rows past M and code rows past K
    // are clamped (their results are not stored). dy chunks at or past N
    // (8 n each, all or none valid since N % 8 == 0) and code chunks past the
    // row's padded length come from a zero array: the dy factor is then 0.
    const uint16_t* a_src[A_INSTR];
    int a_chunk[A_INSTR];
#pragma unroll
    for (int i = 0; i < A_INSTR; ++i) {
        const int r = wave * A_ROWS + A_RPI * i + lane / CH_A;
        a_chunk[i] = (lane % CH_A) ^ ste_swz_a<CH_A>(r);
        a_src[i] = dy + (size_t)min(m0 + r, M - 1) * N + 8 * a_chunk[i];
    }
    const uint8_t* b_src[B_INSTR];
    int b_chunk[B_INSTR];
#pragma unroll
    for (int i = 0; i < B_INSTR; ++i) {
        const int r = wave * B_ROWS + B_RPI * i + lane / CH_B;
        b_chunk[i] = (lane % CH_B) ^ ste_swz_b<CH_B>(r);
        b_src[i] = qT + (size_t)min(k0 + r, K - 1) * RBT + 16 * b_chunk[i];
    }

    const uint32_t smem_base = (uint32_t)(size_t)(lds_u8_t*)smem;
    auto issue = [&](int kt) {
        const uint32_t st = smem_base + (uint32_t)((kt % STAGES) * STAGE);
        const int n0 = kt * BR;
#pragma unroll
        for (int i = 0; i < A_INSTR; ++i) {
            const void* src = n0 + 8 * a_chunk[i] < N ? (const void*)(a_src[i] + n0)
                                                      : (const void*)kSteZero16;
            lds_dma16(src, st + (wave * A_ROWS + A_RPI * i) * AROW);
        }
#pragma unroll
        for (int i = 0; i < B_INSTR; ++i) {
            const void* src = n0 / 4 + 16 * b_chunk[i] < RBT ? (const void*)(b_src[i] + n0 / 4)
                                                            : (const void*)kSteZero16;
            lds_dma16(src, st + A_STAGE + (wave * B_ROWS + B_RPI * i) * BROW);
        }
    };

    f32x16 acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

    const int fr = lane % 32, fg = lane / 32;
    // Byte selectors of this lane group's code bytes within a stage dword.
    const uint32_t rep_lo = 0x01010101u * (2 * fg), rep_hi = 0x01010101u * (2 * fg + 1);

    // The codes of a B-fragment row for the whole stage: CH_B * 4 dwords,
    // dword s feeding substep s.
    auto read_b = [&](uint4 (*bp)[CH_B], int kt) {
        const uint8_t* Bs = smem + (kt % STAGES) * STAGE + A_STAGE;
#pragma unroll
        for (int j = 0; j < TN; ++j) {
            const int r = wn0 + 32 * j + fr;
#pragma unroll
            for (int h = 0; h < CH_B; ++h)
                bp[j][h] = *reinterpret_cast<const uint4*>(Bs + r * BROW +
                                                           16 * (h ^ ste_swz_b<CH_B>(r)));
        }
    };
    // A fragment of substep s: row r, n = 16s + 8g .. +8 = logical chunk 2s + g.
    auto read_a = [&](bf16x8* af, int kt, int s) {
        const uint8_t* As = smem + (kt % STAGES) * STAGE;
#pragma unroll
        for (int i = 0; i < TM; ++i) {
            const int r = wm0 + 32 * i + fr;
            af[i] = *reinterpret_cast<const bf16x8*>(As + r * AROW +
                                                     16 * ((2 * s + fg) ^ ste_swz_a<CH_A>(r)));
        }
    };
    auto decode = [&](bf16x8* bf, const uint4 (*bp)[CH_B], int s) {
#pragma unroll
        for (int j = 0; j < TN; ++j) {
            const uint4 q4 = bp[j][s / 4];
            const int d = s % 4;
            const uint32_t w = d == 0 ? q4.x : d == 1 ? q4.y : d == 2 ? q4.z : q4.w;
            bf[j] = decode_codes8(w, rep_lo, rep_hi);
        }
    };

    // Pipeline as in the forward GEMM: stage kt+STAGES-1 is issued in
    // substep 1 of step kt, right after the barrier that follows this wave's
    // wait for stage kt+1 (so stage kt+1 is visible to all) and proves every
    // wave is done with step kt-1 (whose buffer is refilled).
#pragma unroll
    for (int st = 0; st < STAGES - 1; ++st)
        if (st < NK) issue(st);
    {
        wait_stages<LOADS, STAGES - 2>(min(STAGES - 2, NK - 1));
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
    }
    uint4 bp[TN][CH_B], bpn[TN][CH_B];
    bf16x8 af[TM], an[TM], bf[TN], bfn[TN];
    read_b(bp, 0);
    read_a(af, 0, 0);
    decode(bf, bp, 0);

    for (int kt = 0; kt < NK; ++kt) {
        const bool more = kt + 1 < NK;
#pragma unroll
        for (int s = 0; s < SUB; ++s) {
            if (s < SUB - 1) {
                read_a(an, kt, s + 1);
                decode(bfn, bp, s + 1);
            } else if (more) {
                read_a(an, kt + 1, 0);
                decode(bfn, bpn, 0);
            }
#pragma unroll
            for (int i = 0; i < TM; ++i)
#pragma unroll
                for (int j = 0; j < TN; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bf[j], acc[i][j],
                                                                        0, 0, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, TM, 0);
#pragma unroll
            for (int q = 0; q < TM * TN; ++q) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);
            }
            if (s == 1 && more) {
                wait_stages<LOADS, STAGES - 3>(min(STAGES - 3, NK - 2 - kt));
                __builtin_amdgcn_s_barrier();
                asm volatile("" ::: "memory");
                if (kt + STAGES - 1 < NK) issue(kt + STAGES - 1);
                read_b(bpn, kt + 1);
            }
#pragma unroll
            for (int i = 0; i < TM; ++i) af[i] = an[i];
#pragma unroll
            for (int j = 0; j < TN; ++j) bf[j] = bfn[j];
            __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int h = 0; h < CH_B; ++h) bp[j][h] = bpn[j][h];
    }

    // C layout of the 32x32 MFMA: lane l, register v holds row
    // 8*(v/4) + 4*(l/32) + v%4 (token) and column l%32 (input feature).
    const float g = *gamma_p;
#pragma unroll
    for (int i = 0; i < TM; ++i) {
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            const int m = m0 + wm0 + 32 * i + 8 * (v / 4) + 4 * (lane / 32) + (v % 4);
            if (m < M) {
                float* row = dx + (size_t)m * K;
#pragma unroll
                for (int j = 0; j < TN; ++j) {
                    const int k = k0 + wn0 + 32 * j + (lane % 32);
                    if (k < K) __builtin_nontemporal_store(acc[i][j][v] * g, row + k);
                }
            }
            __builtin_amdgcn_sched_barrier(0);
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

template <int BM, int BN, int WGM, int WGN, int BR, int STAGES, int WPE>
static hipError_t launch_ste_tile(const uint16_t* dy, int M, int N, const uint8_t* qT,
                                  const float* gamma, int K, float* dx, hipStream_t stream) {
    constexpr size_t lds = (size_t)STAGES * (BM * 2 * BR + BN * BR / 4);
    static_assert(lds <= 160 * 1024, "a workgroup holds at most 160 KiB of LDS");
    auto kern = &k_ste_dx<BM, BN, WGM, WGN, BR, STAGES, WPE>;
    static std::atomic<uint64_t> lds_set{0};
    {
        hipError_t e = allow_dynamic_lds(reinterpret_cast<const void*>(kern), lds, lds_set);
        if (e != hipSuccess) return e;
    }
    const int tiles = ((M + BM - 1) / BM) * ((K + BN - 1) / BN);
    hipLaunchKernelGGL(kern, dim3(tiles), dim3(64 * WGM * WGN), lds, stream, dy, M, N, qT,
                       (int)ste_t_row_bytes(N), gamma, K, dx);
    return hipGetLastError();
}

hipError_t launch_ste_dx(const uint16_t* dy, int M, int N, const uint8_t* qT, const float* gamma,
                         int K, float* dx, hipStream_t stream) {
    // The forward GEMM's rule between 128 x 512 tiles (one 8-wave workgroup
    // per CU) and 128 x 256 tiles (two 4-wave workgroups per CU).
    constexpr int64_t kCUs = 256;
    auto tiles = [&](int bm, int bn) {
        return (int64_t)((M + bm - 1) / bm) * ((K + bn - 1) / bn);
    };
    const int64_t t512 = tiles(128, 512), t256 = tiles(128, 256);
    if (t512 >= kCUs / 2 && 2 * ((t512 + kCUs - 1) / kCUs) <= (t256 + kCUs - 1) / kCUs)
        return launch_ste_tile<128, 512, 1, 8, 128, 3, 2>(dy, M, N, qT, gamma, K, dx, stream);
    return launch_ste_tile<128, 256, 1, 4, 64, 3, 2>(dy, M, N, qT, gamma, K, dx, stream);
}

}  // namespace bl
