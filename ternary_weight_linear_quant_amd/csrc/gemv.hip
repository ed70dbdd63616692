// Decode BitLinear (M <= 16 tokens): stream the packed weights once.
//
// Source: inferownia.pl, "BitNet b1.58: era 1-bitowych LLM-ów", section
// "Mnożenie? Jakie mnożenie" and juhe.plus (Habr repost), section «Когда - три
// лучше двух»: with weights in {-1, 0, +1} the product is a sum of the inputs
// with +1 weights minus the sum with -1 weights; zero weights drop out. Here
// the sign selection is done by the int8 matrix cores: the packed codes are
// expanded in registers to {+1, 0, -1} bytes (the negated weights; a zero
// weight contributes a zero product) and fed to v_mfma_i32_16x16x64_i8
// against the int8 activations, so the int32 sums are exact and only need a
// sign flip at the end.
//
// Three storage formats share the kernel (a policy class each):
//   Ternary2  2 bits per ternary weight (the library's main format);
//   Binary1   1 bit per {-1, +1} weight, the original BitNet's binary
//             weights (same page, section "Dlaczego akurat ternarne, a nie
//             czyste zero-jeden");
//   Base3     five ternary weights per byte as a base-3 number, 1.6 bits per
//             weight, near the log2(3) bound of section "Skąd te 1,58 bita".
// A lane always loads 16 bytes of its row; the format decides how many
// weights that is (64, 128 or 80) and so how many 16-weight MFMA sub-steps
// (4, 8 or 5) it feeds. Base-3 bytes are decoded through a 8 KB LDS table:
// for each byte value and each of the four byte alignments of a 5-weight
// group in the output stream, the five weight bytes already shifted into
// place, so one 8-byte table read and two ORs place five weights.
//
// Layout of the work. A workgroup of RG x KS waves owns RG groups of 16
// weight rows (the MFMA A operand: lane l -> row l % 16, k-group l / 16);
// wave (rg, ks) takes group rg and every KS-th 64-byte chunk of its rows.
// Several row groups per workgroup share one staging of the activations.
// Each lane loads 16 bytes of its row per chunk; the 4 lanes of a row cover
// 64 contiguous bytes. The whole [M][K] int8 activation block is staged once
// per workgroup in LDS by direct global-to-LDS loads issued before the weight
// loads, one token row after another (rows padded by 16 bytes against bank
// conflicts; bytes past K, where a format pads its rows, hold zeros), each
// load 1 KB of one row. Then each wave
// issues up to R chunk loads of its weights and waits only for its
// activation loads before the workgroup barrier, so the weight stream stays
// in flight; a ring of R slots refills each chunk R ahead. Tokens >= M read
// zero. Waves that split K for the same rows reduce in LDS; the epilogue
// rescales by x_scale[m] * gamma.
//
// One launch may cover two weight matrices that share the input (the gate
// and up projections of an FFN): workgroups [0, blocks0) serve the first,
// the rest the second.
//
// Roofline: HBM. Algorithmic bytes per matrix = N * row_bytes (packed
// weights) + M*K (activations) + 4*M (scales) + 4 (gamma) + 4*M*N (y).
#include "common.hpp"
#include "launch.hpp"

namespace bl {

constexpr int kGemvMaxM = 16;
constexpr int64_t kGemvMaxXBytes = 128 * 1024;
constexpr int kBase3TableBytes = 4 * 256 * 8;

// ------------------------------------------------------------ formats ----

// kWaves: waves per SIMD the short-row configuration allows (the decoders
// of the denser formats hold more registers).
struct Ternary2 {
    static constexpr int kSub = 4;
    static constexpr bool kTable = false;
    static constexpr int kWaves = 8;
    __host__ __device__ static int row_bytes(int K) { return K / 4; }
    __host__ __device__ static int k_extent(int K) { return K; }
};

struct Binary1 {
    static constexpr int kSub = 8;
    static constexpr bool kTable = false;
    static constexpr int kWaves = 4;
    __host__ __device__ static int row_bytes(int K) { return 16 * ((K + 127) / 128); }
    __host__ __device__ static int k_extent(int K) { return 128 * ((K + 127) / 128); }
};

struct Base3 {
    static constexpr int kSub = 5;
    static constexpr bool kTable = true;
    static constexpr int kWaves = 4;
    __host__ __device__ static int row_bytes(int K) { return 16 * (((K + 4) / 5 + 15) / 16); }
    __host__ __device__ static int k_extent(int K) { return 5 * row_bytes(K); }
};

// Sub-step s of a 16-byte lane load as an MFMA A fragment of 16 negated
// weights, k increasing.
template <class F>
struct Decoder;

template <>
struct Decoder<Ternary2> {
    uint32_t w[4];
    __device__ __forceinline__ Decoder(const uint4 v, const uint2*) : w{v.x, v.y, v.z, v.w} {}
    __device__ __forceinline__ v4i frag(int s) const { return expand_word_neg(w[s]); }
};

// Bits of word s/2, half s%2: (w >> p) & 0x01010101 holds the bits of four
// consecutive weights; v_perm maps bit 0 (weight -1) to +1 and bit 1 (weight
// +1) to -1.
template <>
struct Decoder<Binary1> {
    uint32_t w[4];
    __device__ __forceinline__ Decoder(const uint4 v, const uint2*) : w{v.x, v.y, v.z, v.w} {}
    __device__ __forceinline__ v4i frag(int s) const {
        const uint32_t x = w[s / 2];
        const int p0 = 4 * (s % 2);
        v4i a;
#pragma unroll
        for (int d = 0; d < 4; ++d)
            a[d] = (int)__builtin_amdgcn_perm(0u, 0x0000FF01u, (x >> (p0 + d)) & 0x01010101u);
        return a;
    }
};

// Byte j of the load holds weights 5j .. 5j+4 of the lane's 80; they go to
// bytes 5j .. 5j+4 of a 20-dword stream, i.e. dword 5j/4 at byte offset j%4.
template <>
struct Decoder<Base3> {
    uint32_t d[20];
    __device__ __forceinline__ Decoder(const uint4 v, const uint2* tab) {
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int i = 0; i < 20; ++i) d[i] = 0;
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            const uint32_t b = (w[j / 4] >> (8 * (j % 4))) & 0xFFu;
            const uint2 e = tab[(j % 4) * 256 + b];
            d[(5 * j) / 4] |= e.x;
            d[(5 * j) / 4 + 1] |= e.y;
        }
    }
    __device__ __forceinline__ v4i frag(int s) const {
        return v4i{(int)d[4 * s], (int)d[4 * s + 1], (int)d[4 * s + 2], (int)d[4 * s + 3]};
    }
};

// Table entry (a, b): the five negated weights of base-3 byte b (weight =
// digit - 1, least significant digit first) as bytes a .. a+4 of 8. Bytes
// above 242 (never written by the packer) decode to zeros.
__device__ __forceinline__ void build_base3_table(uint2* tab, int tid, int nthreads) {
    for (int e = tid; e < 1024; e += nthreads) {
        const int a = e / 256;
        int b = e % 256;
        uint64_t v = 0;
        if (b < 243) {
#pragma unroll
            for (int i = 0; i < 5; ++i) {
                const int c = b % 3;
                b /= 3;
                v |= (uint64_t)(uint8_t)(int8_t)(1 - c) << (8 * (a + i));
            }
        }
        tab[e] = make_uint2((uint32_t)v, (uint32_t)(v >> 32));
    }
}

// -------------------------------------------------------------- kernel ----

struct GemvMat {
    const uint8_t* W;
    const float* gamma;
    float* y;
    int32_t* acc;
    int N;
    int blocks;
};
struct GemvArgs {
    GemvMat mat[2];
};

// RG: row groups per workgroup; KS: waves splitting K; R: ring of chunk
// loads in flight per lane; WPE: waves per SIMD the register allocation must
// allow (short rows want many waves, long rows a deep ring).
template <class F, int RG, int KS, int R, int WPE>
__global__ __launch_bounds__(64 * RG * KS, WPE) void k_gemv(const int8_t* __restrict__ xq,
                                                          const float* __restrict__ xs, int M,
                                                          int K, GemvArgs args) {
    constexpr int NT = 64 * RG * KS;
    extern __shared__ __align__(16) uint8_t smem[];
    __shared__ v4i red[RG * KS][kWave];

    const bool second = (int)blockIdx.x >= args.mat[0].blocks;
    const GemvMat P = second ? args.mat[1] : args.mat[0];
    const int lb = second ? (int)blockIdx.x - args.mat[0].blocks : (int)blockIdx.x;
    const int N = P.N;

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int lane = tid % kWave;
    const int rg = wave % RG, ks = wave / RG;
    const int r = lane % 16, g = lane / 16;
    const int row0 = (lb * RG + rg) * 16;
    const int row = min(row0 + r, N - 1);
    const int RB = F::row_bytes(K);   // bytes per packed row, a multiple of 16
    const int nfull = RB / 64;        // full 64-byte chunks per row
    const uint8_t* wrow = P.W + (size_t)row * RB + 16 * g;
    // This wave's chunks: c_i = ks + KS * i, i < nw.
    const int nw = ks < nfull ? (nfull - ks + KS - 1) / KS : 0;

    // 1. Activations straight into LDS, issued first. LDS layout: token t's
    //    row at t * pitch, pitch = K extent + 16 bytes (16 times an odd
    //    number, so the 16 tokens of a B fragment read fall on distinct
    //    16-byte bank groups). Each DMA instruction fills 1 KB of one token's
    //    row from 1 KB of contiguous memory (lanes past the row's end idle):
    //    a CU draws about 44 GB/s from contiguous 16-byte loads against
    //    25-33 GB/s when the lanes of a load spread over the tokens.
    const int pitch = F::k_extent(K) + 16;
    const int rowv = K / 16;                 // 16-byte pieces per token
    const int nblk = (rowv + kWave - 1) / kWave;
    const uint32_t xbase = lds_offset(smem);
    for (int q = wave; q < M * nblk; q += NT / kWave) {
        const int t = q / nblk, b = q - t * nblk;
        const int v = b * kWave + lane;
        if (v < rowv)
            lds_dma16(xq + (size_t)t * K + 16 * v, xbase + t * pitch + b * kWave * 16);
    }
    asm volatile("" ::: "memory");

    // 2. Up to R chunks of weight loads, before anything waits.
    uint4 wb[R];
#pragma unroll
    for (int i = 0; i < R; ++i)
        if (i < nw) wb[i] = *reinterpret_cast<const uint4*>(wrow + 64 * (ks + KS * i));
    asm volatile("" ::: "memory");

    // Each row's padded K extent holds zeros; the base-3 table follows the
    // activations.
    const int padv = (F::k_extent(K) - K) / 16;
    for (int p = tid; p < M * padv; p += NT) {
        const int t = p / padv;
        *reinterpret_cast<uint4*>(smem + t * pitch + K + 16 * (p - t * padv)) =
            make_uint4(0, 0, 0, 0);
    }
    uint2* tab = reinterpret_cast<uint2*>(smem + M * pitch);
    if constexpr (F::kTable) build_base3_table(tab, tid, NT);

    // 3. Wait for this wave's activation DMA only (the weight loads, issued
    //    after it, may stay in flight) and its LDS stores, then make every
    //    wave's part visible.
    wait_vmcnt_le8(min(nw, R));
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");

    const int tok = lane % 16;
    const bool tok_ok = tok < M;
    const int8_t* xl = reinterpret_cast<const int8_t*>(smem) + (tok_ok ? tok : 0) * pitch;

    v4i acc = {0, 0, 0, 0};
    const v4i zero = {0, 0, 0, 0};
    // B fragment of chunk c, sub-step s: activation chunk
    // j = c * 4*kSub + g * kSub + s (lane group g's weights are contiguous).
    auto process = [&](const uint4 wv, int c) {
        const Decoder<F> dec(wv, tab);
#pragma unroll
        for (int s = 0; s < F::kSub; ++s) {
            const v4i a = dec.frag(s);
            const int j = c * (4 * F::kSub) + g * F::kSub + s;
            const v4i b = tok_ok ? *reinterpret_cast<const v4i*>(xl + 16 * j) : zero;
            acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, acc, 0, 0, 0);
        }
    };

    // 4. Ring of R chunk slots: consume a chunk, then refill its slot with
    //    the chunk R ahead, so up to R loads stay in flight.
    for (int b0 = 0; b0 < nw; b0 += R) {
#pragma unroll
        for (int i = 0; i < R; ++i) {
            const int ci = b0 + i;
            if (ci < nw) {
                process(wb[i], ks + KS * ci);
                if (ci + R < nw)
                    wb[i] = *reinterpret_cast<const uint4*>(wrow + 64 * (ks + KS * (ci + R)));
            }
        }
    }

    // Tail: RB % 64 bytes (a multiple of 16). Lane group g holds 16 bytes of
    // the partial chunk when g < rem16.
    const int rem16 = (RB % 64) / 16;
    if (rem16 != 0 && ks == nfull % KS) {
        const bool gv = g < rem16;
        const uint4 wv = gv ? *reinterpret_cast<const uint4*>(wrow + 64 * nfull)
                            : make_uint4(0, 0, 0, 0);
        const Decoder<F> dec(wv, tab);
#pragma unroll
        for (int s = 0; s < F::kSub; ++s) {
            const v4i a = gv ? dec.frag(s) : zero;
            const int j = nfull * (4 * F::kSub) + g * F::kSub + s;
            const v4i b = (gv && tok_ok) ? *reinterpret_cast<const v4i*>(xl + 16 * j) : zero;
            acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, acc, 0, 0, 0);
        }
    }

    if (KS > 1) {
        red[wave][lane] = acc;
        __syncthreads();
        if (ks != 0) return;
#pragma unroll
        for (int t = 1; t < KS; ++t) acc += red[rg + t * RG][lane];
    }

    // The weights were expanded negated: flip the exact sums back.
    acc = -acc;
    // C layout of the 16x16 MFMA: lane l holds rows 4*(l/16)+i (weights),
    // column l%16 (token).
    if (tok_ok) {
        const float sc = xs[tok] * (*P.gamma);
        const int nbase = row0 + 4 * (lane / 16);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int n = nbase + i;
            if (n < N) {
                P.y[(size_t)tok * N + n] = (float)acc[i] * sc;
                if (P.acc) P.acc[(size_t)tok * N + n] = acc[i];
            }
        }
    }
}

template <class F>
static bool gemv_fits(int64_t M, int64_t K) {
    return M >= 1 && M <= kGemvMaxM && M * F::k_extent((int)K) <= kGemvMaxXBytes;
}

bool gemv_supported(int64_t M, int64_t K) { return gemv_fits<Ternary2>(M, K); }
bool gemv_binary_supported(int64_t M, int64_t K) { return gemv_fits<Binary1>(M, K); }
bool gemv_base3_supported(int64_t M, int64_t K) { return gemv_fits<Base3>(M, K); }

template <class F, int RG, int KS, int R, int WPE>
static hipError_t launch_gemv_cfg(const int8_t* xq, const float* xs, int M, int K,
                                 const GemvArgs& args, hipStream_t stream) {
    // Token rows of K extent + 16 bytes, then the base-3 table.
    const size_t lds = (size_t)M * (F::k_extent(K) + 16) + (F::kTable ? kBase3TableBytes : 0);
    // The attribute takes the largest block any supported shape stages.
    static std::atomic<uint64_t> lds_set{0};
    if (lds > 64 * 1024) {
        hipError_t e = allow_dynamic_lds(
            reinterpret_cast<const void*>(&k_gemv<F, RG, KS, R, WPE>),
            (size_t)(kGemvMaxXBytes + 16 * kGemvMaxM + kBase3TableBytes), lds_set);
        if (e != hipSuccess) return e;
    }
    GemvArgs a = args;
    for (int i = 0; i < 2; ++i)
        a.mat[i].blocks = a.mat[i].W ? (a.mat[i].N + 16 * RG - 1) / (16 * RG) : 0;
    const int blocks = a.mat[0].blocks + a.mat[1].blocks;
    hipLaunchKernelGGL((k_gemv<F, RG, KS, R, WPE>), dim3(blocks), dim3(64 * RG * KS), lds, stream,
                       xq, xs, M, K, a);
    return hipGetLastError();
}

// Four waves per row group, sixteen for very long rows, or eight when the
// grid has fewer than 512 row
// groups (few output rows, as in a down projection) and rows of at least 16
// chunks, so that the CUs hold enough waves; rows of more than 8 chunks per
// wave take the deep ring. With 8 or more tokens and many row groups, two row
// groups share a workgroup: the activation block, staged once per workgroup,
// is then read from L2 half as often.
template <class F>
static hipError_t launch_gemv_auto(const int8_t* xq, const float* xs, int M, int K,
                                   const GemvArgs& args, hipStream_t stream) {
    const int chunks = F::row_bytes(K) / 64;
    const int groups = args.mat[0].blocks + args.mat[1].blocks;
    // Very long rows (>= 64 chunks, as a 28672-wide down projection): 16
    // waves split K so that each streams a few chunks.
    if (chunks >= 64) return launch_gemv_cfg<F, 1, 16, 4, 4>(xq, xs, M, K, args, stream);
    if (M >= 8 && groups >= 384) {
        if ((chunks + 3) / 4 > 4) return launch_gemv_cfg<F, 2, 4, 8, 2>(xq, xs, M, K, args, stream);
        return launch_gemv_cfg<F, 2, 4, 4, 2>(xq, xs, M, K, args, stream);
    }
    if (groups < 512 && chunks >= 16) {
        if ((chunks + 7) / 8 > 8) return launch_gemv_cfg<F, 1, 8, 8, 2>(xq, xs, M, K, args, stream);
        return launch_gemv_cfg<F, 1, 8, 4, 4>(xq, xs, M, K, args, stream);
    }
    if ((chunks + 3) / 4 > 8) return launch_gemv_cfg<F, 1, 4, 8, 1>(xq, xs, M, K, args, stream);
    return launch_gemv_cfg<F, 1, 4, 4, F::kWaves>(xq, xs, M, K, args, stream);
}

static GemvMat make_mat(const void* Wp, const float* gamma, int N, float* y, int32_t* acc,
                        int rows_per_block) {
    GemvMat m;
    m.W = static_cast<const uint8_t*>(Wp);
    m.gamma = gamma;
    m.y = y;
    m.acc = acc;
    m.N = N;
    m.blocks = Wp ? (N + rows_per_block - 1) / rows_per_block : 0;
    return m;
}

template <class F>
static hipError_t launch_gemv_one(const int8_t* xq, const float* xs, int M, int K, const void* Wp,
                                  const float* gamma, int N, float* y, int32_t* acc,
                                  hipStream_t stream) {
    if (!gemv_fits<F>(M, K)) return hipErrorInvalidValue;
    GemvArgs a;
    a.mat[0] = make_mat(Wp, gamma, N, y, acc, 16);
    a.mat[1] = make_mat(nullptr, nullptr, 1, nullptr, nullptr, 16);
    return launch_gemv_auto<F>(xq, xs, M, K, a, stream);
}

hipError_t launch_gemv(const int8_t* xq, const float* xs, int M, int K, const uint32_t* Wp,
                       const float* gamma, int N, float* y, int32_t* acc, hipStream_t stream) {
    return launch_gemv_one<Ternary2>(xq, xs, M, K, Wp, gamma, N, y, acc, stream);
}

hipError_t launch_gemv_binary(const int8_t* xq, const float* xs, int M, int K,
                              const uint32_t* Wb, const float* gamma, int N, float* y,
                              int32_t* acc, hipStream_t stream) {
    return launch_gemv_one<Binary1>(xq, xs, M, K, Wb, gamma, N, y, acc, stream);
}

hipError_t launch_gemv_base3(const int8_t* xq, const float* xs, int M, int K, const uint8_t* W3,
                             const float* gamma, int N, float* y, int32_t* acc,
                             hipStream_t stream) {
    return launch_gemv_one<Base3>(xq, xs, M, K, W3, gamma, N, y, acc, stream);
}

hipError_t launch_gemv_pair(const int8_t* xq, const float* xs, int M, int K, const uint32_t* W1,
                            const float* g1, int N1, float* y1, const uint32_t* W2,
                            const float* g2, int N2, float* y2, hipStream_t stream) {
    if (!gemv_supported(M, K)) return hipErrorInvalidValue;
    GemvArgs a;
    a.mat[0] = make_mat(W1, g1, N1, y1, nullptr, 16);
    a.mat[1] = make_mat(W2, g2, N2, y2, nullptr, 16);
    return launch_gemv_auto<Ternary2>(xq, xs, M, K, a, stream);
}

int64_t packed_row_bytes_binary(int64_t K) { return Binary1::row_bytes((int)K); }
int64_t packed_row_bytes_base3(int64_t K) { return Base3::row_bytes((int)K); }

}  // namespace bl
