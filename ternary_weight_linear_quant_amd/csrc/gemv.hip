// Decode BitLinear (M <= 16 tokens): stream the 2-bit packed weights once.
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
// Layout of the work. A wave owns 16 weight rows (the MFMA A operand: lane
// l -> row l % 16, k-group l / 16) and every KS-th 256-weight chunk of K. Each
// lane loads 16 bytes of its row per chunk (4 packed words = 64 weights); the
// 4 lanes of a row cover 64 contiguous bytes. A wave issues the loads of up to
// 4 chunks at once, before anything else, so the whole weight stream of a
// small matrix is in flight within the first microsecond; longer rows are
// double-buffered in batches of 4. Registers are capped for 8 waves per SIMD,
// which keeps the 70B-class grids resident in one round. Word s of a lane's
// 16 bytes feeds MFMA s; the B operand (lane l -> token l % 16) reads the 16
// activation bytes of the same k positions from LDS, where the whole [M][K]
// int8 activation block is staged once per workgroup by direct global-to-LDS
// loads issued before the weight loads, token-minor so that a fragment read
// is 16 consecutive 16-byte slots. Only that staging is waited for before the
// workgroup barrier, so the weight stream stays in flight. Tokens >= M read
// zero. Waves that split K for
// the same rows reduce in LDS; the epilogue rescales by x_scale[m] * gamma.
//
// One launch may cover two weight matrices that share the input (the gate
// and up projections of an FFN): workgroups [0, blocks0) serve the first,
// the rest the second.
//
// Roofline: HBM. Algorithmic bytes per matrix = N*K/4 (packed weights) + M*K
// (activations) + 4*M (scales) + 4 (gamma) + 4*M*N (y).
#include "common.hpp"
#include "launch.hpp"

namespace bl {

constexpr int kGemvThreads = 256;
constexpr int kGemvMaxM = 16;
constexpr int64_t kGemvMaxXBytes = 128 * 1024;

struct GemvMat {
    const uint32_t* W;
    const float* gamma;
    float* y;
    int32_t* acc;
    int N;
    int blocks;
};
struct GemvArgs {
    GemvMat mat[2];
};

// R: ring of chunk loads in flight per lane; WPE: waves per SIMD the register
// allocation must allow (short rows want many waves, long rows a deep ring).
template <int RG, int R, int WPE>
__global__ __launch_bounds__(kGemvThreads, WPE) void k_gemv(const int8_t* __restrict__ xq,
                                                       const float* __restrict__ xs, int M,
                                                       int K, GemvArgs args) {
    constexpr int KS = 4 / RG;  // waves splitting K within a row group
    extern __shared__ __align__(16) uint8_t smem[];
    __shared__ v4i red[4][kWave];

    const bool second = (int)blockIdx.x >= args.mat[0].blocks;
    const GemvMat P = second ? args.mat[1] : args.mat[0];
    const int lb = second ? (int)blockIdx.x - args.mat[0].blocks : (int)blockIdx.x;
    const int N = P.N;

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int lane = tid % kWave;
    const int rg = wave % RG, ks = wave / RG;
    const int r = lane % 16, g = lane / 16;
    const int row0 = lb * (16 * RG) + rg * 16;
    const int row = min(row0 + r, N - 1);
    const int KW = K / 16;       // packed words per row
    const int nfull = KW / 16;   // full 256-weight chunks per row
    const uint32_t* wrow = P.W + (size_t)row * KW + 4 * g;
    // This wave's chunks: c_i = ks + KS * i, i < nw.
    const int nw = ks < nfull ? (nfull - ks + KS - 1) / KS : 0;

    // 1. Activations straight into LDS, issued first. LDS layout: 16-byte
    //    chunk j of token t at slot j*M + t, so the 16 tokens of a B fragment
    //    read 16 consecutive slots. Each DMA instruction fills 64 slots.
    const int cpr = K / 16;
    const int total = M * cpr;
    const uint32_t xbase = lds_offset(smem);
    for (int p0 = wave * kWave; p0 < total; p0 += kGemvThreads) {
        const int p = p0 + lane;
        if (p < total) {
            const int j = p / M, t = p - j * M;
            lds_dma16(xq + (size_t)t * K + 16 * j, xbase + 16 * p0);
        }
    }
    asm volatile("" ::: "memory");

    // 2. Up to R chunks of weight loads, before anything waits.
    uint4 wb[R];
#pragma unroll
    for (int i = 0; i < R; ++i)
        if (i < nw) wb[i] = *reinterpret_cast<const uint4*>(wrow + 16 * (ks + KS * i));
    asm volatile("" ::: "memory");

    // 3. Wait for this wave's activation DMA only (the weight loads, issued
    //    after it, may stay in flight), then make every wave's part visible.
    wait_vmcnt_le8(min(nw, R));
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");

    const int tok = lane % 16;
    const bool tok_ok = tok < M;
    const int8_t* xl = reinterpret_cast<const int8_t*>(smem) + 16 * (tok_ok ? tok : 0);

    v4i acc = {0, 0, 0, 0};
    const v4i zero = {0, 0, 0, 0};
    // B fragment of chunk c, sub-step s: activation chunk j = 16c + 4g + s.
    auto process = [&](const uint4 wv, int c) {
        const uint32_t w4[4] = {wv.x, wv.y, wv.z, wv.w};
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            const v4i a = expand_word_neg(w4[s]);
            const int j = 16 * c + 4 * g + s;
            const v4i b = tok_ok ? *reinterpret_cast<const v4i*>(xl + 16 * j * M) : zero;
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
                    wb[i] = *reinterpret_cast<const uint4*>(wrow + 16 * (ks + KS * (ci + R)));
            }
        }
    }

    // Tail: KW % 16 words (a multiple of 4, since K % 64 == 0). Lane group g
    // holds words 4g..4g+3 of the partial chunk when 4g < rem.
    const int rem = KW - 16 * nfull;
    if (rem != 0 && ks == nfull % KS) {
        const bool gv = 4 * g < rem;
        const uint4 wv = gv ? *reinterpret_cast<const uint4*>(wrow + 16 * nfull)
                            : make_uint4(0, 0, 0, 0);
        const uint32_t w4[4] = {wv.x, wv.y, wv.z, wv.w};
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            const v4i a = gv ? expand_word_neg(w4[s]) : zero;
            const int j = 16 * nfull + 4 * g + s;
            const v4i b = (gv && tok_ok) ? *reinterpret_cast<const v4i*>(xl + 16 * j * M) : zero;
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

bool gemv_supported(int64_t M, int64_t K) {
    return M >= 1 && M <= kGemvMaxM && M * K <= kGemvMaxXBytes;
}

template <int RG, int R, int WPE>
static hipError_t launch_gemv_cfg(const int8_t* xq, const float* xs, int M, int K,
                                 const GemvArgs& args, hipStream_t stream) {
    const size_t lds = (size_t)M * K;
    static bool attr_set = false;
    if (lds > 64 * 1024 && !attr_set) {
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_gemv<RG, R, WPE>),
                                           hipFuncAttributeMaxDynamicSharedMemorySize,
                                           (int)kGemvMaxXBytes);
        if (e != hipSuccess) return e;
        attr_set = true;
    }
    const int blocks = args.mat[0].blocks + args.mat[1].blocks;
    hipLaunchKernelGGL((k_gemv<RG, R, WPE>), dim3(blocks), dim3(kGemvThreads), lds, stream, xq, xs, M, K,
                       args);
    return hipGetLastError();
}

// Rows of more than 8 chunks per wave (K > 8192) take the deep ring.
static hipError_t launch_gemv_auto(const int8_t* xq, const float* xs, int M, int K,
                                   const GemvArgs& args, hipStream_t stream) {
    const int chunks_per_wave = (K / 256 + 3) / 4;
    if (chunks_per_wave > 8) return launch_gemv_cfg<1, 8, 1>(xq, xs, M, K, args, stream);
    return launch_gemv_cfg<1, 4, 8>(xq, xs, M, K, args, stream);
}

static GemvMat make_mat(const uint32_t* Wp, const float* gamma, int N, float* y, int32_t* acc,
                        int rows_per_block) {
    GemvMat m;
    m.W = Wp;
    m.gamma = gamma;
    m.y = y;
    m.acc = acc;
    m.N = N;
    m.blocks = Wp ? (N + rows_per_block - 1) / rows_per_block : 0;
    return m;
}

hipError_t launch_gemv(const int8_t* xq, const float* xs, int M, int K, const uint32_t* Wp,
                       const float* gamma, int N, float* y, int32_t* acc, hipStream_t stream) {
    if (!gemv_supported(M, K)) return hipErrorInvalidValue;
    GemvArgs a;
    a.mat[0] = make_mat(Wp, gamma, N, y, acc, 16);
    a.mat[1] = make_mat(nullptr, nullptr, 1, nullptr, nullptr, 16);
    return launch_gemv_auto(xq, xs, M, K, a, stream);
}

hipError_t launch_gemv_pair(const int8_t* xq, const float* xs, int M, int K, const uint32_t* W1,
                            const float* g1, int N1, float* y1, const uint32_t* W2,
                            const float* g2, int N2, float* y2, hipStream_t stream) {
    if (!gemv_supported(M, K)) return hipErrorInvalidValue;
    GemvArgs a;
    a.mat[0] = make_mat(W1, g1, N1, y1, nullptr, 16);
    a.mat[1] = make_mat(W2, g2, N2, y2, nullptr, 16);
    return launch_gemv_auto(xq, xs, M, K, a, stream);
}

}  // namespace bl
