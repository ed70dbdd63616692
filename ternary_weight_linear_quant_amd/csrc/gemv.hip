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
// int8 activation block is staged once per workgroup. Tokens >= M read zero. Waves that split K for
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
constexpr int kXPad = 16;  // LDS row padding (bytes) against bank conflicts
constexpr int kNB = 4;     // chunks per lane in flight per batch

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

template <int RG>
__global__ __launch_bounds__(kGemvThreads, 8) void k_gemv(const int8_t* __restrict__ xq,
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
    const int wave = tid / kWave, lane = tid % kWave;
    const int rg = wave % RG, ks = wave / RG;
    const int r = lane % 16, g = lane / 16;
    const int row0 = lb * (16 * RG) + rg * 16;
    const int row = min(row0 + r, N - 1);
    const int KW = K / 16;       // packed words per row
    const int nfull = KW / 16;   // full 256-weight chunks per row
    const uint32_t* wrow = P.W + (size_t)row * KW + 4 * g;
    // This wave's chunks: c_i = ks + KS * i, i < nw.
    const int nw = ks < nfull ? (nfull - ks + KS - 1) / KS : 0;

    // 1. First batch of weight loads, before anything waits.
    uint4 wb[kNB];
#pragma unroll
    for (int i = 0; i < kNB; ++i)
        if (i < nw) wb[i] = *reinterpret_cast<const uint4*>(wrow + 16 * (ks + KS * i));

    // 2. Stage the activations: M rows of K bytes, 16 B per thread per step.
    const int xstride = K + kXPad;
    {
        const int cpr = K / 16;  // 16-byte chunks per row
        const int nchunks = M * cpr;
        const uint4* src = reinterpret_cast<const uint4*>(xq);
        for (int c = tid; c < nchunks; c += kGemvThreads) {
            const int mm = c / cpr, cc = c - mm * cpr;
            *reinterpret_cast<uint4*>(smem + mm * xstride + 16 * cc) = src[c];
        }
    }
    const int tok = lane % 16;
    const bool tok_ok = tok < M;
    const int8_t* xrow =
        reinterpret_cast<const int8_t*>(smem) + (tok_ok ? tok : 0) * xstride + 64 * g;
    __syncthreads();

    v4i acc = {0, 0, 0, 0};
    const v4i zero = {0, 0, 0, 0};
    auto process = [&](const uint4 wv, int c) {
        const uint32_t w4[4] = {wv.x, wv.y, wv.z, wv.w};
        const int8_t* xb = xrow + 256 * c;
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            const v4i a = expand_word_neg(w4[s]);
            const v4i b = tok_ok ? *reinterpret_cast<const v4i*>(xb + 16 * s) : zero;
            acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, acc, 0, 0, 0);
        }
    };

    // 3. Batches: issue the next batch's loads, then consume the current one.
    for (int b0 = 0; b0 < nw; b0 += kNB) {
        uint4 wn[kNB];
        const int nb = b0 + kNB;
#pragma unroll
        for (int i = 0; i < kNB; ++i)
            if (nb + i < nw) wn[i] = *reinterpret_cast<const uint4*>(wrow + 16 * (ks + KS * (nb + i)));
#pragma unroll
        for (int i = 0; i < kNB; ++i)
            if (b0 + i < nw) process(wb[i], ks + KS * (b0 + i));
#pragma unroll
        for (int i = 0; i < kNB; ++i) wb[i] = wn[i];
    }

    // Tail: KW % 16 words (a multiple of 4, since K % 64 == 0). Lane group g
    // holds words 4g..4g+3 of the partial chunk when 4g < rem.
    const int rem = KW - 16 * nfull;
    if (rem != 0 && ks == nfull % KS) {
        const bool gv = 4 * g < rem;
        const uint4 wv = gv ? *reinterpret_cast<const uint4*>(wrow + 16 * nfull)
                            : make_uint4(0, 0, 0, 0);
        const uint32_t w4[4] = {wv.x, wv.y, wv.z, wv.w};
        const int8_t* xb = xrow + 256 * nfull;
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            const v4i a = gv ? expand_word_neg(w4[s]) : zero;
            const v4i b = (gv && tok_ok) ? *reinterpret_cast<const v4i*>(xb + 16 * s) : zero;
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

template <int RG>
static hipError_t launch_gemv_rg(const int8_t* xq, const float* xs, int M, int K,
                                 const GemvArgs& args, hipStream_t stream) {
    const size_t lds = (size_t)M * (K + kXPad);
    static bool attr_set = false;
    if (lds > 64 * 1024 && !attr_set) {
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_gemv<RG>),
                                           hipFuncAttributeMaxDynamicSharedMemorySize,
                                           (int)(kGemvMaxXBytes + kGemvMaxM * kXPad));
        if (e != hipSuccess) return e;
        attr_set = true;
    }
    const int blocks = args.mat[0].blocks + args.mat[1].blocks;
    hipLaunchKernelGGL(k_gemv<RG>, dim3(blocks), dim3(kGemvThreads), lds, stream, xq, xs, M, K,
                       args);
    return hipGetLastError();
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
    return launch_gemv_rg<1>(xq, xs, M, K, a, stream);
}

hipError_t launch_gemv_pair(const int8_t* xq, const float* xs, int M, int K, const uint32_t* W1,
                            const float* g1, int N1, float* y1, const uint32_t* W2,
                            const float* g2, int N2, float* y2, hipStream_t stream) {
    if (!gemv_supported(M, K)) return hipErrorInvalidValue;
    GemvArgs a;
    a.mat[0] = make_mat(W1, g1, N1, y1, nullptr, 16);
    a.mat[1] = make_mat(W2, g2, N2, y2, nullptr, 16);
    return launch_gemv_rg<1>(xq, xs, M, K, a, stream);
}

}  // namespace bl
