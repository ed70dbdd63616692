// Decode BitLinear (M <= 16 tokens): stream the 2-bit packed weights once.
//
// Source: inferownia.pl, "BitNet b1.58: era 1-bitowych LLM-ów", section
// "Mnożenie? Jakie mnożenie" and juhe.plus (Habr repost), section «Когда - три
// лучше двух»: with weights in {-1, 0, +1} the product is a sum of the inputs
// with +1 weights minus the sum with -1 weights; zero weights drop out. Here
// the sign selection is done by the int8 matrix cores: the packed codes are
// expanded in registers to {-1, 0, +1} bytes (a zero weight contributes a zero
// product) and fed to v_mfma_i32_16x16x64_i8 against the int8 activations, so
// the int32 sums are exact.
//
// Layout of the work. A wave owns 16 weight rows (the MFMA A operand: lane
// l -> row l % 16, k-group l / 16) and a share of K. Each lane loads 16 bytes
// of its row per step (4 packed words = 64 weights); the 4 lanes of a row
// cover 64 contiguous bytes, so a wave load covers 16 rows x 64 B. Word s of a
// lane's 16 bytes feeds MFMA s; the B operand (lane l -> token l % 16) reads
// the 16 activation bytes of the same k positions from LDS, where the whole
// [M][K] int8 activation block is staged once per workgroup. Tokens >= M read
// zero. Waves that split K for the same rows reduce in LDS; the epilogue
// rescales by x_scale[m] * gamma.
//
// Roofline: HBM. Algorithmic bytes per call = N*K/4 (packed weights) + M*K
// (activations) + 4*M (scales) + 4 (gamma) + 4*M*N (y).
#include "common.hpp"
#include "launch.hpp"

namespace bl {

constexpr int kGemvThreads = 256;
constexpr int kGemvMaxM = 16;
constexpr int64_t kGemvMaxXBytes = 128 * 1024;
constexpr int kXPad = 16;  // LDS row padding (bytes) against bank conflicts

template <int RG>
__global__ __launch_bounds__(kGemvThreads) void k_gemv(
    const int8_t* __restrict__ xq, const float* __restrict__ xs, int M, int K,
    const uint32_t* __restrict__ Wp, const float* __restrict__ gamma_p, int N,
    float* __restrict__ y, int32_t* __restrict__ acc_out) {
    constexpr int KS = 4 / RG;  // waves splitting K within a row group
    extern __shared__ __align__(16) uint8_t smem[];
    __shared__ v4i red[4][kWave];

    const int tid = threadIdx.x;
    const int xstride = K + kXPad;

    // Stage the activations: M rows of K bytes, 16 B per thread per step.
    {
        const int cpr = K / 16;  // 16-byte chunks per row
        const int nchunks = M * cpr;
        const uint4* src = reinterpret_cast<const uint4*>(xq);
        for (int c = tid; c < nchunks; c += kGemvThreads) {
            const int mm = c / cpr, cc = c - mm * cpr;
            *reinterpret_cast<uint4*>(smem + mm * xstride + 16 * cc) = src[c];
        }
    }

    const int wave = tid / kWave, lane = tid % kWave;
    const int rg = wave % RG, ks = wave / RG;
    const int r = lane % 16, g = lane / 16;
    const int row0 = blockIdx.x * (16 * RG) + rg * 16;
    const int row = min(row0 + r, N - 1);
    const int KW = K / 16;  // packed words per row
    const uint32_t* wrow = Wp + (size_t)row * KW + 4 * g;
    const int tok = lane % 16;
    const bool tok_ok = tok < M;
    const int8_t* xrow = reinterpret_cast<const int8_t*>(smem) + (tok_ok ? tok : 0) * xstride + 64 * g;

    __syncthreads();

    v4i acc = {0, 0, 0, 0};
    const v4i zero = {0, 0, 0, 0};
    const int nfull = KW / 16;  // full 256-weight chunks per row

    auto process = [&](const uint4 wv, int c) {
        const uint32_t w4[4] = {wv.x, wv.y, wv.z, wv.w};
        const int8_t* xb = xrow + 256 * c;
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            const v4i a = expand_word(w4[s]);
            const v4i b = tok_ok ? *reinterpret_cast<const v4i*>(xb + 16 * s) : zero;
            acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, acc, 0, 0, 0);
        }
    };

    constexpr int U = 4;
    int c = ks;
    if (c + (U - 1) * KS < nfull) {
        uint4 cur[U];
#pragma unroll
        for (int u = 0; u < U; ++u)
            cur[u] = *reinterpret_cast<const uint4*>(wrow + 16 * (c + u * KS));
        for (;;) {
            const int cn = c + U * KS;
            const bool more = cn + (U - 1) * KS < nfull;
            uint4 nxt[U];
            if (more) {
#pragma unroll
                for (int u = 0; u < U; ++u)
                    nxt[u] = *reinterpret_cast<const uint4*>(wrow + 16 * (cn + u * KS));
            }
#pragma unroll
            for (int u = 0; u < U; ++u) process(cur[u], c + u * KS);
            c = cn;
            if (!more) break;
#pragma unroll
            for (int u = 0; u < U; ++u) cur[u] = nxt[u];
        }
    }
    for (; c < nfull; c += KS) process(*reinterpret_cast<const uint4*>(wrow + 16 * c), c);

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
            const v4i a = gv ? expand_word(w4[s]) : zero;
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

    // C layout of the 16x16 MFMA: lane l holds rows 4*(l/16)+i (weights),
    // column l%16 (token).
    if (tok_ok) {
        const float sc = xs[tok] * (*gamma_p);
        const int nb = row0 + 4 * (lane / 16);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int n = nb + i;
            if (n < N) {
                y[(size_t)tok * N + n] = (float)acc[i] * sc;
                if (acc_out) acc_out[(size_t)tok * N + n] = acc[i];
            }
        }
    }
}

bool gemv_supported(int64_t M, int64_t K) {
    return M >= 1 && M <= kGemvMaxM && M * K <= kGemvMaxXBytes;
}

template <int RG>
static hipError_t launch_gemv_rg(const int8_t* xq, const float* xs, int M, int K,
                                 const uint32_t* Wp, const float* gamma, int N, float* y,
                                 int32_t* acc, hipStream_t stream) {
    const size_t lds = (size_t)M * (K + kXPad);
    static bool attr_set = false;
    if (lds > 64 * 1024 && !attr_set) {
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_gemv<RG>),
                                           hipFuncAttributeMaxDynamicSharedMemorySize,
                                           (int)(kGemvMaxXBytes + kGemvMaxM * kXPad));
        if (e != hipSuccess) return e;
        attr_set = true;
    }
    const int blocks = (N + 16 * RG - 1) / (16 * RG);
    hipLaunchKernelGGL(k_gemv<RG>, dim3(blocks), dim3(kGemvThreads), lds, stream, xq, xs, M, K,
                       Wp, gamma, N, y, acc);
    return hipGetLastError();
}

hipError_t launch_gemv(const int8_t* xq, const float* xs, int M, int K, const uint32_t* Wp,
                       const float* gamma, int N, float* y, int32_t* acc, hipStream_t stream) {
    if (!gemv_supported(M, K)) return hipErrorInvalidValue;
    return launch_gemv_rg<1>(xq, xs, M, K, Wp, gamma, N, y, acc, stream);
}

}  // namespace bl
