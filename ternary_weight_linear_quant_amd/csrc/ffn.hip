// Decode step of a 2B4T-style FFN in two launches.
//
// Source: inferownia.pl, "BitNet b1.58: era 1-bitowych LLM-ów", sections
// "Mnożenie? Jakie mnożenie" (ternary product as adds and subtracts) and
// "Zrób to sam — Microsoft wypuścił konkretny model" (2B4T: squared ReLU);
// comrad404.com, "BitNet b1.58: что показала работа Microsoft об «эре
// 1-битных LLM»", section «Метод: как устроен BitNet b1.58» (8-bit
// activations, quantised before each low-bit product).
//
// Launch A: every workgroup quantises the layer input x (bf16 [M][K]) per
//   token into LDS itself, then computes 16 rows of BOTH the gate and the up
//   projection (KS waves each, splitting K) and writes
//   h = bf16(relu(y_gate)^2 * y_up) for those rows.
// Launch B: every workgroup quantises h per token into LDS itself and
//   computes 16 rows of the down projection (KS waves splitting K) into y.
// The K split is chosen so that every wave's weight chunks are in flight at
// once (a few chunks per wave).
// Each step uses exactly the arithmetic of bl_quantize_acts, bl_bitlinear
// and bl_relu2_glu, so the output bits equal the unfused sequence. The
// per-workgroup quantisation re-reads the M tokens from L2 in every
// workgroup: cheap for a few tokens, and still ahead of the four-launch
// sequence at 8 (the bf16 inputs are cached in registers, up to 16 units of
// 16 values per thread). At 16 tokens launch B's reads of h (221 KB per
// workgroup on the 2B4T shapes) cost more than one act quant launch and the
// plain GEMV on the codes, so the step runs launch A alone, then those two.
//
// Ordering inside a workgroup: the activation loads are issued first, the
// R weight-chunk loads right after (always R, clamped to the wave's range),
// so waiting for the activations leaves the weight stream in flight; LDS
// barriers wait on LDS traffic only.
//
// Roofline: HBM / launch latency. Algorithmic bytes per layer = packed
// weights of the three matrices + 2*M*K (x) + 2*M*N_ff (h, written and read)
// + 4*M*K (y).
#include "common.hpp"
#include "launch.hpp"

namespace bl {

typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

constexpr int kFfnMaxThreads = 1024;
constexpr int kFfnMinThreads = 256;
constexpr int kFfnMaxCache = 16;  // 16-value activation units cached per thread, at most
constexpr int kFfnSublnCache = 4;  // with the norm's gain cached beside them
constexpr int kFfnR = 4;      // weight chunks in flight per lane

// lgkmcnt(0) only: LDS traffic done, vector loads may stay in flight.
#define BL_WAIT_LGKM0() __builtin_amdgcn_s_waitcnt(15 | (7 << 4) | (0 << 8) | (3 << 14))

__device__ __forceinline__ void lds_barrier() {
    BL_WAIT_LGKM0();
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// SUBLN (quantising launch B only): the sub-layer RMSNorm with gain `gain`
// before the quantisation, as bl_quantize_acts(h, gain) computes it: codes
// of z = h*g, scale a / (127 * rms(h)), sum h^2 in fp64.
// KIND: the gating of launch A (relu^2 or SiLU).
// RG: groups of 16 rows per workgroup (all share the staged activations).
// CU: activation units (16 values of one token) cached per thread; the M
// tokens' K values must fit NT * CU units.
template <bool GLU, int KS, bool SUBLN, int KIND, int RG, int CU>
__global__ __launch_bounds__(64 * (GLU ? 2 : 1) * RG * KS) void k_ffn_gemv(
    const uint16_t* __restrict__ xin, int M, int K, const uint32_t* __restrict__ W0,
    const float* __restrict__ g0, const uint32_t* __restrict__ W1,
    const float* __restrict__ g1, int N, float* __restrict__ y, uint16_t* __restrict__ h,
    const uint16_t* __restrict__ gain, float rms_eps) {
    static_assert(!(GLU && SUBLN), "the norm precedes the down projection only");
    constexpr int NW = (GLU ? 2 : 1) * RG * KS;  // waves: (matrix, row group, K split)
    constexpr int NT = 64 * NW;             // threads
    constexpr int CACHE = CU;
    static_assert(NT >= kFfnMinThreads && NT <= kFfnMaxThreads && CACHE >= 1 &&
                      CACHE <= kFfnMaxCache,
                  "block shape");
    static_assert(!SUBLN || CU <= kFfnSublnCache, "register budget of the norm's gain cache");
    extern __shared__ __align__(16) uint8_t smem[];  // int8 activations, token-minor
    __shared__ v4i red[NW][kWave];
    __shared__ float s_amax[NW][16];
    __shared__ double s_ss[SUBLN ? NW : 1][16];
    __shared__ float s_scale[16];

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int lane = tid % kWave;
    const int mat = GLU ? wave / (KS * RG) : 0;
    const int rg = (wave / KS) % RG;
    const int ks = wave % KS;
    const uint32_t* W = (GLU && mat) ? W1 : W0;
    const int r = lane % 16, g = lane / 16;
    const int row0 = ((int)blockIdx.x * RG + rg) * 16;
    const int row = min(row0 + r, N - 1);
    const int KW = K / 16;
    const int nfull = KW / 16;  // >= KS (checked on the host)
    const uint32_t* wrow = W + (size_t)row * KW + 4 * g;
    const int nw = (nfull - ks + KS - 1) / KS;

    // 1. Activation loads: unit u = 16 consecutive values of one token; the
    //    units of thread t all belong to token t % M (M divides 256).
    const int U = M * (K / 16);
    const int mt = tid % M;
    uint4 xa[CACHE], xb[CACHE];
    uint4 ga[SUBLN ? CACHE : 1], gb[SUBLN ? CACHE : 1];
#pragma unroll
    for (int i = 0; i < CACHE; ++i) {
        const int u = tid + NT * i;
        if (u < U) {
            const uint4* src = reinterpret_cast<const uint4*>(xin + (size_t)mt * K + 16 * (u / M));
            xa[i] = src[0];
            xb[i] = src[1];
            if constexpr (SUBLN) {
                const uint4* gsrc = reinterpret_cast<const uint4*>(gain + 16 * (u / M));
                ga[i] = gsrc[0];
                gb[i] = gsrc[1];
            }
        }
    }
    asm volatile("" ::: "memory");  // keep the activation loads first
    // 2. The first R weight chunks (clamped to this wave's range, so the
    //    count is fixed and the waits below are exact).
    uint4 wb[kFfnR];
#pragma unroll
    for (int i = 0; i < kFfnR; ++i)
        wb[i] = load_stream16(wrow + 16 * (ks + KS * min(i, nw - 1)));

    // 3. Per-token absmax (exact, order-free) of the cached units (of h*g
    //    under SUBLN, with sum h^2 beside it).
    auto gain_of = [&](int i, int e) -> float {  // gain of value e (0..15) of unit i
        const int c = SUBLN ? i : 0;
        const uint32_t g8[8] = {ga[c].x, ga[c].y, ga[c].z, ga[c].w,
                                gb[c].x, gb[c].y, gb[c].z, gb[c].w};
        return bf16_to_f32((g8[e / 2] >> (16 * (e % 2))) & 0xFFFFu);
    };
    float amax = 0.0f;
    double ss = 0.0;
    // Without the norm, max |x| over finite bf16 values is the integer max
    // of their sign-cleared bit patterns, two per packed 16-bit max.
    u16x2 mbits = {0, 0};
#pragma unroll
    for (int i = 0; i < CACHE; ++i) {
        if (tid + NT * i < U) {
            const uint32_t w8[8] = {xa[i].x, xa[i].y, xa[i].z, xa[i].w,
                                    xb[i].x, xb[i].y, xb[i].z, xb[i].w};
            if constexpr (SUBLN) {
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    const float xf = bf16_to_f32((w8[e / 2] >> (16 * (e % 2))) & 0xFFFFu);
                    amax = fmaxf(amax, fabsf(xf * gain_of(i, e)));
                    ss += (double)xf * (double)xf;
                }
            } else {
#pragma unroll
                for (int d = 0; d < 8; ++d)
                    mbits = __builtin_elementwise_max(
                        mbits, __builtin_bit_cast(u16x2, w8[d] & 0x7FFF7FFFu));
            }
        }
    }
    if constexpr (!SUBLN)
        amax = bf16_to_f32(mbits[0] > mbits[1] ? mbits[0] : mbits[1]);
    // Lanes with equal lane % M hold the same token. One token: the max on DPP
    // (magnitudes, so the unsigned order of the bits; exact in any order),
    // the fp64 sum in the butterfly's order as for several tokens.
    if (M == 1) {
        amax = __uint_as_float(wave_max_u32(__float_as_uint(amax)));
        if constexpr (SUBLN) {
#pragma unroll
            for (int o = 32; o > 0; o >>= 1) ss += __shfl_xor(ss, o, kWave);
        }
    } else {
#pragma unroll
        for (int o = 32; o > 0; o >>= 1)
            if (o >= M) {
                amax = fmaxf(amax, __shfl_xor(amax, o, kWave));
                if constexpr (SUBLN) ss += __shfl_xor(ss, o, kWave);
            }
    }
    if (lane < M) {
        s_amax[wave][lane] = amax;
        if constexpr (SUBLN) s_ss[wave][lane] = ss;
    }
    lds_barrier();
    float a = s_amax[0][mt];
#pragma unroll
    for (int w = 1; w < NW; ++w) a = fmaxf(a, s_amax[w][mt]);
    a = a > 1e-5f ? a : 1e-5f;
    const float inv = 127.0f / a;
    if (tid < M) {
        if constexpr (SUBLN) {
            double st = s_ss[0][tid];
#pragma unroll
            for (int w = 1; w < NW; ++w) st += s_ss[w][tid];
            const double rms = sqrt(st / (double)K + (double)rms_eps);
            s_scale[tid] = (float)((double)a / (127.0 * rms));
        } else {
            s_scale[tid] = a / 127.0f;
        }
    }

    // 4. Codes into LDS slot u (chunk u / M of token u % M).
#pragma unroll
    for (int i = 0; i < CACHE; ++i) {
        const int u = tid + NT * i;
        if (u < U) {
            const uint32_t w8[8] = {xa[i].x, xa[i].y, xa[i].z, xa[i].w,
                                    xb[i].x, xb[i].y, xb[i].z, xb[i].w};
            float t[16];
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                float z = bf16_to_f32((w8[e / 2] >> (16 * (e % 2))) & 0xFFFFu);
                if constexpr (SUBLN) z = z * gain_of(i, e);
                t[e] = z * inv;
            }
            uint32_t q[4];
#pragma unroll
            for (int d = 0; d < 4; ++d)
                q[d] = pack_codes4(t[4 * d], t[4 * d + 1], t[4 * d + 2], t[4 * d + 3]);
            *reinterpret_cast<uint4*>(smem + 16 * u) = make_uint4(q[0], q[1], q[2], q[3]);
        }
    }
    lds_barrier();

    // 5. Ternary x int8 product on the matrix cores (negated weights).
    const int tok = lane % 16;
    const bool tok_ok = tok < M;
    const int8_t* xl = reinterpret_cast<const int8_t*>(smem) + 16 * (tok_ok ? tok : 0);
    v4i acc = {0, 0, 0, 0};
    const v4i zero = {0, 0, 0, 0};
    auto process = [&](const uint4 wv, int c) {
        const uint32_t w4[4] = {wv.x, wv.y, wv.z, wv.w};
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            const v4i av = expand_word_neg(w4[s]);
            const int j = 16 * c + 4 * g + s;
            const v4i bv = tok_ok ? *reinterpret_cast<const v4i*>(xl + 16 * j * M) : zero;
            acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(av, bv, acc, 0, 0, 0);
        }
    };
    for (int b0 = 0; b0 < nw; b0 += kFfnR) {
#pragma unroll
        for (int i = 0; i < kFfnR; ++i) {
            const int ci = b0 + i;
            if (ci < nw) {
                process(wb[i], ks + KS * ci);
                if (ci + kFfnR < nw)
                    wb[i] = load_stream16(wrow + 16 * (ks + KS * (ci + kFfnR)));
            }
        }
    }
    // Tail chunk (KW % 16 words, a multiple of 4): the last K-split wave.
    const int rem = KW - 16 * nfull;
    if (rem != 0 && ks == KS - 1) {
        const bool gv = 4 * g < rem;
        const uint4 wv = gv ? load_stream16(wrow + 16 * nfull)
                            : make_uint4(0, 0, 0, 0);
        const uint32_t w4[4] = {wv.x, wv.y, wv.z, wv.w};
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            const v4i av = gv ? expand_word_neg(w4[s]) : zero;
            const int j = 16 * nfull + 4 * g + s;
            const v4i bv = (gv && tok_ok) ? *reinterpret_cast<const v4i*>(xl + 16 * j * M) : zero;
            acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(av, bv, acc, 0, 0, 0);
        }
    }

    // 6. Reduce the K split and write the epilogue (wave 0).
    red[wave][lane] = acc;
    __syncthreads();
    if (ks != 0 || mat != 0 || !tok_ok) return;  // one wave per row group
    const float xs = s_scale[tok];
    const int nbase = row0 + 4 * (lane / 16);
    if constexpr (GLU) {
        v4i ga = red[rg * KS][lane], ua = red[(RG + rg) * KS][lane];
#pragma unroll
        for (int w = 1; w < KS; ++w) {
            ga += red[rg * KS + w][lane];
            ua += red[(RG + rg) * KS + w][lane];
        }
        ga = -ga;
        ua = -ua;
        const float sg = xs * (*g0), su = xs * (*g1);
        // N is a multiple of 64 (checked on the host), so the lane's four
        // outputs are all in range or all out, and 8-byte aligned.
        if (nbase < N) {
            uint32_t hb[4];
#pragma unroll
            for (int i = 0; i < 4; ++i)
                hb[i] = glu_bits<KIND>((float)ga[i] * sg, (float)ua[i] * su);
            *reinterpret_cast<uint2*>(h + (size_t)tok * N + nbase) =
                make_uint2(hb[0] | (hb[1] << 16), hb[2] | (hb[3] << 16));
        }
    } else {
        v4i ta = red[rg * KS][lane];
#pragma unroll
        for (int w = 1; w < KS; ++w) ta += red[rg * KS + w][lane];
        ta = -ta;
        const float sc = xs * (*g0);
        if (nbase < N)  // four in range, 16-byte aligned (as above)
            *reinterpret_cast<float4*>(y + (size_t)tok * N + nbase) =
                make_float4((float)ta[0] * sc, (float)ta[1] * sc, (float)ta[2] * sc,
                            (float)ta[3] * sc);
    }
}

// Launch shapes (measured on the 2B4T FFN): A (gate + up) with 2 waves per
// matrix splitting K; B (down, few output rows, long K) with 8 waves so that
// every wave's chunks are in flight at once, or 4 for hidden sizes under
// 2048.
constexpr int kKsA = 2, kKsB = 8, kKsBSmall = 4;

// Row groups per workgroup (launch A / launch B) by token count. Above one
// token, launch A shares its staged activations between two groups (2B4T
// layer at 4 tokens 13.3 -> 12.1 us); launch B keeps one, since its 2560
// output rows would give only 80 workgroups (14.8 us with two).
constexpr int kRgA1 = 1, kRgAn = 2, kRgB1 = 1;

namespace {

// Threads of launch A (gate + up) and launch B (down) at M tokens.
int threads_a(int M) { return 64 * 2 * kKsA * (M == 1 ? kRgA1 : kRgAn); }
int threads_b(int N_ff) { return 64 * (N_ff / 256 >= kKsB ? kKsB : kKsBSmall) * kRgB1; }

// Smallest instantiated cache (4, 8 or 16 units per thread) holding `units`
// over `threads`; 0 if none does.
int cache_for(int64_t units, int threads) {
    for (int cu : {4, 8, 16})
        if (units <= (int64_t)cu * threads) return cu;
    return 0;
}

}  // namespace

bool ffn_fused_supported(int64_t M, int64_t K, int64_t N_ff, bool subln) {
    // Token counts dividing a wave (lanes with equal lane % M hold one token).
    if (M != 1 && M != 2 && M != 4 && M != 8 && M != 16) return false;
    if (K % 64 != 0 || N_ff % 64 != 0) return false;  // whole 4-output stores
    if (K > (1 << 20) || N_ff > (1 << 20)) return false;
    // Every K-split wave needs at least one full 256-weight chunk.
    if (K / 256 < kKsA || N_ff / 256 < kKsBSmall) return false;
    const int ca = cache_for(M * (K / 16), threads_a((int)M));
    const int cb = cache_for(M * (N_ff / 16), threads_b((int)N_ff));
    if (ca == 0 || cb == 0) return false;
    if (subln && cb > kFfnSublnCache) return false;
    // The int8 activations of either launch must fit LDS beside the statics.
    return M * K <= 128 * 1024 && M * N_ff <= 128 * 1024;
}

namespace {

// Every supported launch stages at most 128 KiB of int8 activations
// (ffn_fused_supported, ffn_gate_up_supported); the kernels' static LDS,
// under 10 KiB, fits beside it.
constexpr size_t kFfnMaxDynLds = 128 * 1024;

// `done` is a flag set of the launcher's own kernel instance.
template <typename Kern>
hipError_t allow_lds(Kern kern, size_t lds, std::atomic<uint64_t>& done) {
    if (lds <= 64 * 1024) return hipSuccess;
    if (lds > kFfnMaxDynLds) return hipErrorInvalidValue;
    return allow_dynamic_lds(reinterpret_cast<const void*>(kern), kFfnMaxDynLds, done);
}

template <int KS, bool SUBLN, int RG, int CU>
hipError_t launch_ffn_down(const uint16_t* h, int M, int N_ff, const uint32_t* Wd,
                           const float* gd, int K, float* y, const uint16_t* gain,
                           float rms_eps, hipStream_t stream) {
    auto kern = &k_ffn_gemv<false, KS, SUBLN, kGluRelu2, RG, CU>;
    const size_t lds = (size_t)M * N_ff;
    static std::atomic<uint64_t> lds_set{0};
    hipError_t e = allow_lds(kern, lds, lds_set);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kern, dim3((K + 16 * RG - 1) / (16 * RG)), dim3(64 * KS * RG), lds,
                       stream, h, M, N_ff, Wd, gd, (const uint32_t*)nullptr,
                       (const float*)nullptr, K, y, (uint16_t*)nullptr, gain, rms_eps);
    return hipGetLastError();
}

template <int KS, bool SUBLN>
hipError_t launch_ffn_down_cu(const uint16_t* h, int M, int N_ff, const uint32_t* Wd,
                              const float* gd, int K, float* y, const uint16_t* gain,
                              float rms_eps, hipStream_t stream) {
    const int cu = cache_for((int64_t)M * (N_ff / 16), 64 * KS * kRgB1);
    if constexpr (!SUBLN) {
        if (cu == 16)
            return launch_ffn_down<KS, false, kRgB1, 16>(h, M, N_ff, Wd, gd, K, y, gain, rms_eps,
                                                         stream);
        if (cu == 8)
            return launch_ffn_down<KS, false, kRgB1, 8>(h, M, N_ff, Wd, gd, K, y, gain, rms_eps,
                                                        stream);
    }
    return launch_ffn_down<KS, SUBLN, kRgB1, 4>(h, M, N_ff, Wd, gd, K, y, gain, rms_eps, stream);
}

template <int KIND, int RG, int CU>
hipError_t launch_ffn_up(const uint16_t* x, int M, int K, const uint32_t* Wg, const float* gg,
                         const uint32_t* Wu, const float* gu, int N_ff, uint16_t* h,
                         hipStream_t stream) {
    auto kern = &k_ffn_gemv<true, kKsA, false, KIND, RG, CU>;
    const size_t lds = (size_t)M * K;
    static std::atomic<uint64_t> lds_set{0};
    hipError_t e = allow_lds(kern, lds, lds_set);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kern, dim3((N_ff + 16 * RG - 1) / (16 * RG)), dim3(64 * 2 * kKsA * RG),
                       lds, stream, x, M, K, Wg, gg, Wu, gu, N_ff, (float*)nullptr, h,
                       (const uint16_t*)nullptr, 0.0f);
    return hipGetLastError();
}

template <int KIND, int RG>
hipError_t launch_ffn_up_cu(const uint16_t* x, int M, int K, const uint32_t* Wg,
                            const float* gg, const uint32_t* Wu, const float* gu, int N_ff,
                            uint16_t* h, hipStream_t stream) {
    const int cu = cache_for((int64_t)M * (K / 16), 64 * 2 * kKsA * RG);
    if (cu == 16) return launch_ffn_up<KIND, RG, 16>(x, M, K, Wg, gg, Wu, gu, N_ff, h, stream);
    if (cu == 8) return launch_ffn_up<KIND, RG, 8>(x, M, K, Wg, gg, Wu, gu, N_ff, h, stream);
    return launch_ffn_up<KIND, RG, 4>(x, M, K, Wg, gg, Wu, gu, N_ff, h, stream);
}

template <int KIND>
hipError_t launch_ffn_up_rg(const uint16_t* x, int M, int K, const uint32_t* Wg,
                            const float* gg, const uint32_t* Wu, const float* gu, int N_ff,
                            uint16_t* h, hipStream_t stream) {
    if ((M == 1 ? kRgA1 : kRgAn) == 2)
        return launch_ffn_up_cu<KIND, 2>(x, M, K, Wg, gg, Wu, gu, N_ff, h, stream);
    return launch_ffn_up_cu<KIND, 1>(x, M, K, Wg, gg, Wu, gu, N_ff, h, stream);
}

}  // namespace

hipError_t launch_ffn_fused(const uint16_t* x, int M, int K, const uint32_t* Wg,
                            const float* gg, const uint32_t* Wu, const float* gu, int N_ff,
                            const uint32_t* Wd, const float* gd, uint16_t* h, float* y,
                            int kind, const uint16_t* subln_gain, float subln_eps,
                            hipStream_t stream) {
    hipError_t e =
        kind == kGluSwiglu
            ? launch_ffn_up_rg<kGluSwiglu>(x, M, K, Wg, gg, Wu, gu, N_ff, h, stream)
            : launch_ffn_up_rg<kGluRelu2>(x, M, K, Wg, gg, Wu, gu, N_ff, h, stream);
    if (e != hipSuccess) return e;
    const bool big = N_ff / 256 >= kKsB;
    if (subln_gain)
        return big ? launch_ffn_down_cu<kKsB, true>(h, M, N_ff, Wd, gd, K, y, subln_gain,
                                                    subln_eps, stream)
                   : launch_ffn_down_cu<kKsBSmall, true>(h, M, N_ff, Wd, gd, K, y, subln_gain,
                                                         subln_eps, stream);
    return big ? launch_ffn_down_cu<kKsB, false>(h, M, N_ff, Wd, gd, K, y, nullptr, 0.0f, stream)
               : launch_ffn_down_cu<kKsBSmall, false>(h, M, N_ff, Wd, gd, K, y, nullptr, 0.0f,
                                                      stream);
}

// Launch A alone (act quant + gate/up + gating into h), for a step whose
// down projection runs as a separate act quant and GEMV.
bool ffn_gate_up_supported(int64_t M, int64_t K, int64_t N_ff) {
    if (M != 1 && M != 2 && M != 4 && M != 8 && M != 16) return false;
    if (K % 64 != 0 || N_ff % 64 != 0) return false;
    if (K > (1 << 20) || N_ff > (1 << 20)) return false;
    if (K / 256 < kKsA) return false;
    return cache_for(M * (K / 16), threads_a((int)M)) != 0 && M * K <= 128 * 1024;
}

hipError_t launch_ffn_gate_up(const uint16_t* x, int M, int K, const uint32_t* Wg,
                              const float* gg, const uint32_t* Wu, const float* gu, int N_ff,
                              uint16_t* h, int kind, hipStream_t stream) {
    return kind == kGluSwiglu
               ? launch_ffn_up_rg<kGluSwiglu>(x, M, K, Wg, gg, Wu, gu, N_ff, h, stream)
               : launch_ffn_up_rg<kGluRelu2>(x, M, K, Wg, gg, Wu, gu, N_ff, h, stream);
}

}  // namespace bl
